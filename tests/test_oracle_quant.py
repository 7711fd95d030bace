"""Pins of the oracle's block quantisers: golden hand-derived cases, exact
scaling invariances, the lossless special case that fixes the MX exponent
offset, brute-force nearest scale values, and error bounds."""
import os

import numpy as np
import pytest

from oracle import codecs, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_cases.txt")


def _golden(kind):
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            parts = [p.strip() for p in line.strip().split("|")]
            if len(parts) >= 3 and parts[0] == kind:
                rows.append(parts[1:3])
    assert rows
    return rows


# ------------------------------------------------------------------ MXFP8


def test_mx_golden():
    for first, want in _golden("mx"):
        blk = np.zeros(32, np.float32)
        blk[0] = float(first)
        c, s = quant.mxfp8_quantize(blk[None])
        b, code = want.split()
        assert int(s[0, 0]) == int(b), first
        assert int(c[0, 0]) == int(code, 16), first


def test_mx_floor_rule_480():
    # distinguishes the floor rule (byte 127, saturating 480 -> 448) from the
    # ceil(log2(amax/448)) alternative (byte 128, 480/2 = 240 exact)
    blk = np.full(32, 1.0, np.float32)
    blk[5] = 480.0
    c, s = quant.mxfp8_quantize(blk[None])
    assert s[0, 0] == 127 and c[0, 5] == 0x7E


@pytest.mark.parametrize("a", [-20, -3, 0, 4, 17])
def test_mx_lossless_special_case(a):
    """A block whose amax is 2^a and whose elements are e4m3 values times
    2^(a-8) is reproduced exactly; s = a-9 would saturate 2^a, s = a-7 would
    drop the low mantissa bits of the smallest elements."""
    rng = np.random.default_rng(a + 100)
    mags = codecs.E4M3_MAG[1:121]  # up to 2^8 = 256 (code 0x78)
    vals = rng.choice(mags, (64, 32)) * rng.choice([-1.0, 1.0], (64, 32))
    vals[:, 3] = 256.0  # amax = 2^8 before scaling
    x = (vals * 2.0 ** (a - 8)).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), vals * 2.0 ** (a - 8))
    c, s = quant.mxfp8_quantize(x)
    assert np.all(s == a - 8 + 127)
    assert np.array_equal(quant.mxfp8_dequantize(c, s), x.astype(np.float64))


def test_mx_power_of_two_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    c0, s0 = quant.mxfp8_quantize(x)
    for n in (-30, -5, 1, 7, 40):
        c, s = quant.mxfp8_quantize((x * np.float32(2.0**n)).astype(np.float32))
        assert np.array_equal(c, c0)
        assert np.array_equal(s.astype(int), s0.astype(int) + n)


def test_mx_error_bound():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((200, 256)) * np.exp(rng.uniform(-8, 8, (200, 1)))).astype(np.float32)
    c, s = quant.mxfp8_quantize(x)
    xh = quant.mxfp8_dequantize(c, s)
    sc = np.repeat(codecs.e8m0_decode(s), 32, axis=-1)
    scaled = np.abs(x.astype(np.float64)) / sc
    sat = scaled >= 448
    normal = (scaled >= 2.0**-6) & ~sat
    err = np.abs(xh - x)
    # half an e4m3 ulp (3 mantissa bits) in the normal range
    assert np.all(err[normal] <= 2.0**-4 * np.abs(x[normal]) * (1 + 1e-12))
    # half the subnormal quantum 2^-9 below it
    assert np.all(err[~normal & ~sat] <= 2.0**-10 * sc[~normal & ~sat])
    # saturation to 448 only happens to values within [448, 512) scaled units
    assert np.all(np.abs(xh[sat]) == 448 * sc[sat])
    assert np.all(scaled < 512)


def test_mx_shapes_and_errors():
    with pytest.raises(ValueError):
        quant.mxfp8_quantize(np.zeros((2, 33), np.float32))
    c, s = quant.mxfp8_quantize(np.zeros((3, 4, 64), np.float32))
    assert c.shape == (3, 4, 64) and s.shape == (3, 4, 2)


# ------------------------------------------------------------------ NVFP4


def test_nv_golden():
    for first, want in _golden("nv"):
        blk = np.zeros(16, np.float32)
        blk[0] = float(first)
        p, s = quant.nvfp4_quantize(blk[None])
        sc, code = want.split()
        assert int(s[0, 0]) == int(sc, 16), first
        assert int(codecs.unpack_e2m1(p)[0, 0]) == int(code, 16), first


@pytest.mark.parametrize("n", range(-6, 9))
def test_nv_amax_six_times_pow2(n):
    # amax = 6 * 2^n gives the exact scale 2^n while 2^n is a normal e4m3
    rng = np.random.default_rng(n + 50)
    x = (rng.uniform(-6, 6, (8, 16)) * 2.0**n).astype(np.float32)
    x[:, 0] = 6 * 2.0**n
    _, s = quant.nvfp4_quantize(x)
    assert np.all(codecs.e4m3_decode(s) == 2.0**n)


def test_nv_scale_is_nearest_e4m3_of_amax_over_6():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((500, 16)) * np.exp(rng.uniform(-6, 6, (500, 1)))).astype(np.float32)
    _, s = quant.nvfp4_quantize(x)
    target = (np.max(np.abs(x), axis=1) / np.float32(6)).astype(np.float64)
    mags = codecs.E4M3_MAG
    d = np.abs(target[:, None] - mags[None, :])
    best = mags[np.argmin(d, axis=1)]
    got = codecs.e4m3_decode(s[:, 0])
    # nearest (ties impossible here: target is not a short dyadic number)
    assert np.array_equal(got, best)


def test_nv_fp32_scale_decision_equals_exact_for_all_bf16_amax():
    """The scale uses fp32(amax / 6); for bf16 amax values this never differs
    from rounding the exact quotient (the quotient is never within an fp32
    half-ulp of an e4m3 midpoint)."""
    b = np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16)
    a = codecs.bf16_decode(b)
    via32 = codecs.e4m3_encode((a.astype(np.float32) / np.float32(6)).astype(np.float64))
    exact = codecs.e4m3_encode(a / 6.0)
    assert np.array_equal(via32, exact)


def test_nv_codes_are_nearest_multiples_of_scale():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((300, 64)) * 3).astype(np.float32)
    p, s = quant.nvfp4_quantize(x)
    q = codecs.e2m1_decode(codecs.unpack_e2m1(p))
    sc = np.repeat(codecs.e4m3_decode(s), 16, axis=-1)
    cand = codecs.E2M1_MAG[None, None, :] * sc[..., None]
    d = np.abs(np.abs(x.astype(np.float64))[..., None] - cand)
    # the chosen magnitude is at minimum distance (ties are measure-zero here)
    chosen = np.abs(q) * sc
    assert np.allclose(np.abs(np.abs(x) - chosen), d.min(axis=-1), rtol=0, atol=0)


def test_nv_zero_block():
    x = np.zeros((2, 32), np.float32)
    x[1, :16] = -0.0
    p, s = quant.nvfp4_quantize(x)
    assert np.all(s == 0)
    assert np.array_equal(quant.nvfp4_dequantize(p, s), np.zeros((2, 32)))


# ------------------------------------------------------------------ weights


def test_nvfp4_weight_global_scale_convention():
    """The block holding the tensor's amax gets scale 448 (code 0x7E) and the
    amax element code 6, so it dequantises to the amax: pins alpha = amax/2688
    and that alpha is applied on dequantisation."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    p, s, alpha = quant.nvfp4_quantize_weight(w)
    amax = np.max(np.abs(w))
    assert alpha == np.float32(amax / np.float32(2688.0))
    r, c = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert s[r, c // 16] == 0x7E
    assert codecs.unpack_e2m1(p)[r, c] & 7 == 7
    wh = quant.nvfp4_dequantize(p, s, alpha)
    assert abs(abs(wh[r, c]) - amax) <= 1e-6 * amax
    # 4-bit weights: relative L2 error of a normal tensor is ~10 %
    rel = np.linalg.norm(wh - w) / np.linalg.norm(w)
    assert 0.03 < rel < 0.2
    # every element is within half an e2m1 step (<= 1 scale unit at the top)
    sc = np.repeat(codecs.e4m3_decode(s), 16, axis=-1) * np.float64(alpha)
    assert np.all(np.abs(wh - w) <= 1.0 * sc + 1e-12)


def test_mxfp8_weight_error_bound():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    c, s, a = quant.quantize_weight(w, "mxfp8")
    assert a is None
    wh = quant.mxfp8_dequantize(c, s)
    sc = np.repeat(codecs.e8m0_decode(s), 32, -1)
    sat = np.abs(w) >= 448 * sc  # the floor rule saturates [448, 512) scaled units
    assert np.all(np.abs(wh[sat]) == 448 * sc[sat])
    assert np.all((np.abs(wh - w) <= 2.0**-4 * np.abs(w) + 2.0**-10 * sc)[~sat])


def test_bf16_weight_is_nearest():
    rng = np.random.default_rng(13)
    w = rng.standard_normal(10000).astype(np.float32)
    b, _, _ = quant.quantize_weight(w, "bf16")
    wh = quant.bf16_dequantize(b)
    assert np.all(np.abs(wh - w) <= 2.0**-8 * np.abs(w))  # half ulp, 8 significant bits


# ------------------------------------------------------------------ NVFP4 global-scale fold


def _nearest_e4m3_positive(v):
    """Brute force: the positive e4m3 code nearest to each v >= 0 (ties to the
    even code; values past 448 saturate to 448), by exhaustive distance."""
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E, all finite non-negative codes
    vals = codecs.e4m3_decode(codes)
    d = np.abs(np.asarray(v, np.float64)[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, codes[None, :].astype(np.int64), 1 << 20)
    even = np.where(cand % 2 == 0, cand, 1 << 20).min(axis=1)
    return np.where(even < (1 << 20), even, cand.min(axis=1)).astype(np.uint8)


def test_nvfp4_fold_alpha_one_is_identity():
    codes = np.arange(0x7F, dtype=np.uint8)
    out, a = quant.nvfp4_fold_global_scale(codes, 1.0)
    assert np.array_equal(out, codes) and a == np.float32(1.0)


@pytest.mark.parametrize("k", [1, 3, 6])
def test_nvfp4_fold_power_of_two_alpha_shifts_exponents(k):
    """alpha = 2^-k multiplies exactly: every scale whose product stays in
    e4m3's normal range (>= 2^-6) keeps its mantissa."""
    codes = np.arange(0x7F, dtype=np.uint8)
    out, _ = quant.nvfp4_fold_global_scale(codes, 2.0 ** -k)
    v = codecs.e4m3_decode(codes) * 2.0 ** -k
    normal = v >= 2.0 ** -6
    assert np.array_equal(codecs.e4m3_decode(out)[normal], v[normal])


def test_nvfp4_fold_is_nearest_e4m3_of_the_fp32_product():
    """Brute force over every scale code and alphas of the weight quantiser's
    magnitude (amax / 2688 for N(0, 0.02) weights) and beyond."""
    rng = np.random.default_rng(11)
    codes = np.arange(0x7F, dtype=np.uint8)
    for alpha in list(np.float32(rng.uniform(1e-5, 1e-4, 6))) + [np.float32(0.37), np.float32(3.1)]:
        out, _ = quant.nvfp4_fold_global_scale(codes, alpha)
        prod = (codecs.e4m3_decode(codes).astype(np.float32) * np.float32(alpha)).astype(np.float64)
        assert np.array_equal(out, _nearest_e4m3_positive(prod)), alpha


def test_nvfp4_fold_of_weights_reaches_the_subnormal_range():
    """The pages' fold on N(0, 0.02) weights: alpha ~ 4e-5 puts the folded
    scales (~1e-2) into e4m3's subnormal range, so the folded weights differ
    from the unfolded ones by more than the unfolded quantisation error."""
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    c, s, a = quant.nvfp4_quantize_weight(w)
    fs, fa = quant.nvfp4_fold_global_scale(s, a)
    assert fa == np.float32(1.0)
    assert np.mean(codecs.e4m3_decode(fs) < 2.0 ** -6) > 0.5
    ref = quant.nvfp4_dequantize(c, s, a)
    got = quant.nvfp4_dequantize(c, fs, fa)
    err_fold = np.linalg.norm(got - w) / np.linalg.norm(w)
    err_ref = np.linalg.norm(ref - w) / np.linalg.norm(w)
    assert err_fold > err_ref
