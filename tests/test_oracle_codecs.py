"""Pins of the oracle's element codecs against sources other than themselves:
torch's float8 dtypes (an independent implementation of the OCP formats),
brute-force nearest-value search, and hand-derived golden cases."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_cases.txt")


def _golden(kind):
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == kind:
                rows.append(parts[1:3])
    assert rows, kind
    return rows


def _all_finite_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_decode(bits)
    return v[np.isfinite(v)]


def _brute_nearest_code(v, mags):
    """Index of the nearest entry of mags (ascending) to |v| with ties to the
    even index, by exhaustive distance comparison; saturating at the top."""
    a = np.abs(v)[:, None]
    d = np.abs(a - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the tied candidates prefer the even index
    idx = np.where(cand.any(axis=1), 0, 0)
    n = mags.size
    even = cand & (np.arange(n)[None, :] % 2 == 0)
    first_even = np.argmax(even, axis=1)
    first = np.argmax(cand, axis=1)
    idx = np.where(even.any(axis=1), first_even, first)
    return np.where(np.abs(v) >= mags[-1], n - 1, idx)


# ---------------------------------------------------------------- decode


def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e8m0_decode_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = codecs.e8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_e2m1_decode_golden_table():
    # OCP MX v1.0 e2m1 value table, sign bit 3
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == table
    assert list(-got[8:]) == table


def test_bf16_decode_is_top_half_of_fp32():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- encode


@pytest.mark.parametrize("scale_exp", [-12, -9, -3, 0, 2, 5, 8, 9])
def test_e4m3_encode_brute_force_all_bf16(scale_exp):
    v = _all_finite_bf16_values() * 2.0**scale_exp
    v = v[np.isfinite(v)]
    got = codecs.e4m3_encode(v)
    mags = codecs.E4M3_MAG
    want = _brute_nearest_code(v, mags) | (np.signbit(v).astype(np.int64) << 7)
    assert np.array_equal(got.astype(np.int64), want)


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 50,
        rng.standard_normal(50_000).astype(np.float32) * 1e-2,
        (np.arange(0, 464 * 16) / 16.0).astype(np.float32),
    ])
    v = v[np.abs(v) < 464]  # torch's cast does not saturate above 464
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_encode(v)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("scale", [None, 2.0**-9, 0.171875, 1.0, 3.5, 448.0])
def test_e2m1_encode_brute_force_all_bf16(scale):
    v = _all_finite_bf16_values()
    s = 1.0 if scale is None else scale
    v = v[np.abs(v) < 1e30]
    got = codecs.e2m1_encode(v, None if scale is None else np.full(v.shape, s))
    want = _brute_nearest_code(v, codecs.E2M1_MAG * s) | (np.signbit(v).astype(np.int64) << 3)
    assert np.array_equal(got.astype(np.int64), want)


def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # exact ties: low 16 bits == 0x8000 with both parities of bit 16
    tie = (rng.integers(0, 2**16, 10_000).astype(np.uint32) << 16) | 0x8000
    tv = tie.view(np.float32)
    v = np.concatenate([v, tv[np.isfinite(tv)], np.float32([0.0, -0.0, 1e-45, -1e-45, 3.3895e38, 3.4e38])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_encode(v)
    assert np.array_equal(got, ref)


def test_encode_decode_round_trip():
    c = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(codecs.e4m3_encode(codecs.e4m3_decode(c)), c)
    c2 = np.arange(16, dtype=np.uint8)
    assert np.array_equal(codecs.e2m1_encode(codecs.e2m1_decode(c2)), c2)
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = np.isfinite(codecs.bf16_decode(b))
    assert np.array_equal(codecs.bf16_encode(codecs.bf16_decode(b[fin])), b[fin])


def test_encode_monotone():
    v = np.linspace(-500, 500, 200_001)
    mag = codecs.e4m3_decode(codecs.e4m3_encode(v))
    assert np.all(np.diff(mag) >= 0)
    v2 = np.linspace(-7, 7, 20_001)
    assert np.all(np.diff(codecs.e2m1_decode(codecs.e2m1_encode(v2))) >= 0)


def test_pack_unpack_e2m1():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, (5, 32)).astype(np.uint8)
    p = codecs.pack_e2m1(c)
    assert p.shape == (5, 16)
    assert np.array_equal(p[:, 0] & 0xF, c[:, 0]) and np.array_equal(p[:, 0] >> 4, c[:, 1])
    assert np.array_equal(codecs.unpack_e2m1(p), c)


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.nan]))
    with pytest.raises(ValueError):
        codecs.e2m1_encode(np.array([np.inf]))


# ---------------------------------------------------------------- golden


def test_golden_e4m3():
    for val, code in _golden("e4m3"):
        assert int(codecs.e4m3_encode(np.array([float(val)]))[0]) == int(code, 16), val


def test_golden_e2m1():
    for val, code in _golden("e2m1"):
        assert int(codecs.e2m1_encode(np.array([float(val)]))[0]) == int(code, 16), val


def test_golden_e8m0():
    for b, val in _golden("e8m0"):
        assert codecs.e8m0_decode(np.array([int(b)], np.uint8))[0] == float(val)
