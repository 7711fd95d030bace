"""Pins of the oracle's in-kernel activation quantisation (oracle.moe.quantize_x):
hand-derived rows per layer format, and an E=1 layer whose hidden states
every format represents exactly, checked against a dense MLP on the raw x.

The layer takes bf16 hidden states and quantises them inside the kernel
[vLLM PR 40082 report, "Key source excerpts", class docstring of the b12x
experts]: NVFP4 per 16 with global scale 1, MXFP8 per 32 [MegaMoE drop
workflow, §3, the per-block quantise helpers]; the bf16 layer and the bf16 x
MXFP8 layer take x as given.  The expected codes follow the rules of
tests/golden/codec_cases.txt (OCP e4m3fn / e2m1 / e8m0, nearest, ties to even,
saturating); each derivation is written next to the value.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_inputs as mi
from oracle import codecs, moe, quant

H = 64  # two MX blocks, four NVFP4 blocks


def _row(vals):
    """bf16 bits of a row of H values given as {index: value} (the rest 0)."""
    a = np.zeros((1, H), np.float32)
    for i, v in vals.items():
        a[0, i] = v
    bits = mi.f32_to_bf16_bits(a)
    assert np.array_equal(mi.bf16_bits_to_f32(bits), a), "row values must be bf16-exact"
    return bits


# 0.30078125 is bf16(0.3) (0x3E9A): exact in bf16, not on any grid used below
X03 = 0.30078125
ROW = {0: 480.0, 32: -3.0, 33: 1.0, 34: X03}


def test_quantize_x_mxfp8_golden():
    x = _row(ROW)
    c, s, d = moe.quantize_x(x, "mxfp8")
    assert c.shape == (1, H) and c.dtype == np.uint8 and s.shape == (1, 2)
    # block 0: amax 480, floor(log2 480) = 8, s = 0 (byte 127); 480 saturates to 448 (0x7E)
    # block 1: amax 3, floor(log2 3) = 1, s = -7 (byte 120); scaled by 2^7:
    #   -3 -> -384 = -1.5*2^8 (0xFC); 1 -> 128 = 2^7 (exponent 14, 0x70);
    #   X03 -> 38.5, between 36 and 40 (spacing 4 in [32, 64)) -> 40 = 1.25*2^5 (0x62)
    exp_c = np.zeros(H, np.uint8)
    exp_c[0], exp_c[32], exp_c[33], exp_c[34] = 0x7E, 0xFC, 0x70, 0x62
    assert np.array_equal(s[0], np.array([127, 120], np.uint8))
    assert np.array_equal(c[0], exp_c)
    exp_d = np.zeros(H)
    exp_d[0], exp_d[32], exp_d[33], exp_d[34] = 448.0, -3.0, 1.0, 40.0 / 128
    assert np.array_equal(d[0], exp_d)


def test_quantize_x_nvfp4_golden():
    x = _row({0: 6.0, 16: 3.0, 17: 1.0, 18: X03, 32: -2.0})
    c, s, d = moe.quantize_x(x, "nvfp4")
    assert c.shape == (1, H // 2) and s.shape == (1, 4)
    # block 0: amax/6 = 1 -> scale 0x38; 6/1 = 6 -> idx 7
    # block 1: amax/6 = 0.5 -> 0x30; 3/0.5 = 6 -> 7; 1/0.5 = 2 -> idx 4; X03/0.5 = 0.60 -> 0.5 (idx 1)
    # block 2: amax/6 = 0.333 -> 1.375*2^-2 = 0.34375 (0x2B); -2/0.34375 = -5.82 -> -6 (0xF)
    # block 3: all zero -> scale 0, codes 0
    assert np.array_equal(s[0], np.array([0x38, 0x30, 0x2B, 0x00], np.uint8))
    exp_c = np.zeros(H // 2, np.uint8)
    exp_c[0] = 0x07                 # elements 0 (low nibble) and 1
    exp_c[8] = 0x07 | (0x04 << 4)   # elements 16, 17
    exp_c[9] = 0x01                 # element 18
    exp_c[16] = 0x0F                # element 32
    assert np.array_equal(c[0], exp_c)
    exp_d = np.zeros(H)
    exp_d[0], exp_d[16], exp_d[17], exp_d[18], exp_d[32] = 6.0, 3.0, 1.0, 0.25, -6 * 0.34375
    assert np.array_equal(d[0], exp_d)


@pytest.mark.parametrize("dtype", ["bf16", "bf16_mxfp8"])
def test_quantize_x_bf16_passthrough(dtype):
    x = _row(ROW)
    c, s, d = moe.quantize_x(x, dtype)
    assert s is None
    assert c.dtype == np.uint16 and np.array_equal(c, x)  # the bf16 bits themselves
    assert np.array_equal(d, mi.bf16_bits_to_f32(x).astype(np.float64))


def test_quantize_x_formats_disagree():
    """The same row gives a different result per activation format, so a
    dispatch to the wrong rule cannot pass the goldens above."""
    x = _row(ROW)
    d = {f: moe.quantize_x(x, f)[2] for f in ("bf16", "mxfp8", "nvfp4")}
    assert not np.array_equal(d["bf16"], d["mxfp8"])
    assert not np.array_equal(d["bf16"], d["nvfp4"])
    assert not np.array_equal(d["mxfp8"], d["nvfp4"])


def _representable_x(T, rng):
    """Hidden states that every format represents exactly: every block of 16
    holds values of {0, +-.5, +-1, +-1.5, +-2, +-3, +-4} and one +-6, so the
    NVFP4 scale is 6/6 = 1 and MX scales values by 2^6 onto e4m3 grid points."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4], np.float32)
    x = grid[rng.integers(0, len(grid), (T, H))] * rng.choice([-1.0, 1.0], (T, H)).astype(np.float32)
    x[:, ::16] = 6.0 * rng.choice([-1.0, 1.0], (T, H // 16))
    return mi.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4", "bf16_mxfp8"])
def test_representable_x_passes_unchanged(dtype):
    x = _representable_x(5, np.random.default_rng(0))
    _, _, d = moe.quantize_x(x, dtype)
    assert np.array_equal(d, mi.bf16_bits_to_f32(x).astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4", "bf16_mxfp8"])
def test_e1_layer_on_representable_x_is_dense_mlp_of_raw_x(dtype):
    """E=1, top-1 layer on exactly representable x equals the dense SwiGLU MLP
    of the raw x (torch.nn.functional, fp64): the layer's own quantisation of x
    (in whichever format) must leave such x unchanged."""
    w = mi.Workload(f"qx_{dtype}", 6, H, 64, 1, 1, dtype, "none", 93)
    w13, w2 = mi.host_all_master_weights(w)
    W = moe.quantize_weights({0: w13[0]}, {0: w2[0]}, dtype)
    x = _representable_x(w.T, np.random.default_rng(1))
    logits = np.zeros((w.T, 1), np.float32)
    r = moe.moe_layer(x, logits, W, 1)
    W13, W2 = W.dequant(0)
    xt = torch.from_numpy(mi.bf16_bits_to_f32(x).astype(np.float64))
    I = W13.shape[0] // 2
    h = (F.silu(F.linear(xt, torch.from_numpy(W13[:I]))) * F.linear(xt, torch.from_numpy(W13[I:]))).numpy()
    act = "bf16" if dtype == "bf16_mxfp8" else dtype
    c, s = quant.quantize_act(h.astype(np.float32), act)
    ref = F.linear(torch.from_numpy(quant.dequantize_act(c, s, act)), torch.from_numpy(W2)).numpy()
    assert np.allclose(r.out_f64, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r.out, codecs.bf16_encode(ref.astype(np.float32)))
