"""Pins of the oracle's dense NVFP4 linear layer: one-hot activations read
back weight columns (closed form), operands exactly representable in NVFP4
give torch.nn.functional.linear of the raw fp64 values, a power-of-two alpha
scales the output exactly, and the activation quantisation is the pinned
NVFP4 rule (golden rows of tests/golden/codec_cases.txt)."""
import numpy as np
import torch
import torch.nn.functional as F

import moe_inputs as mi
from oracle import codecs, linear, quant


def _weights(N, K, seed):
    w = (np.random.default_rng(seed).standard_normal((N, K)) * 0.02).astype(np.float32)
    return quant.quantize_weight(w, "nvfp4")


def test_one_hot_rows_read_weight_columns():
    N, K = 48, 64
    c, s, a = _weights(N, K, 1)
    wh = quant.dequantize_weight(c, s, a, "nvfp4")
    # x = 6 at column j (its block amax is 6: scale 1, code 6 exactly), 0 elsewhere
    x = np.zeros((K, K), np.float32)
    x[np.arange(K), np.arange(K)] = 6.0
    out_bits, out64 = linear.nvfp4_linear(mi.f32_to_bf16_bits(x), c, s, a)
    col = 6.0 * wh.T + 0.0  # (+0.0: the sum over k turns a -0 weight into +0)
    assert np.array_equal(out64, col)
    assert np.array_equal(out_bits, codecs.bf16_encode(col.astype(np.float32)))


def test_representable_operands_equal_dense_linear():
    M, N, K = 5, 40, 128
    rng = np.random.default_rng(2)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4], np.float32)
    x = grid[rng.integers(0, 7, (M, K))] * rng.choice([-1.0, 1.0], (M, K)).astype(np.float32)
    x[:, ::16] = 6.0  # every block's amax is 6: NVFP4 scale 1, every value exact
    c, s, a = _weights(N, K, 3)
    _, out64 = linear.nvfp4_linear(mi.f32_to_bf16_bits(x), c, s, a)
    wh = quant.dequantize_weight(c, s, a, "nvfp4")
    ref = F.linear(torch.from_numpy(x.astype(np.float64)), torch.from_numpy(wh)).numpy()
    assert np.allclose(out64, ref, rtol=1e-13, atol=1e-15)


def test_power_of_two_alpha_scales_exactly():
    M, N, K = 3, 16, 64
    c, s, a = _weights(N, K, 4)
    x = mi.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((M, K)).astype(np.float32))
    _, o1 = linear.nvfp4_linear(x, c, s, np.float32(a))
    _, o2 = linear.nvfp4_linear(x, c, s, np.float32(a) * np.float32(4.0))
    assert np.array_equal(o2, 4.0 * o1)


def test_activation_quantisation_is_the_nvfp4_rule():
    # first row of tests/golden/codec_cases.txt's nv block: 6.0 -> scale 0x38, code 7
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0
    xc, xs = quant.quantize_act(x, "nvfp4")
    assert xs[0, 0] == 0x38 and (xc[0, 0] & 0xF) == 0x7
