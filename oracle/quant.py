"""Block quantisers of the layer (oracle; test infrastructure).

Activation quantisation (hidden states x, and the SwiGLU intermediate h):

* The b12x fused MoE takes bf16 hidden states and quantises them inside the
  kernel [vLLM PR 40082 report, "Key source excerpts", class docstring of the
  b12x experts].
* The intermediate activation uses dynamic per-block quantisation with the
  calibrated global scale replaced by 1.0, because the calibrated value
  saturates [vLLM PR 40082 report, "Key source excerpts"
  (process_weights_after_loading) and "Review highlights", the a2_gscale item].
* Block sizes 16 (NVFP4) and 32 (MXFP8) come from the per-block-16 /
  per-block-32 quantise helpers [MegaMoE drop workflow, §3 "kernel_helpers.py"].

Readings (the pages give no formulas for the dynamic block scales):

* MXFP8 block of 32: OCP MX v1.0 rule.  amax = max |v|;
  s = clamp(floor(log2 amax) - 8, -127, 127) (8 = exponent of e4m3's largest
  power of two; amax = 0 gives s = -127); scale byte = s + 127;
  code = e4m3_rne_satfinite(v * 2^-s).  The scaling is by a power of two, so
  it is exact, and no division is involved.
* NVFP4 block of 16, global scale 1: sc = e4m3_rne_satfinite(fp32(amax / 6))
  (6 = largest e2m1 magnitude); sc = 0 gives zero codes (sign kept);
  otherwise code = e2m1_rne_satfinite(v / sc), decided by comparing |v|
  with the exact midpoints {.25, .75, 1.25, 1.75, 2.5, 3.5, 5} * sc.
* Decisions are taken on fp32 inputs (the kernel's precision): callers pass
  fp32 arrays (bf16 values are exact in fp32).

Weight quantisation of the synthetic test weights (a harness step, not part of
the layer), following the NVFP4 weight convention the pages state: block scale
= block amax * global scale / 6 (6 = fp4 max), dequant multiplier
alpha = 1 / global scale [vLLM PR 40082 report, "Key source excerpts",
comment in process_weights_after_loading].  Reading: global scale
= 6 * 448 / amax over the whole expert tensor, so alpha_e = amax_e / 2688, and
the fp32 alpha is kept (not folded into the e4m3 block scales).

* BF16 weights: round to nearest even.
* MXFP8 weights: the MXFP8 block rule above, along K, per 32.
* NVFP4 weights (fp32 arithmetic, each step correctly rounded):
  alpha = fp32(amax_e / 2688) (1.0 if amax_e == 0);
  sc = e4m3_rne_satfinite(fp32(fp32(amax_blk / 6) / alpha));
  code = e2m1_rne_satfinite(fp32(w / fp32(sc * alpha))) (zero if sc == 0).
  Dequantised weight = code * sc * alpha.
"""
from __future__ import annotations

import numpy as np

from . import codecs

MX_BLOCK = 32
NV_BLOCK = 16
E4M3_EMAX = 8      # 448 = 1.75 * 2^8
NVFP4_WEIGHT_GS_DEN = 6.0 * 448.0  # fp4 max * e4m3 max


def _blocks(v: np.ndarray, b: int) -> np.ndarray:
    v = np.asarray(v)
    if v.shape[-1] % b:
        raise ValueError(f"last dimension {v.shape[-1]} is not a multiple of {b}")
    return v.reshape(v.shape[:-1] + (v.shape[-1] // b, b))


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for a > 0, exact (from the binary exponent)."""
    _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    return e - 1


# ------------------------------------------------------------------- MXFP8


def mxfp8_quantize(v32: np.ndarray):
    """MX block quantisation along the last axis (block 32).

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32]).
    """
    v = np.asarray(v32, np.float32).astype(np.float64)
    b = _blocks(v, MX_BLOCK)
    amax = np.max(np.abs(b), axis=-1)
    s = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - E4M3_EMAX, -127)
    s = np.clip(s, -127, 127)
    codes = codecs.e4m3_encode(b * np.ldexp(1.0, -s)[..., None])
    return codes.reshape(v.shape), (s + 127).astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _blocks(codecs.e4m3_decode(codes), MX_BLOCK)
    out = q * codecs.e8m0_decode(scales)[..., None]
    return out.reshape(np.shape(codes))


# ------------------------------------------------------------------- NVFP4


def nvfp4_quantize(v32: np.ndarray):
    """NVFP4 block quantisation along the last axis (block 16, global 1).

    Returns (packed codes uint8 [..., K/2], e4m3 scale codes uint8 [..., K/16]).
    """
    v = np.asarray(v32, np.float32)
    b32 = _blocks(v, NV_BLOCK)
    amax = np.max(np.abs(b32), axis=-1)                       # fp32, exact
    sc_code = codecs.e4m3_encode(amax / np.float32(6.0))      # fp32 division
    sc = codecs.e4m3_decode(sc_code)
    b = b32.astype(np.float64)
    safe = np.where(sc > 0, sc, 1.0)
    codes = codecs.e2m1_encode(b, safe[..., None])
    codes = np.where((sc > 0)[..., None], codes, codes & 0x8)  # sc == 0: zero
    return codecs.pack_e2m1(codes.reshape(v.shape)), sc_code


def nvfp4_dequantize(packed: np.ndarray, scales: np.ndarray, alpha=1.0) -> np.ndarray:
    q = _blocks(codecs.e2m1_decode(codecs.unpack_e2m1(packed)), NV_BLOCK)
    out = q * codecs.e4m3_decode(scales)[..., None]
    out = out.reshape(q.shape[:-2] + (-1,))
    return out * np.float64(np.float32(alpha))


def nvfp4_quantize_weight(w32: np.ndarray):
    """Quantise one expert's fp32 weight tensor [rows, K] to NVFP4.

    Returns (packed uint8 [rows, K/2], e4m3 scales uint8 [rows, K/16], alpha fp32).
    """
    w = np.asarray(w32, np.float32)
    amax_e = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    alpha = np.float32(amax_e / np.float32(NVFP4_WEIGHT_GS_DEN)) if amax_e > 0 else np.float32(1.0)
    b = _blocks(w, NV_BLOCK)
    amax = np.max(np.abs(b), axis=-1)
    t = (amax / np.float32(6.0)).astype(np.float32)
    u = (t / alpha).astype(np.float32)
    sc_code = codecs.e4m3_encode(u)
    sc = codecs.e4m3_decode(sc_code).astype(np.float32)       # exact
    d = (sc * alpha).astype(np.float32)
    pos = d > 0
    r = (b / np.where(pos, d, np.float32(1.0))[..., None]).astype(np.float32)
    codes = codecs.e2m1_encode(r)
    codes = np.where(pos[..., None], codes, codes & 0x8)
    return codecs.pack_e2m1(codes.reshape(w.shape)), sc_code, alpha


def nvfp4_fold_global_scale(scales: np.ndarray, alpha):
    """Fold an NVFP4 weight tensor's alpha into its block scales, as the pages'
    weight preprocessing does [vLLM PR 40082 report, "Key source excerpts",
    process_weights_after_loading: the block scales are multiplied in fp32 by
    the per-tensor factor and cast back to e4m3; the factor becomes 1].

    Returns (new e4m3 scale codes, fp32 alpha 1.0)."""
    prod = (codecs.e4m3_decode(scales).astype(np.float32) * np.float32(alpha)).astype(np.float32)
    return codecs.e4m3_encode(prod), np.float32(1.0)


# ------------------------------------------------------------------- BF16


def bf16_quantize(v32: np.ndarray) -> np.ndarray:
    return codecs.bf16_encode(np.asarray(v32, np.float32))


def bf16_dequantize(bits: np.ndarray) -> np.ndarray:
    return codecs.bf16_decode(bits)


# ------------------------------------------------------------------- dispatch


def quantize_act(v32: np.ndarray, dtype: str):
    """Activation quantisation of the layer's format.

    Returns (codes, scales) where scales is None for bf16.
    """
    if dtype == "bf16":
        return bf16_quantize(v32), None
    if dtype == "mxfp8":
        return mxfp8_quantize(v32)
    if dtype == "nvfp4":
        return nvfp4_quantize(v32)
    raise ValueError(dtype)


def dequantize_act(codes, scales, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_dequantize(codes)
    if dtype == "mxfp8":
        return mxfp8_dequantize(codes, scales)
    if dtype == "nvfp4":
        return nvfp4_dequantize(codes, scales)
    raise ValueError(dtype)


def quantize_weight(w32: np.ndarray, dtype: str):
    """Canonical quantised form of one expert's weight tensor [rows, K].

    Returns (codes, scales, alpha): bf16 -> (bits, None, None);
    mxfp8 -> (e4m3 codes, e8m0 bytes, None); nvfp4 -> (packed, e4m3, alpha).
    """
    if dtype == "bf16":
        return bf16_quantize(w32), None, None
    if dtype == "mxfp8":
        c, s = mxfp8_quantize(w32)
        return c, s, None
    if dtype == "nvfp4":
        return nvfp4_quantize_weight(w32)
    raise ValueError(dtype)


def dequantize_weight(codes, scales, alpha, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_dequantize(codes)
    if dtype == "mxfp8":
        return mxfp8_dequantize(codes, scales)
    if dtype == "nvfp4":
        return nvfp4_dequantize(codes, scales, alpha)
    raise ValueError(dtype)
