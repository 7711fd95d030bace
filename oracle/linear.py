"""Dense NVFP4 block-scaled linear layer (oracle; test infrastructure).

The pages' second b12x kernel is a dense GEMM for NVFP4 linear layers: the
bf16 activations are quantised to NVFP4 and multiplied by NVFP4 weights
[vLLM PR 40082 report, "Implementation" item 2: FlashInferB12xNvFp4LinearKernel,
apply_weights quantises with scaled_fp4_quant and calls the b12x scaled fp4
matrix product].  Readings (the pages give no formulas):

* weights W [N, K]: e2m1 codes, one e4m3 scale per 16 along K and one fp32
  alpha per tensor (= 1 / global scale), the NVFP4 weight convention of the
  MoE layer (oracle.quant, the same quantiser);
* activations: dynamic per-block NVFP4 quantisation of the bf16 rows with
  global scale 1, exactly as the MoE layer quantises its hidden states;
* out = bf16_rne( alpha * sum_k x_hat[m, k] * w_hat[n, k] ), the sum exact
  (float64 of exactly dequantised operands).
"""
from __future__ import annotations

import numpy as np

from . import codecs, quant


def nvfp4_linear(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, alpha: float):
    """x_bits bf16 [M, K]; codes [N, K/2], scales [N, K/16], alpha fp32.
    Returns (out bf16 bits [M, N], the float64 sum before rounding)."""
    x32 = codecs.bf16_decode(np.asarray(x_bits, np.uint16)).astype(np.float32)
    xc, xs = quant.quantize_act(x32, "nvfp4")
    xh = quant.dequantize_act(xc, xs, "nvfp4")
    wh = quant.dequantize_weight(codes, scales, alpha, "nvfp4")  # [N, K], alpha applied (exact per element)
    out64 = xh @ wh.T
    return codecs.bf16_encode(out64.astype(np.float32)), out64
