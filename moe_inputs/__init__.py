"""Seeded synthetic inputs for the fused MoE expert layer.

This module is shared by the CPU oracle and the HIP library's tests and
benchmark.  It holds no arithmetic of the layer itself: it only draws random
numbers, adds the routing-skew biases that define the workloads, and casts to
the storage types the workloads name (bf16 hidden states, fp32 logits, fp32
master weights).  Quantisation of the master weights into MXFP8 / NVFP4 is NOT
done here (the oracle and the library each have their own quantiser).

Workloads (shapes and value distributions of the layer the pages describe):

=================  =====  ====  ====  ===  ==  =====  ===========================
name               T      H     I     E    k   dtype  routing skew
=================  =====  ====  ====  ===  ==  =====  ===========================
tiny_bf16          16     256   512   8    2   bf16   none
bf16_decode        64     4096  1408  64   6   bf16   none
mxfp8_decode       32     7168  2048  256  8   mxfp8  + N(0, 2) bias per expert
nvfp4_decode_t8    8      7168  2048  384  8   nvfp4  none
nvfp4_decode_t128  128    7168  2048  384  8   nvfp4  none
mxfp8_prefill      8192   7168  2048  256  8   mxfp8  + Zipf(1.1) popularity bias
=================  =====  ====  ====  ===  ==  =====  ===========================

x ~ N(0,1) rounded to bf16; logits ~ N(0,1) fp32 (+ bias); master weights
~ N(0, 0.02) fp32 (std 0.02), W13 = [E, 2I, H] (gate rows first, then up rows),
W2 = [E, H, I].

Seeds: numpy ``default_rng([cid, stream, sub])`` with stream 0 = x, 1 = logits,
2 = expert bias, 3 = W13, 4 = W2 and sub = expert id for weights.  The two
NVFP4 workloads share cid 4, so the T=8 case is the first 8 tokens of the
T=128 case and both see the same experts.  The device generators (torch on
the GPU) use the same (cid, stream, sub) triples mapped to one integer seed;
they are a different random stream from the host ones, for full-size runs.
"""
from __future__ import annotations

import dataclasses

import numpy as np

X_STREAM, LOGIT_STREAM, BIAS_STREAM, W13_STREAM, W2_STREAM = 0, 1, 2, 3, 4
WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts
    k: int          # experts per token
    dtype: str      # "bf16" | "mxfp8" | "nvfp4" | "bf16_mxfp8" (bf16 activations, MXFP8 weights)
    bias: str       # "none" | "normal2" | "zipf1.1"
    cid: int        # seed id of the workload
    act: str = "swiglu"  # "swiglu" (gated, W13 of 2I rows) | "relu2" (non-gated, W1 of I rows)
    fold: bool = False   # NVFP4: weight alpha folded into the block scales after quantisation
    limit: float = 0.0   # gate/up clamp of SwiGLU experts (0: none)

    @property
    def R13(self) -> int:
        """Rows of W13: 2I (gate and up) for SwiGLU, I (W1) for ReLU^2."""
        return 2 * self.I if self.act == "swiglu" else self.I

    @property
    def P(self) -> int:
        return self.T * self.k

    def scaled(self, **kw) -> "Workload":
        """Same workload with some sizes replaced (for small test cases)."""
        d = dataclasses.asdict(self)
        d.update(kw)
        if "name" not in kw:
            d["name"] = self.name + "_" + "_".join(f"{a}{b}" for a, b in sorted(kw.items()))
        return Workload(**d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_bf16", 16, 256, 512, 8, 2, "bf16", "none", 1),
        Workload("bf16_decode", 64, 4096, 1408, 64, 6, "bf16", "none", 2),
        Workload("mxfp8_decode", 32, 7168, 2048, 256, 8, "mxfp8", "normal2", 3),
        Workload("nvfp4_decode_t8", 8, 7168, 2048, 384, 8, "nvfp4", "none", 4),
        Workload("nvfp4_decode_t128", 128, 7168, 2048, 384, 8, "nvfp4", "none", 4),
        Workload("mxfp8_prefill", 8192, 7168, 2048, 256, 8, "mxfp8", "zipf1.1", 5),
        # bf16 activations over the MXFP8 layers' weights (same seeds, same weights)
        Workload("bf16_mxfp8_decode", 32, 7168, 2048, 256, 8, "bf16_mxfp8", "normal2", 3),
        Workload("bf16_mxfp8_prefill", 8192, 7168, 2048, 256, 8, "bf16_mxfp8", "zipf1.1", 5),
        # non-gated squared-ReLU experts (W1 of I rows) at the NVFP4 decode shape
        Workload("relu2_nvfp4_decode_t128", 128, 7168, 2048, 384, 8, "nvfp4", "none", 4, "relu2"),
        # NVFP4 weights with the per-tensor alpha folded into the block scales (same masters)
        Workload("nvfp4_folded_decode_t128", 128, 7168, 2048, 384, 8, "nvfp4", "none", 4, "swiglu", True),
        # SwiGLU experts with a gate/up clamp at 1.0 (gate and up values have a
        # standard deviation of ~1.7 at this shape, so about half are clamped)
        Workload("clamp_mxfp8_decode", 32, 7168, 2048, 256, 8, "mxfp8", "normal2", 3, "swiglu", False, 1.0),
    ]
}


def _rng(cid: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([cid, stream, sub])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Storage cast fp32 -> bf16 (torch's round-to-nearest-even cast), as uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- biases


def expert_bias(w: Workload) -> np.ndarray:
    """Per-expert logit bias that skews routing (fp32 [E])."""
    if w.bias == "none":
        return np.zeros(w.E, np.float32)
    g = _rng(w.cid, BIAS_STREAM)
    if w.bias == "normal2":
        # mean 0, standard deviation 2
        return g.normal(0.0, 2.0, w.E).astype(np.float32)
    if w.bias == "zipf1.1":
        # expert popularity p_e proportional to rank_e ** -1.1, ranks a seeded
        # permutation of 1..E; the bias is ln p_e (normalised).
        rank = g.permutation(w.E) + 1
        p = rank.astype(np.float64) ** -1.1
        p /= p.sum()
        return np.log(p).astype(np.float32)
    raise ValueError(w.bias)


# ---------------------------------------------------------------- host (numpy)


def host_x(w: Workload) -> np.ndarray:
    """Hidden states x ~ N(0,1), bf16 bits uint16 [T, H]."""
    a = _rng(w.cid, X_STREAM).standard_normal((w.T, w.H), dtype=np.float32)
    return f32_to_bf16_bits(a)


def host_logits(w: Workload) -> np.ndarray:
    """Router logits ~ N(0,1) + expert bias, fp32 [T, E]."""
    a = _rng(w.cid, LOGIT_STREAM).standard_normal((w.T, w.E), dtype=np.float32)
    return (a + expert_bias(w)[None, :]).astype(np.float32)


def host_master_weights(w: Workload, e: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 master weights of expert e: W13 [R13, H], W2 [H, I], ~ N(0, 0.02)."""
    w13 = _rng(w.cid, W13_STREAM, e).standard_normal((w.R13, w.H), dtype=np.float32)
    w2 = _rng(w.cid, W2_STREAM, e).standard_normal((w.H, w.I), dtype=np.float32)
    return w13 * np.float32(WEIGHT_STD), w2 * np.float32(WEIGHT_STD)


def host_all_master_weights(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """All experts' fp32 master weights (small workloads only)."""
    w13 = np.empty((w.E, w.R13, w.H), np.float32)
    w2 = np.empty((w.E, w.H, w.I), np.float32)
    for e in range(w.E):
        w13[e], w2[e] = host_master_weights(w, e)
    return w13, w2


# ---------------------------------------------------------------- device (torch)


def device_seed(cid: int, stream: int, sub: int = 0) -> int:
    return (cid * 1_000_003 + stream) * 65_537 + sub


def device_x(w: Workload, device="cuda"):
    """Hidden states x ~ N(0,1) as a bf16 torch tensor [T, H] on `device`."""
    import torch

    g = torch.Generator(device=device).manual_seed(device_seed(w.cid, X_STREAM))
    return torch.randn(w.T, w.H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def device_logits(w: Workload, device="cuda"):
    """Router logits ~ N(0,1) + expert bias, fp32 [T, E] on `device`."""
    import torch

    g = torch.Generator(device=device).manual_seed(device_seed(w.cid, LOGIT_STREAM))
    a = torch.randn(w.T, w.E, generator=g, device=device, dtype=torch.float32)
    return a + torch.from_numpy(expert_bias(w)).to(device)[None, :]


def device_master_weights(w: Workload, e: int, device="cuda"):
    """fp32 master weights of expert e on `device`: W13 [R13, H], W2 [H, I]."""
    import torch

    g = torch.Generator(device=device).manual_seed(device_seed(w.cid, W13_STREAM, e))
    w13 = torch.randn(w.R13, w.H, generator=g, device=device, dtype=torch.float32)
    g = torch.Generator(device=device).manual_seed(device_seed(w.cid, W2_STREAM, e))
    w2 = torch.randn(w.H, w.I, generator=g, device=device, dtype=torch.float32)
    return w13 * WEIGHT_STD, w2 * WEIGHT_STD
