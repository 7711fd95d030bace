"""GPU-side harness for the parity tests: builds a layer on the device through
the C ABI and unpacks its outputs into numpy for comparison with the oracle.

Nothing here computes any part of the layer: it allocates torch device
memory, calls the library's entry points and copies results back.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import mixture_experts_layer_sort_amd as lib
import moe_inputs as mi


def dev():
    return torch.device("cuda:0")


# the weight / activation formats of a layer format ("bf16_mxfp8": bf16
# activations over MXFP8 weights)
def weight_format(dtype):
    return "mxfp8" if dtype == "bf16_mxfp8" else dtype


def act_format(dtype):
    return "bf16" if dtype == "bf16_mxfp8" else dtype


def row_code_bytes(dtype, K):
    return {"bf16": 2 * K, "mxfp8": K, "nvfp4": K // 2}[act_format(dtype)]


def row_scale_bytes(dtype, K):
    return {"bf16": 0, "mxfp8": K // 32, "nvfp4": K // 16}[act_format(dtype)]


@dataclasses.dataclass
class CanonicalWeights:
    """Canonical quantised weights on the device (torch tensors)."""

    w13: torch.Tensor
    w2: torch.Tensor
    w13_s: torch.Tensor | None
    w2_s: torch.Tensor | None
    w13_a: torch.Tensor | None
    w2_a: torch.Tensor | None


def alloc_canonical(w: mi.Workload) -> CanonicalWeights:
    d, E, H, I, R = dev(), w.E, w.H, w.I, w.R13
    u8 = torch.uint8
    wf = weight_format(w.dtype)
    if wf == "bf16":
        return CanonicalWeights(torch.empty(E, R, H, dtype=torch.bfloat16, device=d),
                                torch.empty(E, H, I, dtype=torch.bfloat16, device=d), None, None, None, None)
    if wf == "mxfp8":
        return CanonicalWeights(torch.empty(E, R, H, dtype=u8, device=d), torch.empty(E, H, I, dtype=u8, device=d),
                                torch.empty(E, R, H // 32, dtype=u8, device=d),
                                torch.empty(E, H, I // 32, dtype=u8, device=d), None, None)
    return CanonicalWeights(torch.empty(E, R, H // 2, dtype=u8, device=d),
                            torch.empty(E, H, I // 2, dtype=u8, device=d),
                            torch.empty(E, R, H // 16, dtype=u8, device=d),
                            torch.empty(E, H, I // 16, dtype=u8, device=d),
                            torch.empty(E, dtype=torch.float32, device=d),
                            torch.empty(E, dtype=torch.float32, device=d))


def _sub(t, e):
    return None if t is None else t[e:e + 1]


def quantize_expert(w: mi.Workload, cw: CanonicalWeights, e: int, w13_f32: torch.Tensor, w2_f32: torch.Tensor):
    """Quantise expert e's fp32 master weights (device tensors) with the library."""
    lib.moe_quantize_weights(w.dtype, 1, w.R13, w.H, w13_f32, cw.w13[e:e + 1], _sub(cw.w13_s, e), _sub(cw.w13_a, e))
    lib.moe_quantize_weights(w.dtype, 1, w.H, w.I, w2_f32, cw.w2[e:e + 1], _sub(cw.w2_s, e), _sub(cw.w2_a, e))
    if w.fold:
        lib.moe_nvfp4_fold_global_scale(1, w.R13, w.H, _sub(cw.w13_s, e), _sub(cw.w13_a, e))
        lib.moe_nvfp4_fold_global_scale(1, w.H, w.I, _sub(cw.w2_s, e), _sub(cw.w2_a, e))


def canonical_from_host_master(w: mi.Workload):
    """Small workloads: host master weights -> device -> library quantiser.
    Returns (CanonicalWeights, host fp32 W13 [E,2I,H], host fp32 W2 [E,H,I])."""
    w13f, w2f = mi.host_all_master_weights(w)
    cw = alloc_canonical(w)
    t13 = torch.from_numpy(w13f).to(dev())
    t2 = torch.from_numpy(w2f).to(dev())
    lib.moe_quantize_weights(w.dtype, w.E, w.R13, w.H, t13, cw.w13, cw.w13_s, cw.w13_a)
    lib.moe_quantize_weights(w.dtype, w.E, w.H, w.I, t2, cw.w2, cw.w2_s, cw.w2_a)
    if w.fold:  # NVFP4: alpha folded into the block scales, in place
        lib.moe_nvfp4_fold_global_scale(w.E, w.R13, w.H, cw.w13_s, cw.w13_a)
        lib.moe_nvfp4_fold_global_scale(w.E, w.H, w.I, cw.w2_s, cw.w2_a)
    return cw, w13f, w2f


def canonical_to_numpy(cw: CanonicalWeights, experts=None):
    """Copy canonical weights (optionally a subset of experts) to host numpy,
    as the dict-of-arrays the oracle's Weights accepts."""
    def conv(t):
        if t is None:
            return None
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        if experts is None:
            a = t.cpu().numpy()
            return {e: a[e] for e in range(a.shape[0])}
        return {e: t[e].cpu().numpy() for e in experts}

    out = {n: conv(getattr(cw, n)) for n in ("w13", "w2", "w13_s", "w2_s", "w13_a", "w2_a")}
    for n in ("w13", "w2"):
        if out[n] is not None and next(iter(out[n].values())).dtype == np.int16:
            out[n] = {e: a.view(np.uint16) for e, a in out[n].items()}
    return out


class DeviceLayer:
    """One layer instance on the GPU: packed weights plus buffers for every
    stage of the staged entry points and the forward workspace."""

    def __init__(self, w: mi.Workload, cw: CanonicalWeights, max_tokens: int | None = None):
        self.w = w
        self.shape = lib.make_shape(w.H, w.I, w.E, w.k, max_tokens or w.T, w.dtype, w.act, w.limit)
        assert lib.moe_check_shape(self.shape) == 0, self.shape
        nbytes = lib.moe_packed_weight_bytes(self.shape)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=dev())
        lib.moe_prepare_weights(self.shape, cw.w13, cw.w13_s, cw.w13_a, cw.w2, cw.w2_s, cw.w2_a, self.packed)
        self.ws = torch.empty(lib.moe_workspace_bytes(self.shape), dtype=torch.uint8, device=dev())
        lib.moe_workspace_init(self.shape, self.ws)

    def staged(self, x: torch.Tensor, logits: torch.Tensor) -> dict:
        """Run the five staged entry points; returns device tensors."""
        w, s, d = self.w, self.shape, dev()
        T, P = x.shape[0], x.shape[0] * w.k
        r = {}
        r["ids"] = torch.empty(T, w.k, dtype=torch.int32, device=d)
        r["wts"] = torch.empty(T, w.k, dtype=torch.float32, device=d)
        lib.moe_route(s, T, logits, r["ids"], r["wts"])
        r["offsets"] = torch.empty(w.E + 1, dtype=torch.int32, device=d)
        r["sorted_pairs"] = torch.empty(max(P, 1), dtype=torch.int32, device=d)
        r["pair_pos"] = torch.empty(max(P, 1), dtype=torch.int32, device=d)
        r["xq"] = torch.empty(max(lib.moe_xq_bytes(s, T), 1), dtype=torch.uint8, device=d)
        lib.moe_permute(s, T, r["ids"], x, r["offsets"], r["sorted_pairs"], r["pair_pos"], r["xq"])
        r["hq"] = torch.empty(max(lib.moe_hq_bytes(s, T), 1), dtype=torch.uint8, device=d)
        lib.moe_gemm13_swiglu_quant(s, T, self.packed, r["offsets"], r["sorted_pairs"], r["xq"], r["hq"])
        r["y"] = torch.empty(max(P, 1), w.H, dtype=torch.bfloat16, device=d)
        lib.moe_gemm2(s, T, self.packed, r["offsets"], r["sorted_pairs"], r["hq"], r["y"])
        r["out"] = torch.empty(T, w.H, dtype=torch.bfloat16, device=d)
        lib.moe_combine(s, T, r["y"], r["wts"], r["out"])
        return r

    def forward(self, x: torch.Tensor, logits: torch.Tensor, out=None, ids=None, wts=None) -> torch.Tensor:
        T = x.shape[0]
        out = torch.empty(T, self.w.H, dtype=torch.bfloat16, device=dev()) if out is None else out
        lib.moe_forward(self.shape, T, self.packed, logits, x, out, self.ws, topk_ids=ids, topk_w=wts)
        return out

    def forward_fused(self, x: torch.Tensor, logits: torch.Tensor, out=None, ids=None, wts=None) -> torch.Tensor:
        T = x.shape[0]
        out = torch.empty(T, self.w.H, dtype=torch.bfloat16, device=dev()) if out is None else out
        lib.moe_forward_fused(self.shape, T, self.packed, logits, x, out, self.ws, topk_ids=ids, topk_w=wts)
        return out

    def forward_knobs(self, x: torch.Tensor, logits: torch.Tensor, knobs, out=None) -> torch.Tensor:
        T = x.shape[0]
        out = torch.empty(T, self.w.H, dtype=torch.bfloat16, device=dev()) if out is None else out
        lib.moe_forward_knobs(self.shape, T, self.packed, logits, x, out, self.ws, knobs)
        return out

    def sync_words(self) -> np.ndarray:
        """The fused kernel's synchronisation words (zero between launches;
        word 2 is its spin-timeout flag)."""
        return self.ws[: 4 * (4 + self.w.E)].cpu().numpy().view(np.uint32)

    # --------------------------------------------------------- unpacking
    def split_act(self, buf: torch.Tensor, rows: int, K: int, scale_off: int):
        dt = self.w.dtype
        a = buf.cpu().numpy()
        codes = a[: rows * row_code_bytes(dt, K)].reshape(rows, row_code_bytes(dt, K))
        if act_format(dt) == "bf16":
            return codes.view(np.uint16), None
        scales = a[scale_off: scale_off + rows * row_scale_bytes(dt, K)].reshape(rows, row_scale_bytes(dt, K))
        return codes, scales

    def xq_numpy(self, r, T):
        return self.split_act(r["xq"], T, self.w.H, lib.moe_xq_scale_offset(self.shape, T))

    def hq_numpy(self, r, T):
        return self.split_act(r["hq"], T * self.w.k, self.w.I, lib.moe_hq_scale_offset(self.shape, T))

    def dequant_numpy(self, buf: torch.Tensor, rows: int, K: int, off: int) -> np.ndarray:
        """The 16-bit dequantised copy of an MXFP8 (bf16) / NVFP4 (fp16) activation
        buffer, widened to float64."""
        a = buf[off: off + rows * K * 2].cpu().numpy().view(np.uint16).reshape(rows, K)
        if act_format(self.w.dtype) == "mxfp8":
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.view(np.float16).astype(np.float64)

    def xq_dequant(self, r, T):
        return self.dequant_numpy(r["xq"], T, self.w.H, lib.moe_xq_dequant_offset(self.shape, T))

    def hq_dequant(self, r, T):
        return self.dequant_numpy(r["hq"], T * self.w.k, self.w.I, lib.moe_hq_dequant_offset(self.shape, T))


def bf16_numpy(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_device_x(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x_bits.view(np.int16)).to(dev()).view(torch.bfloat16)


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a - b))


def out_tolerance(dtype: str) -> float:
    """Relative L2 bound on the layer output: 1e-2 (bf16, MXFP8), 3e-2 (NVFP4)."""
    return 3e-2 if dtype == "nvfp4" else 1e-2


def check_out(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: str, what=""):
    """The output bar: relL2 <= tol and max |diff| <= 5e-2 * RMS(reference)."""
    from oracle import codecs

    g = codecs.bf16_decode(got_bits)
    r = codecs.bf16_decode(ref_bits)
    rel = rel_l2(g, r)
    rms = float(np.sqrt(np.mean(r * r)))
    mad = float(np.max(np.abs(g - r))) if r.size else 0.0
    assert rel <= out_tolerance(dtype), f"{what}: relL2 {rel:.3e} > {out_tolerance(dtype)}"
    assert mad <= 5e-2 * rms, f"{what}: max|diff| {mad:.3e} > 5e-2 * RMS {rms:.3e}"
    return rel, mad / rms if rms else 0.0
