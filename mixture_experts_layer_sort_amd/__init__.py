"""Python binding of libmoe_mi355x.so, the MI355X fused MoE expert layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions take torch tensors (device memory) or raw integer device
pointers, plus an optional stream (default: torch's current stream), and
raise MoeError on a non-zero status.  The names match the C ABI in
include/moe.h.  There is no CPU fallback: the first call (or `load()`) raises
ImportError if the library has not been built
(python -m mixture_experts_layer_sort_amd.build).
"""
from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmoe_mi355x.so")

MOE_BF16, MOE_MXFP8, MOE_NVFP4, MOE_BF16_MXFP8 = 0, 1, 2, 3
# layer formats; "bf16_mxfp8" = bf16 activations over MXFP8 weights
DTYPES = {"bf16": MOE_BF16, "mxfp8": MOE_MXFP8, "nvfp4": MOE_NVFP4, "bf16_mxfp8": MOE_BF16_MXFP8}
# expert activations: gated SwiGLU (W13 of 2I rows) or non-gated squared ReLU (W1 of I rows)
MOE_SWIGLU, MOE_RELU2 = 0, 1
ACTIVATIONS = {"swiglu": MOE_SWIGLU, "relu2": MOE_RELU2}

EXPORTED = [
    "moe_status_string",
    "moe_check_shape",
    "moe_packed_weight_bytes",
    "moe_workspace_bytes",
    "moe_xq_bytes",
    "moe_xq_scale_offset",
    "moe_xq_dequant_offset",
    "moe_hq_bytes",
    "moe_hq_scale_offset",
    "moe_hq_dequant_offset",
    "moe_quantize_weights",
    "moe_nvfp4_fold_global_scale",
    "moe_prepare_weights",
    "moe_route",
    "moe_permute",
    "moe_gemm13_swiglu_quant",
    "moe_gemm2",
    "moe_combine",
    "moe_forward",
    "moe_forward_fused",
    "moe_forward_noalloc",
    "moe_default_knobs",
    "moe_forward_knobs",
    "moe_knob_cache_lookup",
    "moe_workspace_init",
    "moe_batched_workspace_bytes",
    "moe_batched_experts",
    "moe_nvfp4_linear_packed_bytes",
    "moe_nvfp4_linear_workspace_bytes",
    "moe_nvfp4_linear_prepare",
    "moe_nvfp4_linear",
]


class MoeError(RuntimeError):
    pass


class moe_shape(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("gate_up_limit", ctypes.c_float),
    ]

    def __repr__(self):
        return (f"moe_shape(H={self.hidden}, I={self.inter}, E={self.num_experts}, k={self.top_k}, "
                f"max_tokens={self.max_tokens}, dtype={self.dtype}, activation={self.activation}, "
                f"gate_up_limit={self.gate_up_limit})")


class moe_knobs(ctypes.Structure):
    """How the grouped GEMMs of one call run (gemm variant 0 auto / 1 decode
    16-row / 2 decode 32-row / 3 prefill; MXFP8 fp8 down GEMM; prefill band
    rows; in-kernel fc2 reduce; persistent blocks per compute unit; prefill
    item deal over the XCDs and blocks)."""

    _fields_ = [
        ("gemm", ctypes.c_int32),
        ("down_fp8", ctypes.c_int32),
        ("band_rows", ctypes.c_int32),
        ("fc2_reduce", ctypes.c_int32),
        ("blocks_per_cu", ctypes.c_int32),
        ("load_balance", ctypes.c_int32),
    ]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}

    def __repr__(self):
        return "moe_knobs(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"


# the knob cache shipped with the package (written by mixture_experts_layer_sort_amd.tune);
# the environment variable MOE_KNOB_CACHE names another file
KNOB_CACHE_PATH = os.path.join(_PKG_DIR, "knob_cache.txt")


def make_shape(hidden, inter, num_experts, top_k, max_tokens, dtype, activation="swiglu",
               gate_up_limit=0.0) -> moe_shape:
    d = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    a = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    return moe_shape(hidden, inter, num_experts, top_k, max_tokens, d, a, gate_up_limit)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_sort_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(moe_shape), ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_check_shape": (I32, [S]),
        "moe_packed_weight_bytes": (SZ, [S]),
        "moe_workspace_bytes": (SZ, [S]),
        "moe_xq_bytes": (SZ, [S, I32]),
        "moe_xq_scale_offset": (SZ, [S, I32]),
        "moe_hq_bytes": (SZ, [S, I32]),
        "moe_hq_scale_offset": (SZ, [S, I32]),
        "moe_xq_dequant_offset": (SZ, [S, I32]),
        "moe_hq_dequant_offset": (SZ, [S, I32]),
        "moe_quantize_weights": (I32, [I32, I32, I32, I32, P, P, P, P, P]),
        "moe_nvfp4_fold_global_scale": (I32, [I32, I32, I32, P, P, P, P, P]),
        "moe_prepare_weights": (I32, [S, P, P, P, P, P, P, P, SZ, P]),
        "moe_route": (I32, [S, I32, P, P, P, P]),
        "moe_permute": (I32, [S, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_gemm13_swiglu_quant": (I32, [S, I32, P, P, P, P, P, P, SZ, P]),
        "moe_gemm2": (I32, [S, I32, P, P, P, P, P, P, SZ, P]),
        "moe_combine": (I32, [S, I32, P, P, P, P]),
        "moe_forward": (I32, [S, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_forward_fused": (I32, [S, I32, P, P, P, P, P, P, P, SZ, P]),
        "moe_forward_noalloc": (I32, [S, I32, P, P, P, P, P, P, P]),
        "moe_default_knobs": (None, [ctypes.POINTER(moe_knobs)]),
        "moe_forward_knobs": (I32, [S, I32, P, P, P, P, P, P, P, SZ, ctypes.POINTER(moe_knobs), P]),
        "moe_knob_cache_lookup": (I32, [ctypes.c_char_p, S, I32, ctypes.POINTER(moe_knobs),
                                        ctypes.POINTER(ctypes.c_int32)]),
        "moe_batched_workspace_bytes": (SZ, [S, I32]),
        "moe_batched_experts": (I32, [S, I32, P, P, P, P, P, SZ, P]),
        "moe_nvfp4_linear_packed_bytes": (SZ, [I32, I32]),
        "moe_nvfp4_linear_workspace_bytes": (SZ, [I32, I32]),
        "moe_nvfp4_linear_prepare": (I32, [I32, I32, P, P, P, P, SZ, P]),
        "moe_nvfp4_linear": (I32, [I32, I32, I32, P, P, P, P, SZ, P]),
        "moe_workspace_init": (I32, [S, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


class _Lazy:
    """Loads the shared library on first attribute access."""

    _handle = None

    def __getattr__(self, name):
        if _Lazy._handle is None:
            _Lazy._handle = _load()
        return getattr(_Lazy._handle, name)


_lib = _Lazy()


def load():
    """Load (or return) the ctypes handle of the library; raises if missing."""
    _lib.moe_check_shape  # noqa: B018 (forces the load)
    return _Lazy._handle


def _ptr(x):
    """Device address of a tensor, an int, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != 0:
        raise MoeError(f"{what}: {_lib.moe_status_string(status).decode()} ({status})")


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


# ----------------------------------------------------------------- sizes


def moe_check_shape(shape: moe_shape) -> int:
    return _lib.moe_check_shape(ctypes.byref(shape))


def moe_packed_weight_bytes(shape: moe_shape) -> int:
    return _lib.moe_packed_weight_bytes(ctypes.byref(shape))


def moe_workspace_bytes(shape: moe_shape) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shape))


def moe_xq_bytes(shape: moe_shape, T: int) -> int:
    return _lib.moe_xq_bytes(ctypes.byref(shape), T)


def moe_xq_scale_offset(shape: moe_shape, T: int) -> int:
    return _lib.moe_xq_scale_offset(ctypes.byref(shape), T)


def moe_hq_bytes(shape: moe_shape, T: int) -> int:
    return _lib.moe_hq_bytes(ctypes.byref(shape), T)


def moe_hq_scale_offset(shape: moe_shape, T: int) -> int:
    return _lib.moe_hq_scale_offset(ctypes.byref(shape), T)


def moe_xq_dequant_offset(shape: moe_shape, T: int) -> int:
    return _lib.moe_xq_dequant_offset(ctypes.byref(shape), T)


def moe_hq_dequant_offset(shape: moe_shape, T: int) -> int:
    return _lib.moe_hq_dequant_offset(ctypes.byref(shape), T)


# ----------------------------------------------------------------- entry points


def moe_quantize_weights(dtype, count, rows, K, w, codes, scales=None, alpha=None, stream=None):
    d = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(_lib.moe_quantize_weights(d, count, rows, K, _ptr(w), _ptr(codes), _ptr(scales), _ptr(alpha),
                                     _stream(stream)), "moe_quantize_weights")


def moe_nvfp4_fold_global_scale(count, rows, K, scales_in, alpha_in, scales_out=None, alpha_out=None, stream=None):
    """NVFP4 weights: fold alpha into the block scales (in place unless outputs are given)."""
    so = scales_in if scales_out is None else scales_out
    ao = alpha_in if alpha_out is None else alpha_out
    _check(_lib.moe_nvfp4_fold_global_scale(count, rows, K, _ptr(scales_in), _ptr(alpha_in), _ptr(so), _ptr(ao),
                                            _stream(stream)), "moe_nvfp4_fold_global_scale")


def moe_prepare_weights(shape, w13_codes, w13_scales, w13_alpha, w2_codes, w2_scales, w2_alpha, packed,
                        packed_bytes=None, stream=None):
    nbytes = packed_bytes if packed_bytes is not None else packed.numel() * packed.element_size()
    _check(_lib.moe_prepare_weights(ctypes.byref(shape), _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_alpha),
                                    _ptr(w2_codes), _ptr(w2_scales), _ptr(w2_alpha), _ptr(packed), nbytes,
                                    _stream(stream)), "moe_prepare_weights")


def moe_route(shape, T, logits, topk_ids, topk_w, stream=None):
    _check(_lib.moe_route(ctypes.byref(shape), T, _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _stream(stream)),
           "moe_route")


def moe_permute(shape, T, topk_ids, x, offsets, sorted_pairs, pair_pos, xq, ws=None, ws_bytes=0, stream=None):
    _check(_lib.moe_permute(ctypes.byref(shape), T, _ptr(topk_ids), _ptr(x), _ptr(offsets), _ptr(sorted_pairs),
                            _ptr(pair_pos), _ptr(xq), _ptr(ws), ws_bytes, _stream(stream)), "moe_permute")


def moe_gemm13_swiglu_quant(shape, T, packed, offsets, sorted_pairs, xq, hq, ws=None, ws_bytes=0, stream=None):
    _check(_lib.moe_gemm13_swiglu_quant(ctypes.byref(shape), T, _ptr(packed), _ptr(offsets), _ptr(sorted_pairs),
                                        _ptr(xq), _ptr(hq), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_gemm13_swiglu_quant")


def moe_gemm2(shape, T, packed, offsets, sorted_pairs, hq, y, ws=None, ws_bytes=0, stream=None):
    _check(_lib.moe_gemm2(ctypes.byref(shape), T, _ptr(packed), _ptr(offsets), _ptr(sorted_pairs), _ptr(hq),
                          _ptr(y), _ptr(ws), ws_bytes, _stream(stream)), "moe_gemm2")


def moe_combine(shape, T, y, topk_w, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(shape), T, _ptr(y), _ptr(topk_w), _ptr(out), _stream(stream)),
           "moe_combine")


def moe_forward(shape, T, packed, logits, x, out, ws, ws_bytes=None, topk_ids=None, topk_w=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.moe_forward(ctypes.byref(shape), T, _ptr(packed), _ptr(logits), _ptr(x), _ptr(out),
                            _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)), "moe_forward")


def moe_forward_fused(shape, T, packed, logits, x, out, ws, ws_bytes=None, topk_ids=None, topk_w=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.moe_forward_fused(ctypes.byref(shape), T, _ptr(packed), _ptr(logits), _ptr(x), _ptr(out),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes, _stream(stream)), "moe_forward_fused")


def moe_forward_noalloc(shape, T, packed, logits, x, out, topk_ids=None, topk_w=None, stream=None):
    """moe_forward with its intermediates in the library's static device scratch (no workspace)."""
    _check(_lib.moe_forward_noalloc(ctypes.byref(shape), T, _ptr(packed), _ptr(logits), _ptr(x), _ptr(out),
                                    _ptr(topk_ids), _ptr(topk_w), _stream(stream)), "moe_forward_noalloc")


def moe_default_knobs() -> moe_knobs:
    kn = moe_knobs()
    _lib.moe_default_knobs(ctypes.byref(kn))
    return kn


def make_knobs(gemm=0, down_fp8=1, band_rows=0, fc2_reduce=0, blocks_per_cu=0, load_balance=0) -> moe_knobs:
    return moe_knobs(gemm, down_fp8, band_rows, fc2_reduce, blocks_per_cu, load_balance)


def moe_forward_knobs(shape, T, packed, logits, x, out, ws, knobs=None, ws_bytes=None, topk_ids=None, topk_w=None,
                      stream=None):
    """moe_forward with explicit knobs (None: the defaults)."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    kp = ctypes.byref(knobs) if knobs is not None else None
    _check(_lib.moe_forward_knobs(ctypes.byref(shape), T, _ptr(packed), _ptr(logits), _ptr(x), _ptr(out),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes, kp, _stream(stream)),
           "moe_forward_knobs")


def moe_knob_cache_lookup(shape, T, path=None):
    """(knobs, found) for `shape` at T tokens from the knob cache at `path`
    (default: $MOE_KNOB_CACHE, else the package's knob_cache.txt)."""
    path = path or os.environ.get("MOE_KNOB_CACHE") or KNOB_CACHE_PATH
    kn, found = moe_knobs(), ctypes.c_int32(0)
    _check(_lib.moe_knob_cache_lookup(os.fsencode(path), ctypes.byref(shape), T, ctypes.byref(kn),
                                      ctypes.byref(found)), "moe_knob_cache_lookup")
    return kn, bool(found.value)


def moe_workspace_init(shape, ws, ws_bytes=None, stream=None):
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.moe_workspace_init(ctypes.byref(shape), _ptr(ws), nbytes, _stream(stream)), "moe_workspace_init")


def moe_batched_workspace_bytes(shape: moe_shape, max_rows: int) -> int:
    return _lib.moe_batched_workspace_bytes(ctypes.byref(shape), max_rows)


def moe_batched_experts(shape, max_rows, counts, x, packed, y, ws, ws_bytes=None, stream=None):
    """Expert MLPs on tokens bucketed per expert: x, y bf16 [E, max_rows, H], counts int32 [E]."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.moe_batched_experts(ctypes.byref(shape), max_rows, _ptr(counts), _ptr(x), _ptr(packed), _ptr(y),
                                    _ptr(ws), nbytes, _stream(stream)), "moe_batched_experts")


def moe_nvfp4_linear_packed_bytes(N: int, K: int) -> int:
    return _lib.moe_nvfp4_linear_packed_bytes(N, K)


def moe_nvfp4_linear_workspace_bytes(max_M: int, K: int) -> int:
    return _lib.moe_nvfp4_linear_workspace_bytes(max_M, K)


def moe_nvfp4_linear_prepare(N, K, codes, scales, alpha, packed, packed_bytes=None, stream=None):
    nbytes = packed_bytes if packed_bytes is not None else packed.numel() * packed.element_size()
    _check(_lib.moe_nvfp4_linear_prepare(N, K, _ptr(codes), _ptr(scales), _ptr(alpha), _ptr(packed), nbytes,
                                         _stream(stream)), "moe_nvfp4_linear_prepare")


def moe_nvfp4_linear(M, N, K, packed, x, out, ws, ws_bytes=None, stream=None):
    """out bf16 [M, N] = NVFP4(x bf16 [M, K]) . W^T (dense NVFP4 linear layer)."""
    nbytes = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(_lib.moe_nvfp4_linear(M, N, K, _ptr(packed), _ptr(x), _ptr(out), _ptr(ws), nbytes, _stream(stream)),
           "moe_nvfp4_linear")
