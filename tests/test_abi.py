"""CPU checks of the C ABI: the built library loads and exports every symbol
include/moe.h declares, the size queries agree with the documented layouts,
and invalid arguments are rejected on the host with the documented status
before anything is enqueued (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_sort_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    h = lib.load()
    for name in _declared():
        assert hasattr(h, name), name
    out = os.popen(f"nm -D --defined-only {lib.LIB_PATH}").read()
    exported = set(re.findall(r" T (moe_\w+)$", out, re.M))
    assert set(_declared()) <= exported


def S(H=256, I=512, E=8, k=2, T=16, dt="bf16", act="swiglu"):
    return lib.make_shape(H, I, E, k, T, dt, act)


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"H": 200}, UNSUPPORTED), ({"I": 100}, UNSUPPORTED), ({"H": 0}, UNSUPPORTED),
    ({"E": 0}, UNSUPPORTED), ({"E": 1025}, UNSUPPORTED), ({"E": 1024, "k": 32}, OK),
    ({"k": 0}, UNSUPPORTED), ({"k": 33, "E": 64}, UNSUPPORTED), ({"k": 9, "E": 8}, UNSUPPORTED),
    ({"T": 0}, UNSUPPORTED), ({"T": 1 << 22, "k": 8}, UNSUPPORTED), ({"dt": "bf16_mxfp8"}, OK),
    ({"dt": 4}, UNSUPPORTED), ({"dt": -1}, UNSUPPORTED),
    ({"act": "relu2"}, OK), ({"act": "relu2", "dt": "nvfp4"}, OK), ({"act": 2}, UNSUPPORTED), ({"act": -1}, UNSUPPORTED),
])
def test_shape_validation(kw, status):
    args = dict(H=256, I=512, E=8, k=2, T=16, dt="bf16")
    args.update(kw)
    assert lib.moe_check_shape(S(**args)) == status


def test_gate_up_limit_validation():
    s = S(256, 512, 8, 2, 16, "bf16")
    for limit, status in ((0.0, OK), (1.5, OK), (1e30, OK), (-1.0, INVALID), (float("nan"), INVALID),
                          (float("inf"), INVALID)):
        s.gate_up_limit = limit
        assert lib.moe_check_shape(s) == status, limit
    r = S(256, 512, 8, 2, 16, "bf16", "relu2")
    r.gate_up_limit = 1.0
    assert lib.moe_check_shape(r) == UNSUPPORTED  # the clamp belongs to SwiGLU experts


def test_batched_workspace_size():
    s = S(512, 256, 8, 2, 16, "mxfp8")
    n = lib.moe_batched_workspace_bytes(s, 24)
    R = 8 * 24
    xq = ((R * 512 + 255) // 256) * 256 + ((R * 16 + 255) // 256) * 256 + ((R * 512 * 2 + 255) // 256) * 256
    hq = ((R * 256 + 255) // 256) * 256 + ((R * 8 + 255) // 256) * 256 + ((R * 256 * 2 + 255) // 256) * 256
    assert n == 256 + ((R * 4 + 255) // 256) * 256 + xq + hq
    assert lib.moe_batched_workspace_bytes(s, 0) == 0
    assert lib.moe_batched_workspace_bytes(S(512, 256, 1024, 2, 16, "bf16"), 1 << 15) == 0  # E * rows > 2^24


def test_nvfp4_linear_sizes():
    N, K = 384, 512
    tiles = (N // 64) * (K // 128) * 4
    assert lib.moe_nvfp4_linear_packed_bytes(N, K) == tiles * 1024 + tiles * 128 + 256
    M = 5
    xq = ((M * K // 2 + 255) // 256) * 256 + ((M * K // 16 + 255) // 256) * 256 + ((M * K * 2 + 255) // 256) * 256
    assert lib.moe_nvfp4_linear_workspace_bytes(M, K) == 256 + 256 + xq
    assert lib.moe_nvfp4_linear_packed_bytes(96, 512) == 0 and lib.moe_nvfp4_linear_workspace_bytes(0, K) == 0


def test_sizes_match_layouts():
    s = S(4096, 1408, 64, 6, 64, "bf16")
    # packed weights are a byte permutation of the canonical tensors
    assert lib.moe_packed_weight_bytes(s) == 64 * 3 * 4096 * 1408 * 2
    s = S(7168, 2048, 256, 8, 8192, "mxfp8")
    canon = 256 * 3 * 7168 * 2048
    # MXFP8 layers also hold W2's codes in the fp8 instruction's fragment order
    assert lib.moe_packed_weight_bytes(s) == canon + canon // 32 + 256 * 7168 * 2048
    # bf16 activations over MXFP8 weights: no fragment copy
    assert lib.moe_packed_weight_bytes(S(7168, 2048, 256, 8, 8192, "bf16_mxfp8")) == canon + canon // 32
    s = S(7168, 2048, 384, 8, 128, "nvfp4")
    canon = 384 * 3 * 7168 * 2048
    assert lib.moe_packed_weight_bytes(s) == canon // 2 + canon // 16 + 2 * 1536  # + alpha regions (256-aligned)
    T = 37
    s = S(512, 256, 8, 4, 64, "mxfp8")
    assert lib.moe_xq_scale_offset(s, T) == ((T * 512 + 255) // 256) * 256
    dq = lib.moe_xq_scale_offset(s, T) + ((T * 16 + 255) // 256) * 256
    assert lib.moe_xq_dequant_offset(s, T) == dq
    assert lib.moe_xq_bytes(s, T) == dq + ((T * 512 * 2 + 255) // 256) * 256
    assert lib.moe_hq_scale_offset(s, T) == ((T * 4 * 256 + 255) // 256) * 256
    s = S(512, 256, 8, 4, 64, "nvfp4")
    assert lib.moe_xq_scale_offset(s, T) == ((T * 256 + 255) // 256) * 256
    assert lib.moe_xq_bytes(s, 65) == 0  # T beyond max_tokens
    # squared-ReLU experts: W1 holds I rows instead of 2I
    s = S(4096, 1408, 64, 6, 64, "bf16", "relu2")
    assert lib.moe_packed_weight_bytes(s) == 64 * 2 * 4096 * 1408 * 2
    s = S(7168, 2048, 256, 8, 8192, "mxfp8", "relu2")
    canon = 256 * 2 * 7168 * 2048
    assert lib.moe_packed_weight_bytes(s) == canon + canon // 32 + 256 * 7168 * 2048
    assert lib.moe_workspace_bytes(s) == lib.moe_workspace_bytes(S(7168, 2048, 256, 8, 8192, "mxfp8"))
    # bf16 activations over MXFP8 weights: the weights of MXFP8, the activations of BF16
    for shape in [(7168, 2048, 256, 8, 8192), (512, 256, 8, 4, 64)]:
        a, m, b = S(*shape, "bf16_mxfp8"), S(*shape, "mxfp8"), S(*shape, "bf16")
        # (the MXFP8 layer adds W2's fp8 fragment copy)
        assert lib.moe_packed_weight_bytes(a) == lib.moe_packed_weight_bytes(m) - shape[2] * shape[0] * shape[1]
        for f in (lib.moe_xq_bytes, lib.moe_xq_scale_offset, lib.moe_hq_bytes, lib.moe_hq_scale_offset):
            assert f(a, T) == f(b, T), f
        assert lib.moe_workspace_bytes(a) == lib.moe_workspace_bytes(b)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_invalid_arguments_rejected_on_host():
    s = S()
    bad = S(H=200)
    st = lib.load()
    P = ctypes.c_void_p
    # unsupported shape
    assert st.moe_route(ctypes.byref(bad), 4, P(FAKE), P(FAKE), P(FAKE), None) == UNSUPPORTED
    # T out of range
    assert st.moe_route(ctypes.byref(s), 17, P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    assert st.moe_route(ctypes.byref(s), -1, P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    # null pointers
    assert st.moe_route(ctypes.byref(s), 4, None, P(FAKE), P(FAKE), None) == INVALID
    assert st.moe_permute(ctypes.byref(s), 4, P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 0, None) == INVALID
    assert st.moe_gemm13_swiglu_quant(ctypes.byref(s), 4, None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 0, None) == INVALID
    assert st.moe_gemm2(ctypes.byref(s), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, 0, None) == INVALID
    assert st.moe_combine(ctypes.byref(s), 4, P(FAKE), None, P(FAKE), None) == INVALID
    # workspace / packed too small
    ws = lib.moe_workspace_bytes(s)
    assert st.moe_forward(ctypes.byref(s), 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), ws - 1,
                          None) == WORKSPACE
    pb = lib.moe_packed_weight_bytes(s)
    assert st.moe_prepare_weights(ctypes.byref(s), P(FAKE), None, None, P(FAKE), None, None, P(FAKE), pb - 1,
                                  None) == WORKSPACE
    # quantised formats need scales (and alpha for NVFP4)
    s8 = S(dt="mxfp8")
    assert st.moe_prepare_weights(ctypes.byref(s8), P(FAKE), None, None, P(FAKE), P(FAKE), None, P(FAKE), 1 << 40,
                                  None) == INVALID
    s4 = S(dt="nvfp4")
    assert st.moe_prepare_weights(ctypes.byref(s4), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                  1 << 40, None) == INVALID
    assert st.moe_quantize_weights(1, 1, 4, 48, P(FAKE), P(FAKE), P(FAKE), None, None) == UNSUPPORTED  # K % 32
    # NVFP4 global-scale fold
    assert st.moe_nvfp4_fold_global_scale(2, 4, 40, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == UNSUPPORTED  # K % 16
    assert st.moe_nvfp4_fold_global_scale(2, 4, 64, P(FAKE), None, P(FAKE), P(FAKE), None) == INVALID
    assert st.moe_nvfp4_fold_global_scale(-1, 4, 64, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == INVALID
    assert st.moe_nvfp4_fold_global_scale(0, 4, 64, None, None, None, None, None) == OK  # nothing to do
    assert st.moe_quantize_weights(2, 1, 4, 64, P(FAKE), P(FAKE), P(FAKE), None, None) == INVALID  # no alpha
    assert st.moe_quantize_weights(7, 1, 4, 64, P(FAKE), P(FAKE), P(FAKE), None, None) == UNSUPPORTED
    # T == 0 is a no-op that succeeds without touching anything
    assert st.moe_forward(ctypes.byref(s), 0, None, None, None, None, None, None, None, 0, None) == OK
    assert st.moe_quantize_weights(0, 0, 4, 64, None, None, None, None, None) == OK


def test_status_strings():
    assert lib.status_string(0) == "ok"
    assert "workspace" in lib.status_string(-3)
    with pytest.raises(lib.MoeError):
        lib._check(-2, "x")
