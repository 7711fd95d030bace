"""Pins of the oracle's gate/up clamp (reading: with limit L > 0 the SwiGLU
gate is min(g, L) and the up value clamp(u, -L, L), applied before the
activation; L = 0 means none -- the pages name a resolve_gate_up_clamp step
[MegaMoE drop workflow, §2, the adaptation layer's comm.py] and give no rule):
hand-derived closed-form values (tests/golden/swiglu_clamp_cases.txt), the
E=1 top-1 layer against a dense clamped SwiGLU MLP written with
torch.nn.functional, a limit above every pre-activation leaving the layer
bitwise unchanged, and the output bound |h| <= L * max(silu(L), 0.2785)."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_inputs as mi
from oracle import codecs, moe, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swiglu_clamp_cases.txt")


def _cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                g, u, L, h, _ = [p.strip() for p in line.split("|")]
                out.append((float(g), float(u), float(L), float(h)))
    return out


def test_golden_clamped_swiglu():
    cases = _cases()
    assert len(cases) >= 8
    for g, u, L, h in cases:
        got = float(moe.silu_mul(np.array([g]), np.array([u]), L)[0])
        assert got == pytest.approx(h, rel=1e-12, abs=1e-300), (g, u, L)


def _weights(w, limit):
    w13, w2 = mi.host_all_master_weights(w)
    return moe.quantize_weights({e: w13[e] for e in range(w.E)}, {e: w2[e] for e in range(w.E)}, w.dtype,
                                limit=limit)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4", "bf16_mxfp8"])
def test_e1_clamped_layer_is_dense_clamped_mlp(dtype):
    # H = 256: gate/up pre-activations have std ~0.02 * 16 = 0.32; L = 0.25 clamps many
    w = mi.Workload(f"clamp_{dtype}", 7, 256, 64, 1, 1, dtype, "none", 95)
    L = 0.25
    W = _weights(w, L)
    x, l = mi.host_x(w), mi.host_logits(w)
    r = moe.moe_layer(x, l, W, 1)
    _, _, xh = moe.quantize_x(x, dtype)
    W13, W2 = W.dequant(0)
    xt = torch.from_numpy(xh)
    g = F.linear(xt, torch.from_numpy(W13[:64]))
    u = F.linear(xt, torch.from_numpy(W13[64:]))
    assert (g > L).any() and (u.abs() > L).any()  # the clamp is exercised
    h = (F.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L)).numpy()
    act = "bf16" if dtype == "bf16_mxfp8" else dtype
    c, s = quant.quantize_act(h.astype(np.float32), act)
    ref = F.linear(torch.from_numpy(quant.dequantize_act(c, s, act)), torch.from_numpy(W2)).numpy()
    assert np.allclose(r.out_f64, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r.out, codecs.bf16_encode(ref.astype(np.float32)))


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4"])
def test_limit_above_every_preactivation_changes_nothing(dtype):
    w = mi.Workload(f"clamp_big_{dtype}", 6, 64, 64, 5, 2, dtype, "none", 96)
    x, l = mi.host_x(w), mi.host_logits(w)
    a = moe.moe_layer(x, l, _weights(w, 0.0), w.k)
    b = moe.moe_layer(x, l, _weights(w, 1e6), w.k)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.out_f64, b.out_f64)
    c = moe.moe_layer(x, l, _weights(w, 0.05), w.k)
    assert not np.array_equal(a.out, c.out)


def test_clamped_output_bound():
    rng = np.random.default_rng(4)
    g, u = rng.standard_normal(100000) * 5, rng.standard_normal(100000) * 5
    for L in (0.1, 1.0, 3.0):
        h = moe.silu_mul(g, u, L)
        silu_L = L / (1 + np.exp(-L))
        assert np.max(np.abs(h)) <= L * max(silu_L, 0.2785) * (1 + 1e-12)
        # the bound is reached: silu(min(g, L)) spans [-0.2785, silu(L)] and |clamp(u)| reaches L
        assert np.isclose(np.max(np.abs(h)), L * max(silu_L, 0.2785), rtol=1e-3)
