"""Pins of the oracle's layer: a dense masked fp64 brute force built from
torch.nn.functional, the E=1 top-1 case against a dense SwiGLU MLP, expert
relabelling invariance, agreement of the per-token and expert-grouped forms,
and fp32 vs fp64 accumulation headroom."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import moe_inputs as mi
from oracle import codecs, moe, quant

DTYPES = ["bf16", "mxfp8", "nvfp4", "bf16_mxfp8"]


def _act(dtype):
    """Activation format of a layer format (bf16_mxfp8: bf16 activations)."""
    return "bf16" if dtype == "bf16_mxfp8" else dtype


def _small(dtype, T=6, H=64, I=64, E=5, k=2, bias="none", cid=91, act="swiglu"):
    return mi.Workload(f"small_{dtype}_{act}", T, H, I, E, k, dtype, bias, cid, act)


def _weights(w):
    w13, w2 = mi.host_all_master_weights(w)
    return moe.quantize_weights({e: w13[e] for e in range(w.E)}, {e: w2[e] for e in range(w.E)}, w.dtype, w.act)


def _mlp_torch(x_hat, W13, W2, dtype, act="swiglu"):
    """Dense expert MLP written with torch.nn.functional in fp64 -- SwiGLU
    (gate rows, then up rows) or squared ReLU of W1 -- with the layer's
    requantisation of the intermediate (the quantiser is pinned in
    test_oracle_quant)."""
    xt = torch.from_numpy(x_hat)
    if act == "relu2":
        h = (F.relu(F.linear(xt, torch.from_numpy(W13))) ** 2).numpy()
    else:
        I = W13.shape[0] // 2
        g = F.linear(xt, torch.from_numpy(W13[:I]))
        u = F.linear(xt, torch.from_numpy(W13[I:]))
        h = (F.silu(g) * u).numpy()
    c, s = quant.quantize_act(h.astype(np.float32), _act(dtype))
    hh = quant.dequantize_act(c, s, _act(dtype))
    return F.linear(torch.from_numpy(hh), torch.from_numpy(W2)).numpy()


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_e1_top1_is_dense_mlp(dtype, act):
    w = _small(dtype, T=9, E=1, k=1, act=act)
    W = _weights(w)
    assert W.dequant(0)[0].shape == (w.R13, w.H)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    r = moe.moe_layer(x, l, W, 1)
    xc, xs, xh = moe.quantize_x(x, dtype)
    W13, W2 = W.dequant(0)
    ref = _mlp_torch(xh, W13, W2, dtype, act)
    assert np.allclose(r.out_f64, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r.out, codecs.bf16_encode(ref.astype(np.float32)))


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_dense_masked_brute_force(dtype, act):
    """out_t = sum_e G[t, e] * MLP_e(x_hat_t) with G the renormalised top-k
    gate matrix built from scipy's full softmax."""
    w = _small(dtype, T=7, E=6, k=3, act=act)
    W = _weights(w)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    r = moe.moe_layer(x, l, W, w.k)
    p = scipy.special.softmax(l.astype(np.float64), axis=1)
    thr = np.sort(l, axis=1)[:, -w.k][:, None]
    mask = l >= thr  # no ties in random fp32 logits
    G = np.where(mask, p, 0.0)
    G /= G.sum(axis=1, keepdims=True)
    _, _, xh = moe.quantize_x(x, dtype)
    ref = np.zeros((w.T, w.H))
    for e in range(w.E):
        W13, W2 = W.dequant(e)
        ref += G[:, e:e + 1] * _mlp_torch(xh, W13, W2, dtype, act)
    assert np.allclose(r.out_f64, ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("dtype,act", [(d, "swiglu") for d in DTYPES] + [("mxfp8", "relu2"), ("nvfp4", "relu2")])
def test_relabelling_invariance(dtype, act):
    w = _small(dtype, T=8, E=7, k=3, act=act)
    W = _weights(w)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    base = moe.moe_layer(x, l, W, w.k)
    pi = np.random.default_rng(3).permutation(w.E)  # new id of old expert e is pi[e]
    inv = np.argsort(pi)
    def perm(a):
        return None if a is None else {pi[e]: a[e] for e in range(w.E)}
    Wp = moe.Weights(dtype, perm(W.w13), perm(W.w2), perm(W.w13_s), perm(W.w2_s), perm(W.w13_a), perm(W.w2_a),
                     act=W.act)
    lp = l[:, inv]  # column pi[e] holds old column e
    got = moe.moe_layer(x, lp, Wp, w.k)
    assert np.array_equal(got.out, base.out)
    assert np.array_equal(got.out_f64, base.out_f64)
    assert np.array_equal(got.ids, pi[base.ids])


@pytest.mark.parametrize("dtype,act", [(d, "swiglu") for d in DTYPES] + [("bf16", "relu2"), ("nvfp4", "relu2")])
def test_loop_and_grouped_forms_agree(dtype, act):
    w = _small(dtype, T=20, H=128, I=96, E=8, k=3, bias="normal2", act=act)
    W = _weights(w)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    a = moe.moe_layer(x, l, W, w.k)
    b = moe.moe_layer_grouped(x, l, W, w.k)
    assert np.allclose(a.out_f64, b.out_f64, rtol=1e-9, atol=1e-12)
    # bf16 output: equal except possibly at an fp64-rounding tie
    assert np.mean(a.out != b.out) < 1e-3


@pytest.mark.parametrize("dtype", DTYPES)
def test_fp32_accumulation_headroom(dtype):
    w = _small(dtype, T=16, H=256, I=128, E=8, k=2)
    W = _weights(w)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    a = moe.moe_layer_grouped(x, l, W, w.k)
    b = moe.moe_layer_grouped(x, l, W, w.k, acc_dtype=np.float32)
    ref = codecs.bf16_decode(a.out)
    got = codecs.bf16_decode(b.out)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    tol = 3e-2 if dtype == "nvfp4" else 1e-2
    assert rel < tol / 5, rel


def test_bf16_mxfp8_is_the_bf16_layer_on_widened_mxfp8_weights():
    """Reading of the bf16 x MXFP8 format: MXFP8 weights, the BF16 layer's
    activation path.  e4m3 x 2^s is exact in bf16, so the layer must equal,
    bit for bit, the BF16 layer run on the MXFP8 weights widened to bf16 --
    and differ from the MXFP8 layer, which quantises x and h."""
    w = _small("bf16_mxfp8", T=10, E=6, k=3, bias="normal2")
    W = _weights(w)
    assert W.w13[0].dtype == np.uint8 and W.w13_s is not None  # stored as MXFP8
    wide13, wide2 = {}, {}
    for e in range(w.E):
        a, b = W.dequant(e)
        wide13[e] = codecs.bf16_encode(a.astype(np.float32))
        wide2[e] = codecs.bf16_encode(b.astype(np.float32))
        assert np.array_equal(codecs.bf16_decode(wide13[e]), a)  # exact widening
        assert np.array_equal(codecs.bf16_decode(wide2[e]), b)
    x, l = mi.host_x(w), mi.host_logits(w)
    got = moe.moe_layer(x, l, W, w.k)
    ref = moe.moe_layer(x, l, moe.Weights("bf16", wide13, wide2), w.k)
    assert np.array_equal(got.out_f64, ref.out_f64)
    assert np.array_equal(got.out, ref.out)
    mx = moe.moe_layer(x, l, moe.Weights("mxfp8", W.w13, W.w2, W.w13_s, W.w2_s), w.k)
    assert not np.array_equal(mx.out_f64, got.out_f64)


def test_token_subset_matches_full():
    w = _small("mxfp8", T=12, E=4, k=2)
    W = _weights(w)
    x = mi.host_x(w)
    l = mi.host_logits(w)
    full = moe.moe_layer(x, l, W, 2)
    sub = moe.moe_layer(x, l, W, 2, tokens=[7, 2, 11])
    assert np.array_equal(sub.out, full.out[[7, 2, 11]])


def test_inputs_are_deterministic():
    w = mi.WORKLOADS["tiny_bf16"]
    assert np.array_equal(mi.host_x(w), mi.host_x(w))
    assert np.array_equal(mi.host_logits(w), mi.host_logits(w))
    a, b = mi.host_master_weights(w, 3)
    c, d = mi.host_master_weights(w, 3)
    assert np.array_equal(a, c) and np.array_equal(b, d)
    assert abs(float(np.std(a)) - 0.02) < 1e-3
    z = mi.expert_bias(mi.WORKLOADS["mxfp8_prefill"])
    assert np.isclose(np.exp(z.astype(np.float64)).sum(), 1.0, rtol=1e-5)
