"""Pins of the oracle's batched-experts form (tokens bucketed per expert, no
routing or combine): dispatching a routed layer's (token, slot) pairs into
the batched format, running batched_experts and combining its rows with the
router weights in slot order reproduces the routed layer (pinned in
test_oracle_layer) bit for bit; empty experts, counts above the capacity and
rows past the counts are handled as stated."""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe


def _weights(w):
    w13, w2 = mi.host_all_master_weights(w)
    return moe.quantize_weights({e: w13[e] for e in range(w.E)}, {e: w2[e] for e in range(w.E)}, w.dtype, w.act,
                                limit=w.limit)


@pytest.mark.parametrize("dtype,act,limit", [("bf16", "swiglu", 0.0), ("mxfp8", "swiglu", 0.0),
                                             ("nvfp4", "swiglu", 0.0), ("bf16_mxfp8", "swiglu", 0.0),
                                             ("mxfp8", "relu2", 0.0), ("nvfp4", "swiglu", 0.2)])
def test_dispatch_batched_combine_equals_routed_layer(dtype, act, limit):
    w = mi.Workload(f"batched_{dtype}", 9, 64, 64, 5, 2, dtype, "none", 97, act, False, limit)
    W = _weights(w)
    x, l = mi.host_x(w), mi.host_logits(w)
    ref = moe.moe_layer(x, l, W, w.k)
    ids, wts = moe.route(l, w.k)
    M = 7
    xb = np.zeros((w.E, M, w.H), np.uint16)
    counts = np.zeros(w.E, np.int64)
    where = {}
    for t in range(w.T):
        for j in range(w.k):
            e = int(ids[t, j])
            where[(t, j)] = (e, int(counts[e]))
            xb[e, counts[e]] = x[t]
            counts[e] += 1
    assert counts.max() <= M
    y = moe.batched_experts(xb, counts, W)
    out = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            e, r = where[(t, j)]
            out[t] += wts[t, j] * y[e, r]
    assert np.array_equal(out, ref.out_f64)
    # rows past each expert's count stay zero
    for e in range(w.E):
        assert not y[e, counts[e]:].any()


def test_counts_clamped_and_empty_experts():
    w = mi.Workload("batched_edges", 1, 64, 64, 3, 1, "bf16", "none", 98)
    W = _weights(w)
    rng = np.random.default_rng(2)
    xb = mi.f32_to_bf16_bits(rng.standard_normal((3, 4, 64)).astype(np.float32))
    y_all = moe.batched_experts(xb, [4, 4, 4], W)
    y = moe.batched_experts(xb, [0, 9, -3], W)  # empty, above capacity (-> 4), negative (-> 0)
    assert not y[0].any() and not y[2].any()
    assert np.array_equal(y[1], y_all[1])
    assert y_all[0].any() and y_all[2].any()
