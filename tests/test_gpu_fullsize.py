"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Inputs come from the seeded device generators; the library
quantises all experts' fp32 master weights on the GPU.  The oracle checks:

* routing (all tokens), the permutation (all pairs): bit-exact;
* quantised activations: bit-exact on a sample of token rows;
* for a few sampled tokens: the oracle quantises the fp32 masters of their
  experts itself (codes must equal the library's bit for bit) and evaluates
  the layer for those tokens; intermediate, expert outputs and the layer
  output must meet the tolerance;
* moe_forward equals the staged entry points bit for bit on every token.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os
import time

import numpy as np
import pytest
import torch

import gpu_harness as gh
import mixture_experts_layer_sort_amd as lib
import moe_inputs as mi
from oracle import moe as omoe
from oracle import quant as oquant

pytestmark = pytest.mark.gpu

W = mi.WORKLOADS
MAX_SAMPLE_EXPERTS = 16
# knob settings (gemm, down_fp8, band_rows, fc2_reduce) checked at full size
KNOB_CASES = {"mxfp8_prefill": [(3, 0, 0, 0), (0, 1, 0, 1), (0, 1, 256, 0), (0, 1, 4096, 0), (0, 1, 0, 0, 0, 1),
                                (0, 1, 0, 0, 0, 2), (0, 1, 0, 0, 0, 3)],
              "mxfp8_decode": [(3, 0, 512, 0), (2, 1, 0, 0), (0, 1, 0, 1)]}


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.fixture(scope="module")
def pool():
    n = min(16, os.cpu_count() or 4)
    with cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        yield ex


def _quantize_pair(args):
    w13, w2, dtype, fold = args
    out = []
    for m in (w13, w2):
        c, s, a = oquant.quantize_weight(m, gh.weight_format(dtype))
        if fold:
            s, a = oquant.nvfp4_fold_global_scale(s, a)
        out.append((c, s, a))
    return tuple(out)


def _pick_tokens(ids, k, limit):
    """The first tokens (in a seeded order) whose experts stay within `limit`."""
    order = np.random.default_rng(1234).permutation(ids.shape[0])
    toks, experts = [], set()
    for t in order:
        nxt = experts | set(ids[t].tolist())
        if toks and len(nxt) > limit:
            continue
        toks.append(int(t))
        experts = nxt
        if len(toks) >= 4:
            break
    return sorted(toks), sorted(experts)


def _sorted_positions(off, n_hot=4, item_rows=(128, 256)):
    """Sorted rows of the `n_hot` experts with the most routed rows: the first
    row, the rows on both sides of every 128- and 256-row item boundary among
    the first three, a middle row, the first row of the last (ragged) item and
    the last row.  Returns {expert: sorted row positions}."""
    counts = np.diff(off)
    hot = [int(e) for e in np.argsort(-counts, kind="stable")[:n_hot] if counts[e] > 0]
    out = {}
    for e in hot:
        lo, hi = int(off[e]), int(off[e + 1])
        c = hi - lo
        pos = {lo, lo + c // 2, hi - 1}
        for m in item_rows:
            for b in (1, 2, 3):
                if b * m < c:
                    pos.update({lo + b * m - 1, lo + b * m})
            pos.add(lo + ((c - 1) // m) * m)  # first row of the last item
        out[e] = sorted(p for p in pos if lo <= p < hi)
    return out


@pytest.mark.parametrize("name", ["tiny_bf16", "bf16_decode", "mxfp8_decode", "nvfp4_decode_t8",
                                  "nvfp4_decode_t128", "bf16_mxfp8_decode", "relu2_nvfp4_decode_t128",
                                  "nvfp4_folded_decode_t128", "clamp_mxfp8_decode",
                                  "mxfp8_prefill"])
def test_fullsize_parity(name, pool):
    w = W[name]
    dev = gh.dev()
    _log(f"{name}: building {w}")
    cw = gh.alloc_canonical(w)
    for e in range(w.E):
        a, b = mi.device_master_weights(w, e, dev)
        gh.quantize_expert(w, cw, e, a, b)
    layer = gh.DeviceLayer(w, cw)
    x = mi.device_x(w, dev)
    logits = mi.device_logits(w, dev)
    r = layer.staged(x, logits)
    out_fwd = layer.forward(x, logits)
    out_fused = layer.forward_fused(x, logits)
    torch.cuda.synchronize()
    assert not layer.sync_words().any()
    _log(f"{name}: GPU done")

    x_bits = gh.bf16_numpy(x)
    l_host = logits.cpu().numpy()
    # routing and permutation of every token / pair
    rid, rw = omoe.route(l_host, w.k)
    ids = r["ids"].cpu().numpy()
    assert np.array_equal(ids, rid)
    assert np.max(np.abs(r["wts"].cpu().numpy() - rw)) <= 1e-6
    off, sp, pp = omoe.permute(rid, w.E)
    assert np.array_equal(r["offsets"].cpu().numpy(), off)
    assert np.array_equal(r["sorted_pairs"].cpu().numpy()[: w.P], sp)
    assert np.array_equal(r["pair_pos"].cpu().numpy()[: w.P], pp)
    _log(f"{name}: routing + permutation bit-exact; active experts {int(np.sum(np.diff(off) > 0))}")
    # quantised activations on a sample of rows
    rows = np.unique(np.random.default_rng(7).integers(0, w.T, min(w.T, 64)))
    xc, xs, _ = omoe.quantize_x(x_bits[rows], w.dtype)
    gc, gs = layer.xq_numpy(r, w.T)
    assert np.array_equal(gc[rows], xc)
    if xs is not None:
        assert np.array_equal(gs[rows], xs)
    # both whole-layer entries == the staged entry points on every token
    assert np.array_equal(gh.bf16_numpy(out_fwd), gh.bf16_numpy(r["out"]))
    assert np.array_equal(gh.bf16_numpy(out_fused), gh.bf16_numpy(r["out"]))

    # sampled tokens against the oracle, with the oracle's own weight quantisation
    toks, experts = _pick_tokens(ids, w.k, MAX_SAMPLE_EXPERTS)
    _log(f"{name}: oracle on tokens {toks} ({len(experts)} experts)")
    masters = {}
    for e in experts:
        a, b = mi.device_master_weights(w, e, dev)
        masters[e] = (a.cpu().numpy(), b.cpu().numpy())
    results = list(pool.map(_quantize_pair, [(masters[e][0], masters[e][1], w.dtype, w.fold) for e in experts]))
    del masters
    got = gh.canonical_to_numpy(cw, experts)
    ow = {n: {} for n in ("w13", "w13_s", "w13_a", "w2", "w2_s", "w2_a")}
    for e, ((c13, s13, a13), (c2, s2, a2)) in zip(experts, results):
        ow["w13"][e], ow["w13_s"][e], ow["w13_a"][e] = c13, s13, a13
        ow["w2"][e], ow["w2_s"][e], ow["w2_a"][e] = c2, s2, a2
        assert np.array_equal(np.asarray(got["w13"][e]), c13), e
        assert np.array_equal(np.asarray(got["w2"][e]), c2), e
        if s13 is not None:
            assert np.array_equal(got["w13_s"][e], s13) and np.array_equal(got["w2_s"][e], s2), e
        if a13 is not None:
            assert float(got["w13_a"][e]) == float(a13) and float(got["w2_a"][e]) == float(a2), e
    _log(f"{name}: library weight codes of {len(experts)} experts equal the oracle's")
    if w.dtype == "bf16":
        Wo = omoe.Weights("bf16", ow["w13"], ow["w2"], act=w.act, limit=w.limit)
    elif gh.weight_format(w.dtype) == "mxfp8":
        Wo = omoe.Weights(w.dtype, ow["w13"], ow["w2"], ow["w13_s"], ow["w2_s"], act=w.act, limit=w.limit)
    else:
        Wo = omoe.Weights("nvfp4", ow["w13"], ow["w2"], ow["w13_s"], ow["w2_s"], ow["w13_a"], ow["w2_a"], act=w.act,
                          limit=w.limit)
    ref = omoe.moe_layer(x_bits, l_host, Wo, w.k, tokens=toks, keep=True)
    hc, hs = layer.hq_numpy(r, w.T)
    y = gh.bf16_numpy(r["y"])
    tol = gh.out_tolerance(w.dtype)
    for t in toks:
        for j in range(w.k):
            p = t * w.k + j
            row = int(pp[p])
            h_got = oquant.dequantize_act(hc[row:row + 1], None if hs is None else hs[row:row + 1],
                                          gh.act_format(w.dtype))[0]
            assert gh.rel_l2(h_got, ref.h[(t, j)][2]) <= tol, (t, j)
            y_got = (y[p].astype(np.uint32) << 16).view(np.float32)
            assert gh.rel_l2(y_got, ref.y[(t, j)]) <= tol, (t, j)
    rel, mad = gh.check_out(gh.bf16_numpy(r["out"])[toks], ref.out, w.dtype, name)
    _log(f"{name}: sampled tokens out relL2 {rel:.2e} max|d|/rms {mad:.2e}")

    if w.T * w.k >= 64 * w.E:
        # prefill-shaped GEMMs: rows at fixed sorted positions of the hottest
        # experts (item boundaries, the ragged last item), intermediate and y
        # per routed pair against the oracle's expert MLP
        sample = _sorted_positions(off)
        hot = sorted(sample)
        _log(f"{name}: sorted-position sample of experts {hot}: {sum(len(v) for v in sample.values())} rows")
        res = list(pool.map(_quantize_pair, [(*[m.cpu().numpy() for m in mi.device_master_weights(w, e, dev)],
                                              w.dtype, w.fold) for e in hot]))
        Wh = omoe.Weights(w.dtype, {e: r_[0][0] for e, r_ in zip(hot, res)}, {e: r_[1][0] for e, r_ in zip(hot, res)},
                          {e: r_[0][1] for e, r_ in zip(hot, res)}, {e: r_[1][1] for e, r_ in zip(hot, res)},
                          {e: r_[0][2] for e, r_ in zip(hot, res)}, {e: r_[1][2] for e, r_ in zip(hot, res)}, act=w.act,
                          limit=w.limit)
        worst = 0.0
        for e in hot:
            w13d, w2d = Wh.dequant(e)
            for row in sample[e]:
                p = int(sp[row])
                _, _, xh = omoe.quantize_x(x_bits[p // w.k: p // w.k + 1], w.dtype)
                (_, _, h_ref), y_ref = omoe.expert_mlp(xh[0], w13d, w2d, w.act, w.dtype, w.limit)
                h_got = oquant.dequantize_act(hc[row:row + 1], None if hs is None else hs[row:row + 1],
                                              gh.act_format(w.dtype))[0]
                y_got = (y[p].astype(np.uint32) << 16).view(np.float32)
                rh, ry = gh.rel_l2(h_got, h_ref), gh.rel_l2(y_got, y_ref)
                assert rh <= tol and ry <= tol, (e, row, rh, ry)
                worst = max(worst, rh, ry)
        _log(f"{name}: sorted-position rows within tolerance (worst relL2 {worst:.2e})")

    if name in KNOB_CASES:
        # knob settings at full size: every token's output against the default
        # path's (tolerance), the sampled tokens against the oracle; a band
        # change alone leaves the bits unchanged
        base = gh.bf16_numpy(r["out"])
        for kn in KNOB_CASES[name]:
            got = gh.bf16_numpy(layer.forward_knobs(x, logits, lib.make_knobs(*kn)))
            torch.cuda.synchronize()
            rel, mad = gh.check_out(got[toks], ref.out, w.dtype, f"{name} knobs {kn}")
            if kn[3] == 0 and kn[1] == 1 and kn[0] == 0:  # performance knobs only (band, item deal)
                assert np.array_equal(got, base), kn
            d = gh.rel_l2((got.astype(np.uint32) << 16).view(np.float32),
                          (base.astype(np.uint32) << 16).view(np.float32))
            assert d <= gh.out_tolerance(w.dtype), (kn, d)
            _log(f"{name}: knobs {kn}: sampled out relL2 {rel:.2e} max|d|/rms {mad:.2e}; all tokens vs default {d:.2e}")
    del layer, cw, r, out_fwd, out_fused
    torch.cuda.empty_cache()
