"""Parity of the HIP library with the CPU oracle at sizes the oracle finishes
in seconds (several tiles, ragged tails, edge cases).  Bit-exact: routing ids,
permutation, quantised activations and quantised weights.  Tolerance: router
weights 1e-6 absolute; layer output relative L2 <= 1e-2 (bf16, MXFP8) or
3e-2 (NVFP4) and max |diff| <= 5e-2 * RMS."""
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
SMALL = {
    "tiny_bf16": W["tiny_bf16"],
    "bf16_ragged": W["bf16_decode"].scaled(T=33, H=512, I=384, E=16),
    "mxfp8_decode_small": W["mxfp8_decode"].scaled(T=40, H=640, I=256, E=32),
    "nvfp4_decode_small": W["nvfp4_decode_t8"].scaled(T=13, H=512, I=256, E=48),
    # decode-shaped GEMMs whose experts get 17-32 routed rows (items run as
    # two wave pairs; mxfp8_decode_small and bf16_ragged also have them, and
    # experts above 32 rows)
    "nvfp4_decode_paired": W["nvfp4_decode_t8"].scaled(T=60, H=512, I=256, E=16, k=4),
    "mxfp8_prefill_small": W["mxfp8_prefill"].scaled(T=300, H=512, I=256, E=16, k=4),
    "nvfp4_prefill_small": W["nvfp4_decode_t128"].scaled(T=96, H=384, I=128, E=8, k=3),
    "bf16_prefill_small": W["bf16_decode"].scaled(T=150, H=256, I=256, E=6, k=2),
    # >= 64 routed rows per expert on average: the LDS-staged prefill GEMM
    # (128-row m-tiles with ragged tails, several n-tiles and K steps)
    "bf16_prefill_tiles": W["bf16_decode"].scaled(T=300, H=384, I=256, E=4, k=2),
    "nvfp4_prefill_tiles": W["nvfp4_decode_t128"].scaled(T=200, H=384, I=128, E=4, k=2),
    "mxfp8_prefill_skewed": W["mxfp8_prefill"].scaled(T=520, H=256, I=384, E=8, k=2),
    "bf16_singleton": W["tiny_bf16"].scaled(E=1, k=1, T=5),
    "mxfp8_singleton": W["mxfp8_decode"].scaled(E=1, k=1, T=7, H=256, I=128),
    "nvfp4_singleton": W["nvfp4_decode_t8"].scaled(E=1, k=1, T=3, H=256, I=128),
    "bf16_k_equals_E": W["tiny_bf16"].scaled(E=4, k=4, T=9, H=128, I=128),
    "mxfp8_min": W["mxfp8_decode"].scaled(T=1, H=128, I=128, E=3, k=2),
    # bf16 activations over MXFP8 weights: decode and prefill-shaped GEMMs
    "bf16_mxfp8_decode_small": W["bf16_mxfp8_decode"].scaled(T=40, H=640, I=256, E=32),
    "bf16_mxfp8_prefill_small": W["bf16_mxfp8_prefill"].scaled(T=520, H=256, I=384, E=8, k=2),
    # non-gated squared-ReLU experts, every format, decode- and prefill-shaped GEMMs
    "relu2_bf16_small": W["bf16_decode"].scaled(T=33, H=512, I=384, E=16, act="relu2"),
    "relu2_mxfp8_decode_small": W["mxfp8_decode"].scaled(T=40, H=640, I=256, E=32, act="relu2"),
    "relu2_nvfp4_decode_small": W["nvfp4_decode_t8"].scaled(T=13, H=512, I=256, E=48, act="relu2"),
    "relu2_mxfp8_prefill_skewed": W["mxfp8_prefill"].scaled(T=520, H=256, I=384, E=8, k=2, act="relu2"),
    "relu2_nvfp4_prefill_tiles": W["nvfp4_decode_t128"].scaled(T=200, H=384, I=256, E=4, k=2, act="relu2"),
    "relu2_bf16_mxfp8_prefill": W["bf16_mxfp8_prefill"].scaled(T=300, H=256, I=256, E=4, k=2, act="relu2"),
    # 16 E < T k < 64 E: decode-shaped GEMMs with 32-row token tiles (two
    # 16-wide sub-tiles per wave), every format and both activations
    "mxfp8_nt2": W["mxfp8_decode"].scaled(T=96, H=512, I=256, E=8, k=3),
    "bf16_mxfp8_nt2": W["bf16_mxfp8_decode"].scaled(T=96, H=512, I=256, E=8, k=3),
    "bf16_nt2": W["bf16_decode"].scaled(T=96, H=512, I=256, E=8, k=3),
    "nvfp4_nt2": W["nvfp4_decode_t8"].scaled(T=96, H=512, I=256, E=8, k=3),
    "relu2_bf16_nt2": W["bf16_decode"].scaled(T=96, H=512, I=256, E=8, k=3, act="relu2"),
    "relu2_mxfp8_nt2": W["mxfp8_decode"].scaled(T=96, H=512, I=256, E=8, k=3, act="relu2"),
    "relu2_nvfp4_nt2": W["nvfp4_decode_t8"].scaled(T=96, H=512, I=256, E=8, k=3, act="relu2"),
    "relu2_bf16_mxfp8_nt2": W["bf16_mxfp8_decode"].scaled(T=96, H=512, I=256, E=8, k=3, act="relu2"),
    # squared-ReLU experts of bf16 weights on the prefill-shaped GEMM
    "relu2_bf16_prefill_tiles": W["bf16_decode"].scaled(T=300, H=384, I=256, E=4, k=2, act="relu2"),
    # SwiGLU experts with a gate/up clamp (pre-activations have std ~0.02 sqrt(H),
    # ~0.45 at H = 512: limits of 0.3 - 0.5 clamp a large share), every format
    # and GEMM shape
    "clamp_bf16_decode": W["bf16_decode"].scaled(T=33, H=512, I=384, E=16, limit=0.4),
    "clamp_mxfp8_decode": W["mxfp8_decode"].scaled(T=40, H=640, I=256, E=32, limit=0.5),
    "clamp_nvfp4_nt2": W["nvfp4_decode_t8"].scaled(T=96, H=512, I=256, E=8, k=3, limit=0.3),
    "clamp_mxfp8_prefill": W["mxfp8_prefill"].scaled(T=300, H=512, I=256, E=16, k=4, limit=0.4),
    "clamp_nvfp4_prefill": W["nvfp4_decode_t128"].scaled(T=200, H=384, I=128, E=4, k=2, limit=0.3),
    "clamp_bf16_mxfp8_prefill": W["bf16_mxfp8_prefill"].scaled(T=520, H=256, I=384, E=8, k=2, limit=0.25),
    # NVFP4 with the weight alpha folded into the block scales
    "nvfp4_folded_decode_small": W["nvfp4_decode_t8"].scaled(T=13, H=512, I=256, E=48, fold=True),
    "nvfp4_folded_prefill_tiles": W["nvfp4_decode_t128"].scaled(T=200, H=384, I=128, E=4, k=2, fold=True),
    # the largest expert count and top-k the library accepts
    "max_experts_topk32": W["tiny_bf16"].scaled(E=1024, k=32, T=40, H=128, I=128),
    "max_experts_topk32_nvfp4": W["nvfp4_decode_t8"].scaled(E=1024, k=32, T=24, H=128, I=128),
}


def _setup(w):
    cw, w13f, w2f = gh.canonical_from_host_master(w)
    Wo = omoe.quantize_weights({e: w13f[e] for e in range(w.E)}, {e: w2f[e] for e in range(w.E)}, w.dtype, w.act,
                               w.fold, w.limit)
    return cw, Wo


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_parity_small(name):
    w = SMALL[name]
    print(f"case {name}: {w}", flush=True)
    _check_layer(w, name, mi.host_x(w), mi.host_logits(w))


def _decode_boundary_logits(w, counts, seed):
    """Logits that route exactly counts[e] of the T*2 (token, slot) pairs to
    expert e: token t picks first[t] and second[t] (always distinct)."""
    picks = [e for e, c in enumerate(counts) for _ in range(c)]
    assert len(picks) == 2 * w.T and w.k == 2
    first, second = picks[: w.T], picks[w.T:]
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((w.T, w.E)) - 10.0).astype(np.float32)
    for t in range(w.T):
        assert first[t] != second[t]
        logits[t, first[t]] = np.float32(5.0 + rng.uniform(-0.1, 0.1))
        logits[t, second[t]] = np.float32(4.0 + rng.uniform(-0.1, 0.1))
    return logits


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4"])
def test_decode_item_boundaries(dtype):
    """Decode-shaped layer (T*k <= 16 E: one 16-wide token tile per wave)
    whose experts get exactly 16, 17, 33 and 30 routed rows: a single 16-row
    item, items of 17-32 rows run as two wave pairs, and a 32-row item
    followed by a 1-row one, all tokens against the oracle."""
    base = {"bf16": W["bf16_decode"], "mxfp8": W["mxfp8_decode"], "nvfp4": W["nvfp4_decode_t8"]}[dtype]
    w = base.scaled(T=48, H=256, I=256, E=8, k=2)
    logits = _decode_boundary_logits(w, [16, 17, 33, 30, 0, 0, 0, 0], seed=21)
    _check_layer(w, f"boundaries_{dtype}", mi.host_x(w), logits)


def _check_layer(w, name, x, logits):
    cw, Wo = _setup(w)
    # the library's weight quantiser reproduces the oracle's canonical codes bit for bit
    got = gh.canonical_to_numpy(cw)
    for n in ("w13", "w2", "w13_s", "w2_s", "w13_a", "w2_a"):
        ref = getattr(Wo, n)
        if ref is None:
            assert got[n] is None
            continue
        for e in range(w.E):
            assert np.array_equal(np.asarray(got[n][e]), np.asarray(ref[e])), (n, e)

    layer = gh.DeviceLayer(w, cw)
    xd, ld = gh.to_device_x(x), torch.from_numpy(logits).to(gh.dev())
    r = layer.staged(xd, ld)
    torch.cuda.synchronize()
    ref = omoe.moe_layer(x, logits, Wo, w.k, keep=True)

    # routing
    assert np.array_equal(r["ids"].cpu().numpy(), ref.ids)
    assert np.max(np.abs(r["wts"].cpu().numpy() - ref.weights)) <= 1e-6
    # permutation
    off, sp, pp = omoe.permute(ref.ids, w.E)
    assert np.array_equal(r["offsets"].cpu().numpy(), off)
    assert np.array_equal(r["sorted_pairs"].cpu().numpy()[: w.P], sp)
    assert np.array_equal(r["pair_pos"].cpu().numpy()[: w.P], pp)
    # quantised activations
    xc, xs, xh = omoe.quantize_x(x, w.dtype)
    gc, gs = layer.xq_numpy(r, w.T)
    assert np.array_equal(gc, xc)
    if xs is not None:
        assert np.array_equal(gs, xs)
        # the 16-bit dequantised copy the GEMM reads equals the exact values
        assert np.array_equal(layer.xq_dequant(r, w.T), xh)
    # requantised intermediate, expert-sorted: compare dequantised values
    hc, hs = layer.hq_numpy(r, w.T)
    h_got = oquant.dequantize_act(hc, hs, gh.act_format(w.dtype))
    if hs is not None:
        assert np.array_equal(layer.hq_dequant(r, w.T), h_got)
    h_ref = np.stack([ref.h[(int(p) // w.k, int(p) % w.k)][2] for p in sp])
    assert gh.rel_l2(h_got, h_ref) <= gh.out_tolerance(w.dtype)
    if hs is not None:
        # requantised codes that differ from the oracle's (accumulation order
        # moves a value across a rounding midpoint now and then)
        hc_ref = np.stack([ref.h[(int(p) // w.k, int(p) % w.k)][0] for p in sp])
        flips = float(np.mean(hc != hc_ref))
        print(f"  hq code mismatch fraction {flips:.2e}", flush=True)
        assert flips <= 5e-3, flips
    # expert outputs y (bf16, slot-major)
    y_got = gh.bf16_numpy(r["y"])[: w.P].astype(np.uint32)
    y_ref = np.stack([ref.y[(p // w.k, p % w.k)] for p in range(w.P)])
    assert gh.rel_l2((y_got << 16).view(np.float32), y_ref) <= gh.out_tolerance(w.dtype)
    # the layer output
    out_staged = gh.bf16_numpy(r["out"])
    rel, mad = gh.check_out(out_staged, ref.out, w.dtype, name)
    print(f"  out relL2 {rel:.2e}  max|d|/rms {mad:.2e}", flush=True)

    # both whole-layer entries run the same device code: bitwise equal, reproducible
    ids = torch.empty(w.T, w.k, dtype=torch.int32, device=gh.dev())
    wts = torch.empty(w.T, w.k, dtype=torch.float32, device=gh.dev())
    o1 = layer.forward(xd, ld, ids=ids, wts=wts)
    o2 = layer.forward(xd, ld)
    ids_f = torch.empty_like(ids)
    wts_f = torch.empty_like(wts)
    o3 = layer.forward_fused(xd, ld, ids=ids_f, wts=wts_f)
    o4 = layer.forward_fused(xd, ld)
    torch.cuda.synchronize()
    for o in (o1, o2, o3, o4):
        assert np.array_equal(gh.bf16_numpy(o), out_staged)
    assert torch.equal(ids, r["ids"]) and torch.equal(wts, r["wts"])
    assert torch.equal(ids_f, r["ids"]) and torch.equal(wts_f, r["wts"])
    # the single-launch kernel left its synchronisation words zero and never timed out
    assert not layer.sync_words().any()


@pytest.mark.parametrize("dtype,E,k", [("bf16", 8, 2), ("mxfp8", 64, 6), ("nvfp4", 256, 8), ("mxfp8", 384, 8),
                                        ("bf16", 1024, 32)])
def test_forward_routing_matches_staged(dtype, E, k):
    """At token counts around the routing kernel's 4-token blocks and the
    sorting block's 8-wave segments, moe_forward's routing, weights and output
    equal those of the separate moe_route / moe_permute chain bit for bit,
    and the routing equals the oracle's (ties and E up to 1024, k up to 32)."""
    base = {"bf16": W["bf16_decode"], "mxfp8": W["mxfp8_decode"], "nvfp4": W["nvfp4_decode_t8"]}[dtype]
    w = base.scaled(T=33, H=128, I=128, E=E, k=k)
    cw, _ = _setup(w)
    layer = gh.DeviceLayer(w, cw)
    x_all = mi.host_x(w)
    rng = np.random.default_rng(E * 31 + k)
    for T in (1, 7, 8, 9, 16, 17, 25, 31, 32, 33):
        l = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        l[:, : min(E, 3)] = 0.25  # exact ties, broken by the smaller id
        xd, ld = gh.to_device_x(x_all[:T]), torch.from_numpy(l).to(gh.dev())
        r = layer.staged(xd, ld)
        ids = torch.empty(T, k, dtype=torch.int32, device=gh.dev())
        wts = torch.empty(T, k, dtype=torch.float32, device=gh.dev())
        o = layer.forward(xd, ld, ids=ids, wts=wts)
        torch.cuda.synchronize()
        assert torch.equal(ids, r["ids"]) and torch.equal(wts, r["wts"]), T
        assert np.array_equal(gh.bf16_numpy(o), gh.bf16_numpy(r["out"])), T
        rid, _ = omoe.route(l, k)
        assert np.array_equal(ids.cpu().numpy(), rid), T


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 8, 2), (64, 64, 6), (33, 256, 8), (5, 384, 8), (3, 1024, 32),
                                   (200, 1000, 9), (4, 32, 32),
                                   # around the per-lane key counts (6, 12, 16 keys per lane)
                                   (9, 257, 8), (9, 320, 8), (6, 700, 8), (4, 768, 16), (4, 769, 8)])
def test_route_parity(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    l = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    # plant exact ties and signed zeros
    l[:, : min(E, 5)] = 0.5
    if E > 8:
        l[0, 6] = -0.0
        l[0, 7] = 0.0
    s = lib.make_shape(128, 128, E, k, T, "bf16")
    ids = torch.empty(T, k, dtype=torch.int32, device=gh.dev())
    wts = torch.empty(T, k, dtype=torch.float32, device=gh.dev())
    lib.moe_route(s, T, torch.from_numpy(l).to(gh.dev()), ids, wts)
    torch.cuda.synchronize()
    rid, rw = omoe.route(l, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.max(np.abs(wts.cpu().numpy() - rw)) <= 1e-6


@pytest.mark.parametrize("T,E,k,mode", [(8192, 256, 8, "zipf"), (1, 1, 1, "one"), (100, 64, 6, "all_one_expert"),
                                        (3000, 1024, 4, "uniform"), (513, 7, 7, "uniform"),
                                        # just past the one-block sort (16384 pairs): chunks of the
                                        # multi-block sort with a short last chunk
                                        (2048, 8, 8, "uniform"), (2049, 8, 8, "uniform"), (4097, 300, 4, "zipf"),
                                        (2100, 64, 8, "all_one_expert"),
                                        # the largest accepted shapes: E = 1024 with k = 32, and
                                        # max_tokens * k = 2^24 pairs through the one-block sort
                                        (32768, 1024, 32, "uniform"), (524288, 256, 32, "zipf")])
def test_permute_parity(T, E, k, mode):
    rng = np.random.default_rng(T + E)
    if mode == "all_one_expert":
        ids = np.full((T, k), E - 1, np.int32)
    elif mode == "zipf":
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        ids = rng.choice(E, (T, k), p=p / p.sum()).astype(np.int32)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    H = 128
    s = lib.make_shape(H, 128, E, k, T, "mxfp8")
    d = gh.dev()
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    sp = torch.empty(T * k, dtype=torch.int32, device=d)
    pp = torch.empty(T * k, dtype=torch.int32, device=d)
    xq = torch.empty(lib.moe_xq_bytes(s, T), dtype=torch.uint8, device=d)
    lib.moe_permute(s, T, torch.from_numpy(ids).to(d), gh.to_device_x(x), off, sp, pp, xq)
    torch.cuda.synchronize()
    ro, rs, rp = omoe.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(sp.cpu().numpy(), rs)
    assert np.array_equal(pp.cpu().numpy(), rp)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "nvfp4"])
def test_quantize_weights_edge_values(dtype):
    """Zeros, signed zeros, tiny, huge and tie values through the library's
    weight quantiser, bit-exact against the oracle's."""
    rng = np.random.default_rng(5)
    rows, K = 24, 256
    w = (rng.standard_normal((3, rows, K)) * np.exp(rng.uniform(-30, 30, (3, rows, 1)))).astype(np.float32)
    w[0, 0] = 0.0
    w[0, 1, :16] = -0.0
    w[0, 2] = np.float32(1e-40)  # fp32 subnormals
    w[1, 3, :32] = 480.0
    w[1, 4] = np.float32(3.0e38)
    w[2] = 0.0  # an all-zero matrix (NVFP4 alpha = 1)
    d = gh.dev()
    wd = torch.from_numpy(w).to(d)
    cb = {"bf16": 2 * K, "mxfp8": K, "nvfp4": K // 2}[dtype]
    codes = torch.zeros(3, rows, cb, dtype=torch.uint8, device=d)
    scales = torch.zeros(3, rows, max(K // {"bf16": K, "mxfp8": 32, "nvfp4": 16}[dtype], 1), dtype=torch.uint8, device=d)
    alpha = torch.zeros(3, dtype=torch.float32, device=d)
    lib.moe_quantize_weights(dtype, 3, rows, K, wd, codes, scales, alpha)
    torch.cuda.synchronize()
    for m in range(3):
        c, s_, a = oquant.quantize_weight(w[m], dtype)
        got = codes[m].cpu().numpy()
        if dtype == "bf16":
            got = got.view(np.uint16)
        assert np.array_equal(got, c), m
        if s_ is not None:
            assert np.array_equal(scales[m].cpu().numpy(), s_), m
        if a is not None:
            assert alpha[m].item() == float(a), m


@pytest.mark.parametrize("name", ["bf16_ragged", "mxfp8_decode_small", "nvfp4_prefill_small"])
def test_graph_capture_replays_match_eager(name):
    """moe_forward and moe_forward_fused captured into a HIP graph: every
    replay, over two different inputs written into the captured buffers and
    with eager calls in between, is bitwise equal to the eager result."""
    w = SMALL[name]
    cw, _ = _setup(w)
    layer = gh.DeviceLayer(w, cw)
    x0, l0 = mi.host_x(w), mi.host_logits(w)
    inputs = [(x0, l0), (np.roll(x0, 1, axis=0).copy(), np.roll(l0, 3, axis=1).copy())]
    x_buf = gh.to_device_x(x0)
    l_buf = torch.from_numpy(l0.copy()).to(gh.dev())

    def load(i):
        x_buf.copy_(gh.to_device_x(inputs[i][0]))
        l_buf.copy_(torch.from_numpy(inputs[i][1]))

    refs = []
    for i in range(2):
        load(i)
        refs.append(gh.bf16_numpy(layer.forward(x_buf, l_buf)))
    assert not np.array_equal(refs[0], refs[1])
    for entry in (layer.forward, layer.forward_fused):
        out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=gh.dev())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            entry(x_buf, l_buf, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            entry(x_buf, l_buf, out=out)
        for rep in range(3):
            for i in range(2):
                load(i)
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(gh.bf16_numpy(out), refs[i]), (entry.__name__, rep, i)
                eager = gh.bf16_numpy(entry(x_buf, l_buf))  # eager work between replays
                assert np.array_equal(eager, refs[i])
        del g
    assert not layer.sync_words().any()


def test_nvfp4_fold_global_scale_bit_exact():
    """The library's fold of every e4m3 scale code under several alphas (the
    weight quantiser's magnitude, powers of two, > 1) equals the oracle's,
    out of place and in place; alpha becomes 1."""
    rng = np.random.default_rng(17)
    alphas = np.array([3.7e-5, 1.2e-4, 2.0 ** -10, 0.5, 1.0, 3.1], np.float32)
    count, rows, K = len(alphas), 8, 256
    scales = rng.integers(0, 0x7F, (count, rows, K // 16)).astype(np.uint8)
    scales[0, 0, :] = np.arange(16, dtype=np.uint8) * 7  # spread over the code range
    ref = np.stack([oquant.nvfp4_fold_global_scale(scales[e], alphas[e])[0] for e in range(count)])
    d = gh.dev()
    s_in = torch.from_numpy(scales).to(d)
    a_in = torch.from_numpy(alphas).to(d)
    s_out = torch.empty_like(s_in)
    a_out = torch.empty_like(a_in)
    lib.moe_nvfp4_fold_global_scale(count, rows, K, s_in, a_in, s_out, a_out)
    torch.cuda.synchronize()
    assert np.array_equal(s_out.cpu().numpy(), ref)
    assert np.array_equal(a_out.cpu().numpy(), np.ones(count, np.float32))
    assert np.array_equal(s_in.cpu().numpy(), scales)  # input untouched
    lib.moe_nvfp4_fold_global_scale(count, rows, K, s_in, a_in)  # in place
    torch.cuda.synchronize()
    assert np.array_equal(s_in.cpu().numpy(), ref) and np.all(a_in.cpu().numpy() == 1.0)


def test_zero_tokens_is_a_noop():
    w = SMALL["tiny_bf16"]
    cw, _ = _setup(w)
    layer = gh.DeviceLayer(w, cw)
    out = torch.full((1, w.H), 7.0, dtype=torch.bfloat16, device=gh.dev())
    x = torch.zeros(0, w.H, dtype=torch.bfloat16, device=gh.dev())
    l = torch.zeros(0, w.E, dtype=torch.float32, device=gh.dev())
    layer.forward(x, l, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_fewer_tokens_than_capacity_reuses_workspace():
    """A workspace sized for max_tokens serves any T <= max_tokens."""
    w = SMALL["mxfp8_decode_small"]
    cw, Wo = _setup(w)
    layer = gh.DeviceLayer(w, cw, max_tokens=4 * w.T)
    x = mi.host_x(w)
    logits = mi.host_logits(w)
    for T in (w.T, 5, 1):
        out = layer.forward(gh.to_device_x(x[:T].copy()), torch.from_numpy(logits[:T].copy()).to(gh.dev()))
        torch.cuda.synchronize()
        ref = omoe.moe_layer(x[:T], logits[:T], Wo, w.k)
        gh.check_out(gh.bf16_numpy(out), ref.out, w.dtype, f"T={T}")
