"""Benchmark of the fused MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole layer over one batch (route -> permute +
activation quantisation -> gate/up GEMM + SwiGLU + requant -> down GEMM ->
combine), i.e. one moe_forward_knobs call with the knobs the package's knob
cache holds for the shape (else the defaults; reported in config.knobs),
with inputs and prepared weights already resident in HBM.  The default
workload is the MXFP8 prefill layer (T=8192, H=7168, I=2048, E=256, top-8,
Zipf(1.1)-skewed routing); --workload picks any other (e.g. bf16_decode,
mxfp8_decode, nvfp4_decode_t8, nvfp4_decode_t128).

Prints one JSON line with tokens/s (K steps, the five stage kernels back to
back on torch's stream, each step between HIP events, with the L2 and the
Infinity Cache flushed by reading 1 GiB before every step outside the timed
intervals), the roofline of the dominant kernel (the gate/up GEMM, timed with
HIP events on its launch stream over a second region of K steps through the
staged entry points, flushed the same way), whole-layer HBM / MFMA
fractions, the back-to-back (unflushed) step time, the step time when the
same call is captured into a HIP graph and replayed, the step time with the
in-kernel fc2 reduce, the single-launch entry's step time, a measured device
copy (GB/s) for context, and the CPU oracle (its expert-grouped BLAS form)
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# MI355X dense matrix peaks, published (no sparsity)
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
# The prefill roofline is priced at the dense peak of the layer format's own
# data type: MXFP8 layers against the fp8 peak (whatever instruction the
# kernel uses), bf16 and NVFP4 (run as exact fp16 products) against the
# 16-bit peak; bf16 x MXFP8 runs bf16 products, priced at the bf16 peak.
MFMA_PEAK_TFLOPS = {"bf16": BF16_PEAK_TFLOPS, "mxfp8": FP8_PEAK_TFLOPS, "nvfp4": BF16_PEAK_TFLOPS,
                    "bf16_mxfp8": BF16_PEAK_TFLOPS}
# the arithmetic type of the contractions per layer format ("bf16_mxfp8": bf16
# activations over MXFP8 weights)
# (MXFP8 layers: gate/up on bf16 products of the exact codes, the prefill-shaped
# down GEMM on the e4m3 block-scaled instruction)
ARITH_DTYPE = {"bf16": "bf16", "mxfp8": "bf16/e4m3", "nvfp4": "f16", "bf16_mxfp8": "bf16"}
DEFAULT_WORKLOAD = "mxfp8_prefill"
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mixture_experts_layer_sort_amd", "csrc")


def _bytes_per_elem(fmt):
    # codes + block scales (MXFP8: 1 + 1/32, NVFP4: 1/2 + 1/16)
    return {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32, "nvfp4": 0.5 + 1.0 / 16}[fmt]


def weight_bytes_per_elem(dtype):
    return _bytes_per_elem("mxfp8" if dtype == "bf16_mxfp8" else dtype)


def act_bytes_per_elem(dtype):
    return _bytes_per_elem("bf16" if dtype == "bf16_mxfp8" else dtype)


def kernel_source_hash():
    """Hash of every kernel source (the counters describe one build)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per gate/up GEMM launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"gemm13_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def build_layer(w, device):
    """Device inputs (seeded generators) and the layer with library-quantised,
    prepared weights."""
    import torch

    import mixture_experts_layer_sort_amd as lib
    import moe_inputs as mi
    from mixture_experts_layer_sort_amd.device import Layer

    layer = Layer(lib, w, device)
    x = mi.device_x(w, device)
    logits = mi.device_logits(w, device)
    torch.cuda.synchronize()
    return lib, layer, x, logits


class StagedStep:
    """The layer as its five entry points on torch's current stream, with HIP
    events around each kernel launch (the same kernels moe_forward runs)."""

    NAMES = ("route", "permute", "gemm13", "gemm2", "combine")

    def __init__(self, lib, layer, x, logits):
        import torch

        w, s, d = layer.w, layer.shape, x.device
        self.lib, self.layer, self.x, self.logits, self.s = lib, layer, x, logits, s
        T, P = w.T, w.T * w.k
        self.T = T
        self.ids = torch.empty(T, w.k, dtype=torch.int32, device=d)
        self.wts = torch.empty(T, w.k, dtype=torch.float32, device=d)
        self.off = torch.empty(w.E + 1, dtype=torch.int32, device=d)
        self.sp = torch.empty(P, dtype=torch.int32, device=d)
        self.pp = torch.empty(P, dtype=torch.int32, device=d)
        self.xq = x if w.dtype in ("bf16", "bf16_mxfp8") else torch.empty(lib.moe_xq_bytes(s, T), dtype=torch.uint8,
                                                                          device=d)
        self.hq = torch.empty(lib.moe_hq_bytes(s, T), dtype=torch.uint8, device=d)
        self.y = torch.empty(P, w.H, dtype=torch.bfloat16, device=d)
        self.out = torch.empty(T, w.H, dtype=torch.bfloat16, device=d)
        self.events = []

    def run(self, timed=False):
        import torch

        lib, s, T, L = self.lib, self.s, self.T, self.layer
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)] if timed else None
        rec = (lambda i: ev[i].record()) if timed else (lambda i: None)
        rec(0)
        lib.moe_route(s, T, self.logits, self.ids, self.wts)
        rec(1)
        lib.moe_permute(s, T, self.ids, self.x, self.off, self.sp, self.pp, self.xq)
        rec(2)
        lib.moe_gemm13_swiglu_quant(s, T, L.packed, self.off, self.sp, self.xq, self.hq)
        rec(3)
        lib.moe_gemm2(s, T, L.packed, self.off, self.sp, self.hq, self.y)
        rec(4)
        lib.moe_combine(s, T, self.y, self.wts, self.out)
        rec(5)
        if timed:
            self.events.append(ev)

    def kernel_ms(self):
        """Average duration (ms) of each kernel over the recorded steps."""
        n = len(self.events)
        return {name: sum(e[i].elapsed_time(e[i + 1]) for e in self.events) / n for i, name in enumerate(self.NAMES)}


def layer_bytes_flops(w, n_active):
    """Algorithmic bytes and flops of one step: weights (with scales) of the
    active experts, x in, out, logits; flops 2*H*(R13 + I) per routed pair
    (R13 = 2I rows of W13 for SwiGLU experts, I for ReLU^2)."""
    wb = n_active * (w.R13 + w.I) * w.H * weight_bytes_per_elem(w.dtype)
    B = wb + 2 * w.T * w.H * 2 + 4 * w.T * w.E
    F = w.T * w.k * 2.0 * w.H * (w.R13 + w.I)
    return B, F


def gemm13_bytes(w, n_active):
    """Algorithmic bytes of one gate/up GEMM launch: W13 of the active experts
    (with scales), the quantised activations read, the intermediate written."""
    return (n_active * w.R13 * w.H * weight_bytes_per_elem(w.dtype) + w.T * w.H * act_bytes_per_elem(w.dtype)
            + w.T * w.k * w.I * act_bytes_per_elem(w.dtype))


def _quantize_expert(args):
    """Oracle quantisation of one expert's fp32 masters (worker process)."""
    w13, w2, dtype, act, fold = args
    from oracle import moe as omoe

    W = omoe.quantize_weights({0: w13}, {0: w2}, dtype, act, fold)
    return tuple(None if getattr(W, n) is None else getattr(W, n)[0]
                 for n in ("w13", "w2", "w13_s", "w2_s", "w13_a", "w2_a"))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, device, ids, max_experts=12, max_tokens=1024):
    """The CPU oracle's expert-grouped form (BLAS matrix products) timed on a
    bounded sample of the same workload: the tokens (in index order, at most
    max_tokens) whose k experts all lie among the max_experts experts with the
    most routed rows, with the oracle's own weights quantised from the same
    seeded fp32 masters (quantisation not timed; dequantisation of the sampled
    experts and routing -> output timed)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import moe_inputs as mi
    from oracle import moe as omoe

    counts = np.bincount(ids.ravel(), minlength=w.E)
    hot = set(int(e) for e in np.argsort(-counts, kind="stable")[:max_experts] if counts[e] > 0)
    toks = [t for t in range(w.T) if set(ids[t].tolist()) <= hot][:max_tokens]
    if not toks:  # fall back to the first tokens whose experts fit the budget
        experts = set()
        for t in range(w.T):
            nxt = experts | set(ids[t].tolist())
            if toks and len(nxt) > max_experts:
                break
            toks.append(t)
            experts = nxt
        hot = experts
    toks = np.array(toks)
    experts = sorted(set(int(e) for e in ids[toks].ravel()))
    x = mi.device_x(w, device).view(torch.int16).cpu().numpy().view(np.uint16)[toks]
    logits = mi.device_logits(w, device).cpu().numpy()[toks]
    jobs = []
    for e in experts:
        a, b = mi.device_master_weights(w, e, device)
        jobs.append((a.cpu().numpy(), b.cpu().numpy(), w.dtype, w.act, w.fold))
    with cf.ProcessPoolExecutor(max_workers=min(16, len(jobs)), mp_context=mp.get_context("spawn")) as ex:
        parts = list(ex.map(_quantize_expert, jobs))
    del jobs
    # a dense expert dimension: experts outside the sample are never routed to here
    full = {n: {} for n in ("w13", "w2", "w13_s", "w2_s", "w13_a", "w2_a")}
    for e, p in zip(experts, parts):
        for n, v in zip(("w13", "w2", "w13_s", "w2_s", "w13_a", "w2_a"), p):
            full[n][e] = v
    Wo = omoe.Weights(w.dtype, full["w13"], full["w2"], full["w13_s"] or None, full["w2_s"] or None,
                      full["w13_a"] if all(v is not None for v in full["w13_a"].values()) else None,
                      full["w2_a"] if all(v is not None for v in full["w2_a"].values()) else None, act=w.act,
                      limit=w.limit)
    if Wo.w13_s is not None and any(v is None for v in Wo.w13_s.values()):
        Wo.w13_s = Wo.w2_s = None
    # route on the sampled tokens' logits; the grouped form dequantises each routed expert once
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 10.0 and reps < 20):
        t0 = time.perf_counter()
        omoe.moe_layer_grouped(x, logits, Wo, w.k)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": len(toks) * reps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "sample": f"{len(toks)} of {w.T} tokens (those routed only to the {len(hot)} experts with the most "
                      f"rows; {len(experts)} experts) x {reps} passes of the expert-grouped oracle (numpy BLAS, "
                      f"fp64), {dt:.1f} s wall incl. dequantisation, weight quantisation excluded"}


def measure_achievable(torch, device):
    """Measured context for the HBM peak: a 1 GiB device-to-device copy (GB/s
    of read + write traffic)."""
    res = {}
    a = torch.empty(1 << 28, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    res["device_copy_gbs"] = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-single-launch", action="store_true", help="do not time moe_forward_fused")
    ap.add_argument("--skip-fc2", action="store_true", help="do not time the in-kernel fc2 reduce")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--dma-probe", action="store_true",
                    help="only run the layer on a single-expert MXFP8 prefill shape whose gate/up GEMM fetches "
                         "each operand byte once through its direct-to-LDS loads (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi

    device = torch.device("cuda:0")
    if args.copy_probe:
        a = torch.ones(1 << 28, dtype=torch.float32, device=device)  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": a.numel() * 4}))
        return

    if args.dma_probe:
        # E = 1, T = 256 routed rows, I = 256: the gate/up GEMM (prefill-shaped, 128-row items) runs
        # 2 m-tiles x 2 blocks of 256 weight rows as four items side by side on one XCD (the
        # XCD-contiguous item order); they stream K in near lockstep, so the L2 misses are the unique
        # operand bytes: the W13 codes and scales and the 16-bit copy of the 256 token rows.
        w = mi.WORKLOADS["mxfp8_prefill"].scaled(T=256, I=256, E=1, k=1, bias="none", name="dma_probe")
        lib, layer, x, logits = build_layer(w, device)
        step = StagedStep(lib, layer, x, logits)
        for _ in range(3):
            step.run()
        torch.cuda.synchronize()
        w13 = w.R13 * w.H * (1 + 1 / 32)
        toks = w.T * w.H * 2
        print(json.dumps({"dma_probe_gemm13_unique_fetch_bytes": w13 + toks, "w13_bytes": w13,
                          "token_copy_bytes": toks, "launches": 3}))
        return

    w = mi.WORKLOADS[args.workload]
    lib, layer, x, logits = build_layer(w, device)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=device)
    ids_t = torch.empty(w.T, w.k, dtype=torch.int32, device=device)
    wts_t = torch.empty(w.T, w.k, dtype=torch.float32, device=device)

    # knobs resolved once, as a serving engine would: the package's knob cache, else the defaults
    knobs, cache_hit = lib.moe_knob_cache_lookup(layer.shape, w.T)

    def forward():
        lib.moe_forward_knobs(layer.shape, w.T, layer.packed, logits, x, out, layer.ws, knobs, topk_ids=ids_t,
                              topk_w=wts_t)

    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=device)  # 1 GiB
    flush_sink = torch.empty((), dtype=torch.float32, device=device)

    def flush(i):
        # Evict the L2s and the 256 MB Infinity Cache by reading 1 GiB, enqueued
        # outside the timed intervals.  A read, not a write: a write leaves the
        # memory-side cache full of dirty lines whose write-back then competes
        # with the next step's reads (measured: -20 % on NVFP4 decode).
        flush_sink.copy_(flush_buf.sum())

    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    ids = ids_t.cpu().numpy()
    n_active = int(len(np.unique(ids)))

    # timed region: K steps of moe_forward (five kernels each) on torch's stream,
    # each step between its own HIP event pair, caches flushed before every step
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush(i)
        starts[i].record()
        forward()
        ends[i].record()
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    ms_step = step_ms[len(step_ms) // 2]  # median
    gpu_ms_step = ms_step

    # the same step captured once into a HIP graph and replayed (context):
    # flushed and timed like the eager steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    g_ms = []
    for i in range(args.steps):
        flush(i)
        starts[i].record()
        graph.replay()
        ends[i].record()
    torch.cuda.synchronize()
    g_ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    graph_ms_step = g_ms[len(g_ms) // 2]
    del graph

    # the in-kernel fc2 reduce (a correctness knob: outputs not bitwise
    # reproducible), flushed and timed like the eager steps (context)
    fc2_ms_step = None
    if w.k >= 2 and not args.skip_fc2:
        fc2_knobs = lib.make_knobs(knobs.gemm, knobs.down_fp8, knobs.band_rows, 1, knobs.blocks_per_cu,
                                   knobs.load_balance)

        def forward_fc2():
            lib.moe_forward_knobs(layer.shape, w.T, layer.packed, logits, x, out, layer.ws, fc2_knobs)

        for _ in range(3):
            forward_fc2()
        for i in range(args.steps):
            flush(i)
            starts[i].record()
            forward_fc2()
            ends[i].record()
        torch.cuda.synchronize()
        f_ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
        fc2_ms_step = f_ms[len(f_ms) // 2]

    # back to back, unflushed (context): one event pair around K steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        forward()
    ev1.record()
    torch.cuda.synchronize()
    b2b_ms_step = ev0.elapsed_time(ev1) / args.steps

    # kernel timing region: K steps of the same kernels through the staged entry
    # points, HIP events around every kernel (the events themselves add gaps),
    # caches flushed before every step
    step = StagedStep(lib, layer, x, logits)
    for _ in range(3):
        step.run()
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush(i)
        step.run(timed=True)
    torch.cuda.synchronize()
    kms = step.kernel_ms()
    del flush_buf
    achievable = measure_achievable(torch, device)

    # the single-launch entry, for comparison
    def fused():
        lib.moe_forward_fused(layer.shape, w.T, layer.packed, logits, x, out, layer.ws)

    fused_ms = None
    if not args.skip_single_launch:
        for _ in range(3):
            fused()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(args.steps):
            fused()
        f1.record()
        torch.cuda.synchronize()
        fused_ms = f0.elapsed_time(f1) / args.steps
        if layer.sync_words()[2]:
            raise RuntimeError("the single-launch kernel reported a spin timeout")

    B, F = layer_bytes_flops(w, n_active)
    layer_gbs = B / (gpu_ms_step * 1e-3) / 1e9
    tflops = F / (gpu_ms_step * 1e-3) / 1e12
    g13b = gemm13_bytes(w, n_active)
    g13_gbs = g13b / (kms["gemm13"] * 1e-3) / 1e9
    g13_tflops = w.T * w.k * 2.0 * w.H * w.R13 / (kms["gemm13"] * 1e-3) / 1e12
    traffic = load_traffic(w.name)
    decode = w.T * w.k <= 16 * w.E
    if decode:
        roof = {"bound": "hbm", "kernel": "gemm13_swiglu_quant", "achieved": g13_gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": g13_gbs / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": g13b, "avg_launch_ms": kms["gemm13"]}
    else:
        roof = {"bound": "mfma", "kernel": "gemm13_swiglu_quant", "achieved": g13_tflops,
                "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s", "frac": g13_tflops / MFMA_PEAK_TFLOPS[w.dtype],
                "frac_of_bf16_peak": g13_tflops / BF16_PEAK_TFLOPS,
                "traffic": traffic, "algorithmic_flops_per_launch": w.T * w.k * 2.0 * w.H * w.R13,
                "avg_launch_ms": kms["gemm13"]}
    rec = {
        "metric": "MoE layer tokens/s; % HBM BW (decode) / % MFMA peak (prefill)",
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ARITH_DTYPE[w.dtype],
        "data": "synthetic (seeded N(0,1) x and logits, N(0,0.02) weights; random init)",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "inter": w.I, "experts": w.E, "top_k": w.k,
                   "weights": w.dtype, "activation": w.act, "weight_alpha_folded": w.fold, "routing_skew": w.bias,
                   "active_experts": n_active, "knobs": knobs.as_dict(), "knob_cache_hit": cache_hit},
        "roofline": roof,
        "layer": {"algorithmic_bytes": B, "flops": F, "gpu_ms_per_step": gpu_ms_step, "hbm_gbs": layer_gbs,
                  "hbm_frac": layer_gbs / HBM_PEAK_GBS, "mfma_tflops": tflops,
                  "mfma_frac": tflops / MFMA_PEAK_TFLOPS[w.dtype],
                  "mfma_frac_of_bf16_peak": tflops / BF16_PEAK_TFLOPS,
                  "regime": "decode" if decode else "prefill", "staged_kernel_ms": kms,
                  "step_ms_min_median_max": [step_ms[0], ms_step, step_ms[-1]],
                  "back_to_back_unflushed_ms_per_step": b2b_ms_step,
                  "graph_replay_ms_per_step": graph_ms_step,
                  "fc2_reduce_ms_per_step": fc2_ms_step,
                  "single_launch_ms_per_step": fused_ms,
                  # the staged entry points run the default knobs; the roofline kernel is the step's
                  # own kernel when the resolved knobs are the defaults
                  "staged_knobs_are_step_knobs": knobs.as_dict() == lib.moe_default_knobs().as_dict()},
        "achievable": achievable,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, device, ids)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
