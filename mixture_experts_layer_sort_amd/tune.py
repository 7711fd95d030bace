"""Single-GPU knob sweep that writes the persistent knob cache.

    python -m mixture_experts_layer_sort_amd.tune [--workloads a,b] [--tokens T1,T2]
        [--steps 10] [--warmup 3] [--fc2] [--out PATH]

For every workload (a synthetic layer shape from moe_inputs) and token count,
each candidate knob setting runs the whole layer (moe_forward_knobs) for
`steps` timed steps, each between its own HIP event pair with the L2 and the
Infinity Cache flushed before it; the candidate with the lowest median step
time wins, where settings within 5 % of the fastest (about the spread of
repeated runs of one setting) count as tied and of those the one closest to
the default knobs is kept.  The pages sweep a knob
candidate list per shape, keep the winner in a persistent cache keyed by
shape, and resolve knobs from that cache before a default heuristic
[MegaMoE drop workflow, §4 step 3 and §6]; here every candidate is already
compiled into the library, so a sweep costs only the timed runs.

Candidates: the GEMM variant (decode-shaped 16- or 32-row token tiles,
prefill-shaped items); for decode-shaped items the persistent blocks per
compute unit; for prefill-shaped items the band of the item order (token
rows sharing weight tiles) and, for MXFP8 layers, the fp8 or bf16 down GEMM.  The in-kernel fc2 reduce makes outputs non-reproducible; it is a
candidate only with --fc2.

Lines of the cache cover token ranges: between two swept token counts of one
shape the boundary is their geometric mean; the smallest count's line starts
at 1 and the largest one's runs to 2^24.  A winning GEMM variant that the
default heuristic would pick at that token count is written as 0 (auto), so
that other token counts in the range keep the per-call choice.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEFAULT_WORKLOADS = ("bf16_decode", "mxfp8_decode", "nvfp4_decode_t8", "nvfp4_decode_t128", "mxfp8_prefill")
BANDS = (0, 256, 512, 2048, 4096, 8192)
DECODE_BLOCKS = (0, 2, 4, 5, 6, 8)
LOAD_BALANCE = (0, 1, 2, 3)
MAX_T = 1 << 24
# Settings within this factor of the fastest count as tied (above the spread of single sweep runs:
# repeated runs of one setting differ by up to ~4 %); of the tied settings the one with the fewest
# knobs away from the defaults wins, so the defaults win whenever they are tied.
TIE = 1.05


KNOBS = 6  # gemm, down_fp8, band_rows, fc2_reduce, blocks_per_cu, load_balance


def candidates(w, T, fc2):
    """Knob tuples (gemm, down_fp8, band_rows, fc2_reduce, blocks_per_cu, load_balance) for workload w at T
    tokens."""
    mx = w.dtype == "mxfp8"
    out = []
    for red in ((0, 1) if fc2 and w.k >= 2 else (0,)):
        for gemm in (1, 2):
            for blocks in DECODE_BLOCKS:
                out.append((gemm, 1, 0, red, blocks, 0))
        for down in ((1, 0) if mx else (1,)):
            for band in BANDS:
                out.append((3, down, band, red, 0, 0))
            for balance in LOAD_BALANCE[1:]:
                out.append((3, down, 0, red, 0, balance))
        out.append((3, 1, 0, red, 2, 0))
    return out


def full_knobs(kn):
    """A recorded knob tuple with the knobs added since it was recorded at their defaults (0)."""
    kn = tuple(kn)
    return kn + (0,) * (KNOBS - len(kn))


def auto_gemm(T, k, E):
    """The variant the default heuristic picks (as the library's knob 0)."""
    if T * k >= 64 * E:
        return 3
    return 2 if T * k > 16 * E else 1


def shape_key(w):
    return (w.dtype, w.act, w.H, w.I, w.E, w.k)


def token_ranges(ts):
    """[(t, lo, hi)] for sorted distinct token counts ts."""
    ts = sorted(set(ts))
    out = []
    for i, t in enumerate(ts):
        lo = 1 if i == 0 else int(math.isqrt(ts[i - 1] * t)) + 1
        hi = MAX_T if i == len(ts) - 1 else int(math.isqrt(t * ts[i + 1]))
        out.append((t, lo, hi))
    return out


def sweep(lib, w, tokens, steps, warmup, fc2, device, log):
    """{T: [(knobs, median_ms)]} for one workload."""
    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sort_amd.device import Layer

    tmax = max(tokens)
    wl = w.scaled(T=tmax)
    layer = Layer(lib, wl, device)
    x_all = mi.device_x(wl, device)
    l_all = mi.device_logits(wl, device)
    out = torch.empty(tmax, w.H, dtype=torch.bfloat16, device=device)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=device)  # 1 GiB
    flush_sink = torch.empty((), dtype=torch.float32, device=device)
    res = {}
    for T in tokens:
        x, logits = x_all[:T], l_all[:T]
        rows = []
        for kn in candidates(w, T, fc2):
            knobs = lib.make_knobs(*kn)

            def step():
                lib.moe_forward_knobs(layer.shape, T, layer.packed, logits, x, out, layer.ws, knobs)

            for _ in range(warmup):
                step()
            starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            for i in range(steps):
                flush_sink.copy_(flush_buf.sum())
                starts[i].record()
                step()
                ends[i].record()
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))[steps // 2]
            rows.append((kn, ms))
            log(f"  {w.name} T={T} knobs {kn}: {ms:.4f} ms")
        res[T] = rows
    del layer, flush_buf
    torch.cuda.empty_cache()
    return res


def pick(w, T, rows):
    """(the chosen (knobs, ms), the default knobs' (knobs, ms) or None)."""
    default = (auto_gemm(T, w.k, w.E), 1, 0, 0, 0, 0)
    best = min(r[1] for r in rows)
    tied = [r for r in rows if r[1] <= TIE * best]
    chosen = min(tied, key=lambda r: (sum(a != b for a, b in zip(r[0], default)), r[1]))
    d = [r for r in rows if r[0] == default]
    return chosen, (d[0] if d else None)


def sweep_all(lib, mi, args, device, by_shape, record, log):
    """Sweep every requested shape; fills by_shape {key: {T: (knobs, ms, default_ms, label)}} and record.
    Workloads of one layer shape write one set of cache lines; each token count is timed with the routing
    of the workload that asks for it (a skewed prefill batch and a decode batch of the same shape route
    differently)."""
    groups = {}
    for item in args.workloads.split(","):
        name, _, own = item.partition(":")
        w = mi.WORKLOADS[name]
        if own:
            tokens = {int(t) for t in own.split("+")}
        elif args.tokens:
            tokens = {int(t) for t in args.tokens.split(",")}
        else:
            tokens = {w.T}
        groups.setdefault(shape_key(w), []).append((w, tokens))
    for key, members in groups.items():
        taken = set()
        for w, tokens in members:
            tokens = sorted(tokens - taken)  # a token count two workloads ask for: the first one's routing
            taken.update(tokens)
            if not tokens:
                continue
            log(f"sweeping {w.name} at T = {tokens}")
            res = sweep(lib, w, tokens, args.steps, args.warmup, args.fc2, device, log)
            for T, rows in res.items():
                (kn, ms), dflt = pick(w, T, rows)
                by_shape.setdefault(key, {})[T] = (kn, ms, dflt[1] if dflt else None, w.name)
                record.append({"workloads": [w.name], "shape": list(key), "T": T, "winner": list(kn), "ms": ms,
                               "default_ms": dflt[1] if dflt else None,
                               "candidates": [{"knobs": list(k), "ms": m} for k, m in rows]})
                log(f"{w.name} T={T}: knobs {kn} {ms:.4f} ms (default {dflt[1] if dflt else float('nan'):.4f} ms)")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", default=",".join(DEFAULT_WORKLOADS),
                    help="comma-separated workload names, each optionally with its own token counts "
                         "as name:T1+T2+...")
    ap.add_argument("--tokens", default="", help="token counts to sweep for workloads without their own "
                                                 "(default: each workload's T)")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fc2", action="store_true", help="also try the in-kernel fc2 reduce (non-deterministic)")
    ap.add_argument("--out", default=None, help="cache file to write (default: the package's knob_cache.txt)")
    ap.add_argument("--json", default=None, help="also write every measurement to this JSON file")
    ap.add_argument("--from-json", default=None,
                    help="write the cache from the measurements of an earlier run's --json file (no GPU work)")
    args = ap.parse_args(argv)

    sys.path.insert(0, ROOT)
    import mixture_experts_layer_sort_amd as lib
    import moe_inputs as mi

    def log(msg):
        print(msg, flush=True)

    by_shape = {}
    record = []
    if args.from_json:
        with open(args.from_json) as f:
            data = json.load(f)
            for rec in data["sweeps"] if isinstance(data, dict) else data:
                key = tuple(rec["shape"])
                w = mi.WORKLOADS[rec["workloads"][0]]
                rows = [(full_knobs(c["knobs"]), c["ms"]) for c in rec["candidates"]]
                (kn, ms), dflt = pick(w, rec["T"], rows)
                by_shape.setdefault(key, {})[rec["T"]] = (kn, ms, dflt[1] if dflt else None,
                                                          "+".join(rec["workloads"]))
                record.append(rec)
    else:
        import torch

        device = torch.device("cuda:0")
        sweep_all(lib, mi, args, device, by_shape, record, log)

    cmd = "python -m mixture_experts_layer_sort_amd.tune " + " ".join(argv if argv is not None else sys.argv[1:])
    lines = ["# Knob cache of the MoE layer library (moe_knob_cache_lookup).",
             "# dtype act hidden inter experts top_k t_min t_max : gemm down_fp8 band_rows fc2_reduce blocks_per_cu"
             " load_balance",
             f"# written by: {cmd.strip()}",
             "# each line: the fastest knobs at the swept token count (median of flushed steps on one MI355X)"]
    for key in sorted(by_shape):
        dtype, act, H, I, E, k = key
        for T, lo, hi in token_ranges(by_shape[key]):
            kn, ms, dms, name = by_shape[key][T]
            note = f"{name} T={T}: {ms:.4f} ms" + (f", default knobs {dms:.4f} ms" if dms is not None else "")
            # a winning variant that the heuristic picks anyway is written as 0 (auto), so calls of other
            # sizes in the line's range keep the per-call choice
            gemm = 0 if kn[0] == auto_gemm(T, k, E) else kn[0]
            lines.append(f"{dtype} {act} {H} {I} {E} {k} {lo} {hi} : {gemm} {kn[1]} {kn[2]} {kn[3]} {kn[4]} {kn[5]}"
                         f"  # {note}")
    path = args.out or lib.KNOB_CACHE_PATH
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {path}")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(record, f, indent=1)


if __name__ == "__main__":
    main()
