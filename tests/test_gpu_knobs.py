"""Parity of every knob setting of moe_forward_knobs with the CPU oracle.

Knobs choose among compiled kernel variants [MegaMoE drop workflow, §4 step 3
and §6]: the GEMM variant (decode-shaped 16/32-row token tiles or the
prefill-shaped items) and the MXFP8 fp8 down GEMM change the fp32
accumulation order (correctness knobs: the output must meet the oracle
tolerance); the prefill band, the persistent grid size and the load-balance
deal only reorder work items (performance knobs: the output bits must not
change); the in-kernel fc2 reduce sums w * y with
fp32 atomics in scheduling order (tolerance only, not reproducible bitwise).
Each case forces every variant on shapes the oracle finishes in seconds,
including variants the default heuristic would not pick for that shape.
"""
import itertools

import numpy as np
import pytest
import torch

import gpu_harness as gh
import mixture_experts_layer_sort_amd as lib
import moe_inputs as mi
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

W = mi.WORKLOADS
CASES = {
    # prefill-shaped by default (T k >= 64 E): MXFP8 with the fp8 down GEMM
    "mxfp8_prefill": W["mxfp8_prefill"].scaled(T=300, H=512, I=256, E=4, k=2),
    # 8 n-blocks in both GEMMs: the n-block split (load_balance 3) runs
    "mxfp8_prefill_split": W["mxfp8_prefill"].scaled(T=300, H=2048, I=1024, E=4, k=2),
    "bf16_mxfp8_prefill": W["bf16_mxfp8_prefill"].scaled(T=520, H=256, I=384, E=8, k=2),
    "nvfp4_prefill_relu2": W["nvfp4_decode_t128"].scaled(T=200, H=384, I=256, E=4, k=2, act="relu2"),
    # decode-shaped by default
    "bf16_decode": W["bf16_decode"].scaled(T=33, H=512, I=384, E=16),
    "nvfp4_nt2_clamp": W["nvfp4_decode_t8"].scaled(T=96, H=512, I=256, E=8, k=3, limit=0.3),
    "mxfp8_decode_clamp": W["mxfp8_decode"].scaled(T=40, H=640, I=256, E=32, limit=0.5),
}


def _knob_grid(w):
    down = (0, 1) if gh.weight_format(w.dtype) == "mxfp8" else (1,)
    out = []
    for gemm, d, fc2 in itertools.product((1, 2, 3), down, (0, 1)):
        if fc2 and w.k < 2:
            continue
        # performance knobs: the band and the item deal (prefill-shaped items) and the persistent grid
        perf = ([(0, 0, 0), (128, 0, 0), (4096, 0, 0), (0, 2, 0), (0, 0, 1), (0, 2, 2), (128, 0, 2), (0, 0, 3),
                 (0, 2, 3)] if gemm == 3
                else [(0, 0, 0), (0, 1, 0), (0, 5, 0), (0, 0, 1)])
        for band, blocks, balance in perf:
            out.append((gemm, d, band, fc2, blocks, balance))
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_forward_knobs_parity(name):
    w = CASES[name]
    print(f"case {name}: {w}", flush=True)
    cw, w13f, w2f = gh.canonical_from_host_master(w)
    Wo = omoe.quantize_weights({e: w13f[e] for e in range(w.E)}, {e: w2f[e] for e in range(w.E)}, w.dtype, w.act,
                               w.fold, w.limit)
    x, logits = mi.host_x(w), mi.host_logits(w)
    ref = omoe.moe_layer(x, logits, Wo, w.k)
    layer = gh.DeviceLayer(w, cw)
    xd, ld = gh.to_device_x(x), torch.from_numpy(logits).to(gh.dev())
    base = gh.bf16_numpy(layer.forward(xd, ld))
    # the default knobs are moe_forward's, bit for bit
    assert np.array_equal(gh.bf16_numpy(layer.forward_knobs(xd, ld, None)), base)
    assert np.array_equal(gh.bf16_numpy(layer.forward_knobs(xd, ld, lib.moe_default_knobs())), base)
    by_plan = {}
    for kn in _knob_grid(w):
        got = gh.bf16_numpy(layer.forward_knobs(xd, ld, lib.make_knobs(*kn)))
        rel, mad = gh.check_out(got, ref.out, w.dtype, f"{name} knobs {kn}")
        print(f"  knobs {kn}: out relL2 {rel:.2e} max|d|/rms {mad:.2e}", flush=True)
        gemm, d, band, fc2, blocks, balance = kn
        if not fc2:
            # the band, the grid and the item deal reorder items only: the same bits
            key = (gemm, d)
            if key in by_plan:
                assert np.array_equal(got, by_plan[key]), kn
            by_plan[key] = got
    # forcing the variant the heuristic picks reproduces the default bits
    auto = 3 if w.T * w.k >= 64 * w.E else (2 if w.T * w.k > 16 * w.E else 1)
    assert np.array_equal(by_plan[(auto, 1)], base)
