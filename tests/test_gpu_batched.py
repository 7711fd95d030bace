"""moe_batched_experts (tokens bucketed per expert, no routing or combine)
against the oracle's batched_experts: every valid row within the layer
tolerance (relative L2 per format, max |diff| <= 5e-2 RMS), rows past the
counts untouched; counts of zero, of the capacity and above it (clamped);
decode-shaped (16- and 32-row token tiles) and prefill-shaped GEMMs."""
import numpy as np
import pytest
import torch

import gpu_harness as gh
import mixture_experts_layer_sort_amd as lib
import moe_inputs as mi
from oracle import codecs
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

W = mi.WORKLOADS
CASES = {
    # max_rows 5: 16-row token tiles; 24: 32-row tiles; 96: the prefill-shaped GEMMs
    "bf16_m5": (W["bf16_decode"].scaled(H=512, I=256, E=8), 5),
    "mxfp8_m24": (W["mxfp8_decode"].scaled(H=512, I=256, E=8), 24),
    "nvfp4_m5": (W["nvfp4_decode_t8"].scaled(H=512, I=256, E=8), 5),
    "mxfp8_m96": (W["mxfp8_prefill"].scaled(H=512, I=256, E=6, k=2), 96),
    "nvfp4_m96": (W["nvfp4_decode_t128"].scaled(H=384, I=128, E=4, k=2), 96),
    "bf16_mxfp8_m24": (W["bf16_mxfp8_decode"].scaled(H=512, I=256, E=8), 24),
    "relu2_mxfp8_m5": (W["mxfp8_decode"].scaled(H=512, I=256, E=8, act="relu2"), 5),
    "clamp_bf16_m96": (W["bf16_decode"].scaled(H=256, I=256, E=4, k=2, limit=0.3), 96),
}


@pytest.mark.parametrize("name", list(CASES))
def test_batched_experts_parity(name):
    w, M = CASES[name]
    print(f"case {name}: {w} max_rows={M}", flush=True)
    cw, w13f, w2f = gh.canonical_from_host_master(w)
    Wo = omoe.quantize_weights({e: w13f[e] for e in range(w.E)}, {e: w2f[e] for e in range(w.E)}, w.dtype, w.act,
                               w.fold, w.limit)
    layer = gh.DeviceLayer(w.scaled(T=1), cw)
    rng = np.random.default_rng(len(name))
    counts = rng.integers(1, M + 1, w.E).astype(np.int32)
    counts[0], counts[-1] = 0, M
    if w.E > 2:
        counts[1] = M + 5  # above the capacity: clamped
    xb = mi.f32_to_bf16_bits(rng.standard_normal((w.E, M, w.H)).astype(np.float32))
    d = gh.dev()
    y = torch.full((w.E, M, w.H), 7.0, dtype=torch.bfloat16, device=d)
    ws = torch.empty(lib.moe_batched_workspace_bytes(layer.shape, M), dtype=torch.uint8, device=d)
    lib.moe_batched_experts(layer.shape, M, torch.from_numpy(counts).to(d), gh.to_device_x(xb.reshape(-1, w.H)),
                            layer.packed, y, ws)
    torch.cuda.synchronize()
    got = codecs.bf16_decode(gh.bf16_numpy(y).reshape(w.E, M, w.H))
    ref = omoe.batched_experts(xb, counts, Wo)
    valid = np.arange(M)[None, :] < np.minimum(counts, M)[:, None]
    g, r = got[valid], ref[valid]
    rel = gh.rel_l2(g, r)
    mad = float(np.max(np.abs(g - r))) / float(np.sqrt(np.mean(r * r)))
    print(f"  {int(valid.sum())} rows: relL2 {rel:.2e} max|d|/rms {mad:.2e}", flush=True)
    assert rel <= gh.out_tolerance(w.dtype) and mad <= 5e-2
    assert np.all(got[~valid] == 7.0)


def test_batched_all_empty_is_a_noop():
    w, M = CASES["bf16_m5"]
    cw, _, _ = gh.canonical_from_host_master(w)
    layer = gh.DeviceLayer(w.scaled(T=1), cw)
    d = gh.dev()
    y = torch.full((w.E, M, w.H), 3.0, dtype=torch.bfloat16, device=d)
    x = torch.zeros(w.E * M, w.H, dtype=torch.bfloat16, device=d)
    ws = torch.empty(lib.moe_batched_workspace_bytes(layer.shape, M), dtype=torch.uint8, device=d)
    lib.moe_batched_experts(layer.shape, M, torch.zeros(w.E, dtype=torch.int32, device=d), x, layer.packed, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
