"""moe_forward_noalloc (intermediates in the library's static device scratch)
against moe_forward (caller workspace): two calls in a row on one layer, the
second with fewer tokens, must give bitwise the same outputs, routing ids and
weights; a batch whose intermediates exceed the scratch is refused on the
host with nothing enqueued."""
import numpy as np
import pytest
import torch

import gpu_harness as gh
import mixture_experts_layer_sort_amd as lib
import moe_inputs as mi

pytestmark = pytest.mark.gpu

W = mi.WORKLOADS
CASES = {
    "mxfp8_decode_small": W["mxfp8_decode"].scaled(T=40, H=640, I=256, E=32),
    "nvfp4_t128_wide": W["nvfp4_decode_t128"].scaled(E=16),
    "bf16_nt2": W["bf16_decode"].scaled(T=96, H=512, I=256, E=8, k=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_forward(name):
    w = CASES[name]
    print(f"case {name}: {w}", flush=True)
    cw, _, _ = gh.canonical_from_host_master(w)
    layer = gh.DeviceLayer(w, cw)
    d = gh.dev()
    x_all, l_all = mi.host_x(w), mi.host_logits(w)
    for T, rows in ((w.T, slice(0, w.T)), (max(1, w.T // 3), slice(w.T - max(1, w.T // 3), w.T))):
        x = gh.to_device_x(np.ascontiguousarray(x_all[rows]))
        logits = torch.from_numpy(np.ascontiguousarray(l_all[rows])).to(d)
        ids_a = torch.empty(T, w.k, dtype=torch.int32, device=d)
        wts_a = torch.empty(T, w.k, dtype=torch.float32, device=d)
        out_a = layer.forward(x, logits, ids=ids_a, wts=wts_a)
        ids_b = torch.full((T, w.k), -1, dtype=torch.int32, device=d)
        wts_b = torch.full((T, w.k), -1.0, dtype=torch.float32, device=d)
        out_b = torch.full((T, w.H), 7.0, dtype=torch.bfloat16, device=d)
        lib.moe_forward_noalloc(layer.shape, T, layer.packed, logits, x, out_b, ids_b, wts_b)
        torch.cuda.synchronize()
        assert np.array_equal(gh.bf16_numpy(out_b), gh.bf16_numpy(out_a)), (name, T)
        assert torch.equal(ids_a, ids_b) and torch.equal(wts_a, wts_b), (name, T)
        print(f"  T={T}: bitwise equal to moe_forward", flush=True)


def test_noalloc_refuses_oversized_batch():
    """Prefill-sized batch: the intermediates exceed the scratch array; the
    call returns the workspace error and leaves the output untouched."""
    w = W["mxfp8_prefill"].scaled(H=256, I=128, E=4, k=2, T=64)
    cw, _, _ = gh.canonical_from_host_master(w)
    layer = gh.DeviceLayer(w, cw)
    big = lib.make_shape(7168, 2048, 256, 8, 8192, "mxfp8")
    out = torch.full((1, 7168), 3.0, dtype=torch.bfloat16, device=gh.dev())
    x = torch.zeros(1, 7168, dtype=torch.bfloat16, device=gh.dev())
    logits = torch.zeros(1, 256, dtype=torch.float32, device=gh.dev())
    with pytest.raises(lib.MoeError, match="workspace"):
        lib.moe_forward_noalloc(big, 8192, layer.packed, logits, x, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
