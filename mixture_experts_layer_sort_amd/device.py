"""Device setup shared by the benchmark and the knob sweep: one layer of a
synthetic workload on the GPU, with canonical weights quantised from the
seeded fp32 masters by the library itself (expert by expert), the packed
weights and the forward workspace, plus the seeded device inputs.

Needs the repository root on sys.path (for the seeded input generators in
moe_inputs).
"""
from __future__ import annotations


class Layer:
    """One layer on the device: canonical weights quantised from the seeded
    fp32 masters by the library (expert by expert), the packed weights and the
    forward workspace."""

    def __init__(self, lib, w, device, max_tokens=None):
        import torch

        E, H, I, R = w.E, w.H, w.I, w.R13
        wf = "mxfp8" if w.dtype == "bf16_mxfp8" else w.dtype
        u8 = torch.uint8
        if wf == "bf16":
            c13, c2 = (torch.empty(E, R, H, dtype=torch.bfloat16, device=device),
                       torch.empty(E, H, I, dtype=torch.bfloat16, device=device))
            s13 = s2 = a13 = a2 = None
        elif wf == "mxfp8":
            c13, c2 = torch.empty(E, R, H, dtype=u8, device=device), torch.empty(E, H, I, dtype=u8, device=device)
            s13, s2 = (torch.empty(E, R, H // 32, dtype=u8, device=device),
                       torch.empty(E, H, I // 32, dtype=u8, device=device))
            a13 = a2 = None
        else:
            c13, c2 = (torch.empty(E, R, H // 2, dtype=u8, device=device),
                       torch.empty(E, H, I // 2, dtype=u8, device=device))
            s13, s2 = (torch.empty(E, R, H // 16, dtype=u8, device=device),
                       torch.empty(E, H, I // 16, dtype=u8, device=device))
            a13, a2 = torch.empty(E, dtype=torch.float32, device=device), torch.empty(E, dtype=torch.float32,
                                                                                       device=device)

        def sub(t, e):
            return None if t is None else t[e:e + 1]

        import moe_inputs as mi

        for e in range(E):
            m13, m2 = mi.device_master_weights(w, e, device)
            lib.moe_quantize_weights(w.dtype, 1, R, H, m13, c13[e:e + 1], sub(s13, e), sub(a13, e))
            lib.moe_quantize_weights(w.dtype, 1, H, I, m2, c2[e:e + 1], sub(s2, e), sub(a2, e))
            if w.fold:
                lib.moe_nvfp4_fold_global_scale(1, R, H, sub(s13, e), sub(a13, e))
                lib.moe_nvfp4_fold_global_scale(1, H, I, sub(s2, e), sub(a2, e))
            del m13, m2
        self.w = w
        self.shape = lib.make_shape(H, I, E, w.k, max_tokens or w.T, w.dtype, w.act, w.limit)
        self.packed = torch.empty(lib.moe_packed_weight_bytes(self.shape), dtype=u8, device=device)
        lib.moe_prepare_weights(self.shape, c13, s13, a13, c2, s2, a2, self.packed)
        self.ws = torch.empty(lib.moe_workspace_bytes(self.shape), dtype=u8, device=device)
        lib.moe_workspace_init(self.shape, self.ws)
        torch.cuda.synchronize()
        del c13, c2, s13, s2, a13, a2

    def sync_words(self):
        """The single-launch kernel's synchronisation words (word 2: spin timeout)."""
        import numpy as np

        return self.ws[: 4 * (4 + self.w.E)].cpu().numpy().view(np.uint32)


def build_layer(w, device):
    """Device inputs (seeded generators) and the layer with library-quantised,
    prepared weights."""
    import torch

    import mixture_experts_layer_sort_amd as lib
    import moe_inputs as mi

    layer = Layer(lib, w, device)
    x = mi.device_x(w, device)
    logits = mi.device_logits(w, device)
    torch.cuda.synchronize()
    return lib, layer, x, logits
