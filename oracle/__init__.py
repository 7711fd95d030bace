"""CPU oracle of the fused MoE expert layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the layer
computes, used to check the HIP library.  Only the test suite, the smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The library's
product path never routes through it, and the two share no code: the only
module both sides use is ``moe_inputs`` (seeded random inputs, no layer
arithmetic).

Sources.  The method is described by three web pages:

* [MegaMoE drop workflow] "FlashInfer CuTeDSL MegaMoE kernel drop update
  workflow" (an article on vendoring the Blackwell MegaMoE kernels into
  FlashInfer's expert-parallel MoE runtime);
* [vLLM PR 38050 report] analysis report of vLLM PR 38050 (FlashInfer
  CuteDSL NVFP4 MoE kernel, batched experts);
* [vLLM PR 40082 report] full report of vLLM PR 40082 (FlashInfer b12x
  fused MoE and FP4 GEMM for SM120/SM121).

The pages give the pipeline (routing, token dispatch, W1 GEMM, SwiGLU, W2
GEMM, reduction) and the quantisation conventions, but no numeric worked
example.  Where they are silent this package takes the plainest reading;
each module states its readings.

Parity pins (what checks the oracle against something other than itself)
live in ``tests/test_oracle_*.py``.  Every function here is pinned; none is
"parity unpinned".

Modules:
  codecs  - e4m3fn, e2m1, e8m0, bf16 element codecs
  quant   - MXFP8 / NVFP4 block quantisers (activations and weights)
  moe     - routing, permutation, the layer (per-token loop and
            expert-grouped forms)
"""
