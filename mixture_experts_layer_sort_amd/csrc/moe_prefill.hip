// Prefill-shaped grouped GEMMs: many routed rows per expert, so weight tiles
// are reused across tokens through LDS instead of being streamed once.
//
// Work item = (expert, 128-row m-tile of its sorted rows, n-tile of two
// weight row groups = 128 weight rows).  Items are numbered expert-major,
// then n-tile, with the m-tile fastest, so consecutive items (and blocks)
// share the same weight tiles in L2 / the Infinity Cache.  The grid is
// persistent and derives the item map from `offsets` on the device.
//
// A block of 4 waves computes the 128 x 128 item as a 2 x 2 grid of 64 x 64
// wave tiles (16 MFMAs of 16x16x32 per 32-wide K chunk).  K advances in steps
// of 64 through two LDS buffers: while the waves compute step s from one
// buffer, every thread already holds step s+1's global data in registers and
// writes it (converted to bf16 / fp16) into the other buffer afterwards; one
// barrier per step.  Both operands sit in LDS in the matrix instruction's
// per-lane order (the packed weight layout is already in that order), so each
// lane's fragment is one conflict-free 16-byte LDS read.  The epilogue (SwiGLU
// + requantisation, or y rows) is the decode kernel's.
#include "moe_prefill_item.h"

namespace moe {

template <int DT, bool G13>
__global__ __launch_bounds__(kGemmThreads) void gemm_prefill_kernel(GemmArgs a) {
  __shared__ int cum[1025];
  __shared__ int wsum[4];
  __shared__ u32x4_t lds[2][2][kPfSlots];  // [buffer][A weights / B tokens][slot]
  const int total_mt = build_schedule(a.offsets, a.E, kPfRows, cum, wsum);
  const long long total = (long long)total_mt * (a.G / 2);
  for (long long w = blockIdx.x; w < total; w += gridDim.x) prefill_item<DT, G13>(a, w, cum, lds);
}

template <int DT, bool G13>
static const void* prefill_fn() {
  return reinterpret_cast<const void*>(gemm_prefill_kernel<DT, G13>);
}

static const void* prefill_ptr(int dt, bool g13) {
  if (dt == DT_BF16) return g13 ? prefill_fn<DT_BF16, true>() : prefill_fn<DT_BF16, false>();
  if (dt == DT_MXFP8) return g13 ? prefill_fn<DT_MXFP8, true>() : prefill_fn<DT_MXFP8, false>();
  return g13 ? prefill_fn<DT_NVFP4, true>() : prefill_fn<DT_NVFP4, false>();
}

int prefill_blocks_per_cu(int dt, bool g13) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_ptr(dt, g13), kGemmThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

hipError_t launch_prefill(int dt, bool g13, const GemmArgs& a, int grid, hipStream_t s) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return hipLaunchKernel(prefill_ptr(dt, g13), dim3(grid), dim3(kGemmThreads), args, 0, s);
}

}  // namespace moe
