// Prefill-shaped grouped GEMMs: many routed rows per expert, so weight tiles
// are reused across tokens instead of being streamed once.  The work item
// (256 weight rows x 128 routed rows, weights streamed into registers,
// tokens through a 3-stage direct-to-LDS ring) is in moe_prefill_item.h.
// The grid is persistent, derives the item map from `offsets` on the device
// and walks items in XCD-contiguous order.  The epilogue (SwiGLU +
// requantisation, or y rows) is the decode kernel's.
#include "moe_prefill_fp8.h"
#include "moe_prefill_item.h"

namespace moe {

constexpr int kPfThreads = 2 * kGemmThreads;  // 8 waves: 4 row groups x 2 token halves

// Routed rows per item: 256 for the down GEMM of LDS-staged (MXFP8) weights
// (measured 7 % faster than 128: half the weight loads per flop), else 128
// (the gate/up epilogue and register-staged weights leave no registers for
// a 64 x 128 wave tile; at 256 rows the MXFP8 gate/up GEMM spills and runs
// 4 % slower).
template <int DT, bool G13>
constexpr int pf_stage_rows() { return pf_alds<DT>() && !G13 ? kPfRowsStage : kPfRows; }

template <int DT, bool G13>
__global__ __launch_bounds__(kPfThreads) void gemm_prefill_kernel(GemmArgs a) {
  constexpr int ROWS = pf_stage_rows<DT, G13>();
  __shared__ int cum[1025];
  __shared__ int wsum[4];
  const auto st = pf_make_stages<DT, ROWS>();
  const int total_mt = build_schedule(a.offsets, a.E, ROWS, cum, wsum);
  const int NB = (a.G + kPfGroups - 1) / kPfGroups;
  const long long total = (long long)total_mt * NB;
  if constexpr (G13) {
    for (long long n = 0; n * gridDim.x < total; ++n) {
      const long long w = pf_round_item(n, total, NB, a.balance);
      if (w >= 0) prefill_item<DT, G13, 2, ROWS, true>(a, w, cum, st);
    }
  } else {
    for (long long n = 0; n * gridDim.x < total; ++n) {
      const long long w = n * gridDim.x + pf_chunk_slot(n, a.balance);
      if (w < total) prefill_item<DT, G13, 2, ROWS>(a, w, cum, st);
    }
  }
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

// MXFP8 layers: one 4-wave block per compute unit (256 accumulators per lane)
template <bool G13>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_f8_kernel(GemmArgs a) {
  __shared__ int cum[1025];
  __shared__ int wsum[4];
  const F8Stages st = f8_make_stages();
  const int total_mt = build_schedule(a.offsets, a.E, kF8Rows, cum, wsum);
  const long long total = (long long)total_mt * ((a.G + kPfGroups - 1) / kPfGroups);
  for (long long n = 0; n * gridDim.x < total; ++n) {
    const long long w = n * gridDim.x + pf_chunk_slot(n, a.balance);
    if (w < total) f8_item<G13>(a, w, cum, st);
  }
}

static const void* prefill_f8_ptr(bool g13) {
  (void)g13;  // the down GEMM only
  return reinterpret_cast<const void*>(gemm_f8_kernel<false>);
}

int prefill_f8_blocks_per_cu(bool g13) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_f8_ptr(g13), kGemmThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

int prefill_balance(bool g13, int balance, int G, int grid) {
  const int NB = (G + kPfGroups - 1) / kPfGroups;
  return balance == 3 && (!g13 || NB % 8 != 0 || grid % 8 != 0) ? 0 : balance;
}

hipError_t launch_prefill_f8(bool g13, const GemmArgs& a, int grid, hipStream_t s) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return hipLaunchKernel(prefill_f8_ptr(g13), dim3(grid), dim3(kGemmThreads), args, 0, s);
}

int prefill_blocks_per_cu(int dt, bool g13) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_ptr(dt, g13), kPfThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

hipError_t launch_prefill(int dt, bool g13, const GemmArgs& a, int grid, hipStream_t s) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return hipLaunchKernel(prefill_ptr(dt, g13), dim3(grid), dim3(kPfThreads), args, 0, s);
}

}  // namespace moe
