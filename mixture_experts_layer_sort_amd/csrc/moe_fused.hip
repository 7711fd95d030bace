// The whole layer in one cooperative launch (moe_forward): one b12x-style
// call that routes, dispatches, runs the gate/up GEMM + SwiGLU, the down GEMM
// and the reduction [vLLM PR 40082 report, "Implementation" item 1].
//
// Phases of the persistent grid (all blocks co-resident; cooperative launch):
//   1. route every token (one wave per token) and quantise x (grid-stride)
//      -- grid barrier --
//   2. block 0 sorts the pairs by expert (counting sort in LDS)
//      -- grid barrier --
//   3. the gate/up items, -- grid barrier --, the down items (default), or
//      (MOE_FUSED_GEMM_BARRIER=0) every gate/up item then every down item,
//      where a finished gate/up item bumps its expert's counter (release) and
//      a down item of expert e waits for all of e's gate/up items (acquire).
//      Items are dealt in index order, so a block only ever waits on items
//      that precede its own: with all blocks resident this cannot deadlock.
//      Measured on MI355X the per-item release/acquire costs more than the
//      barrier it saves, hence the default.
//      -- grid barrier --
//   4. combine (slot order, deterministic)
// Every spin-wait is bounded: on timeout it sets an error word and moves on
// (garbage output, never a hang).  The last block out resets every
// synchronisation word to zero for the next launch.
#include "moe_gemm_item.h"
#include "moe_prefill_fp8.h"
#include "moe_prefill_item.h"
#include "moe_stages.h"

namespace moe {

struct FusedArgs {
  GemmArgs g13, g2;
  const float* logits;
  const uint16_t* x;
  uint16_t* out;
  int* ids;
  float* wts;
  int* offsets;
  int* sorted_pairs;
  int* pair_pos;
  uint8_t* xq;
  uint8_t* xq_scales;
  uint16_t* xq_deq;
  uint16_t* y;
  unsigned* sync;  // [0] barrier arrivals, [1] exits, [2] timeout flag, [kSyncHeader + e] gate/up items done
  int quant_x, T, E, H, I, k;
};

constexpr unsigned kSpinLimit = 1u << 22;  // ~10^8-10^9 cycles with the sleep below

// Poll with relaxed device-scope loads (no cache invalidation per poll), then
// one acquire fence once the count is reached.
__device__ __forceinline__ void spin_until_geq(unsigned* p, unsigned target, unsigned* timeout_flag) {
  unsigned n = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++n > kSpinLimit) {
      __hip_atomic_store(timeout_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

#ifndef MOE_FUSED_GEMM_BARRIER  // 1: grid barrier between the GEMMs instead of per-expert counters
#define MOE_FUSED_GEMM_BARRIER 1
#endif

// Monotonic grid barrier: the n-th barrier of a launch waits for n * gridDim.x arrivals.
__device__ __forceinline__ void grid_barrier(unsigned* sync, unsigned target) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    spin_until_geq(&sync[0], target, &sync[2]);
  }
  __syncthreads();
}

// LDS of one block, reused phase by phase: the permutation's histograms, then
// the decode items' cross-wave reduction.  (Prefill items keep their token
// stages in LDS objects of their own.)  V is the GEMM variant: 0 / 1 decode
// items of 16 / 32 rows, 2 prefill items, 3 prefill items of MXFP8 layers on
// the fp8 matrix instruction.
template <int V>
constexpr size_t fused_lds_bytes() {
  constexpr size_t perm = sizeof(int) * permute_lds_ints<kGemmThreads / 64>();
  constexpr size_t gemm = V >= 2 ? 0 : sizeof(f32x4_t) * 3 * 4 * (V + 1) * 64;
  return perm > gemm ? perm : gemm;
}

// A prefill item of the single-launch kernel (128 rows, one wave per row group).
template <int DT>
__device__ __forceinline__ int fused_prefill_item(const GemmArgs& g, bool g13, long long w, const int* cum) {
  const auto st = pf_make_stages<DT, kPfRows>();
  return g13 ? prefill_item<DT, true, 1, kPfRows>(g, w, cum, st) : prefill_item<DT, false, 1, kPfRows>(g, w, cum, st);
}

// An fp8 down item of the single-launch kernel; its token stages reuse the
// LDS of the prefill items' stages (the two GEMM phases are separated by a
// grid barrier).
template <int DT>
__device__ __forceinline__ int fused_f8_down_item(const GemmArgs& g, long long w, const int* cum) {
  static_assert(pf_stages<DT, kPfRows>() >= kF8Stages && pf_stage_slots<DT, kPfRows>() >= kF8StageSlots,
                "fp8 stages fit the prefill stages");
  const auto st = pf_make_stages<DT, kPfRows>();
  F8Stages st8;
  for (int i = 0; i < kF8Stages; ++i) st8.s[i] = reinterpret_cast<u32x4_t(*)[kF8StageSlots]>(st.s[i]);
  return f8_item<false>(g, w, cum, st8);
}

// Waves per SIMD the register allocation may fall to: the fp8 items keep 256
// accumulators per lane and need one wave per SIMD.
template <int V>
constexpr int fused_max_waves() { return V == 3 ? 1 : 8; }


// The single-launch kernel's x quantisation and permutation (one block, LDS
// from the kernel's dynamic shared memory) stay called functions: inlined,
// they push the MXFP8 prefill instance of that kernel further into scratch
// memory.
template <int DT>
__device__ __noinline__ void fused_quantize_x(const uint16_t* x, long long n_elem, uint8_t* codes, uint8_t* scales,
                                              uint16_t* deq, long long gtid, long long gstride) {
  quantize_x_blocks<DT>(x, n_elem, codes, scales, deq, gtid, gstride);
}

__device__ __noinline__ void fused_permute(const int* ids, int P, int E, int* offsets, int* sorted_pairs,
                                           int* pair_pos, int* lds) {
  permute_block<kGemmThreads / 64>(ids, P, E, offsets, sorted_pairs, pair_pos, reinterpret_cast<int(*)[1024]>(lds),
                                   lds + (kGemmThreads / 64) * 1024);
}

template <int DT, int V>
__global__ __launch_bounds__(kGemmThreads)
void fused_kernel(FusedArgs a) {
  constexpr int NT = V >= 2 ? 1 : V + 1;  // decode items: token sub-tiles of 16
  constexpr int MT = V >= 2 ? kPfRows : kDecodeMT;
  __shared__ int cum[1025];
  __shared__ int pcum[V == 0 ? 1025 : 1];
  __shared__ int wsum[4];
  __shared__ __align__(16) unsigned char smem[fused_lds_bytes<V>()];
  const unsigned G = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const long long gtid = (long long)blockIdx.x * kGemmThreads + tid, gstride = (long long)G * kGemmThreads;
  unsigned* done13 = a.sync + kSyncHeader;

  // 1. routing (one wave per token) and x quantisation
  for (int t = (int)(gtid >> 6); t < a.T; t += (int)(gstride >> 6)) route_token(a.logits, t, a.E, a.k, a.ids, a.wts, lane);
  if (a.quant_x) fused_quantize_x<DT>(a.x, (long long)a.T * a.H, a.xq, a.xq_scales, a.xq_deq, gtid, gstride);
  grid_barrier(a.sync, G);

  // 2. permutation
  if (blockIdx.x == 0)
    fused_permute(a.ids, a.T * a.k, a.E, a.offsets, a.sorted_pairs, a.pair_pos, reinterpret_cast<int*>(smem));
  grid_barrier(a.sync, 2 * G);

  // 3. the two grouped GEMMs
  // items per m-tile: one per 64-row weight group (decode) or per 4 groups (prefill)
  const int per13 = V >= 2 ? (a.g13.G + kPfGroups - 1) / kPfGroups : a.g13.G;
  const int per2 = V >= 2 ? (a.g2.G + kPfGroups - 1) / kPfGroups : a.g2.G;
  auto item = [&](const GemmArgs& g, bool g13, long long w, int e = -1) __attribute__((always_inline)) -> int {
    if constexpr (V == 3) {
      // gate/up items on the 16-bit path, down items on the fp8 instruction (256-row m-tiles)
      return g13 ? fused_prefill_item<DT>(g, true, w, cum) : fused_f8_down_item<DT>(g, w, cum);
    } else if constexpr (V == 2) {
      return fused_prefill_item<DT>(g, g13, w, cum);
    } else {
      auto* red = reinterpret_cast<f32x4_t(*)[4 * NT][64]>(smem);
      return g13 ? gemm_item<DT, NT, true>(g, w, cum, red, e) : gemm_item<DT, NT, false>(g, w, cum, red, e);
    }
  };
  int total_pairs = 0;
  const int total_mt =
      V >= 2 ? build_schedule(a.offsets, a.E, MT, cum, wsum) : build_decode_schedule<NT>(a.offsets, a.E, cum, pcum, wsum, total_pairs);
  const long long n13 = (long long)total_mt * per13;
  long long n2 = (long long)total_mt * per2;
  const int lb = V >= 2 ? xcd_logical_block() : (int)blockIdx.x;
  // decode items: the blocks of a compute unit take turns at the top issue
  // priority, as in the stage kernels (later-placed blocks otherwise lag)
  int turn = (int)(blockIdx.x >> 8);
  // decode items of 17-32 rows (NT = 1) take twice as long: the stage
  // kernels' execution order (decode_item_at) keeps the blocks balanced
  auto run_items = [&](const GemmArgs& g, bool g13, long long n) __attribute__((always_inline)) {
    const long long P = (long long)total_pairs * g.G, rp = min(n % (long long)G, n - P);
    for (long long x = lb; x < n; x += G, ++turn) {
      if constexpr (V < 2) set_wave_priority(turn & 3);
      if (total_pairs > 0) {
        int e;
        const long long w = decode_item_at(x, rp, P, g, cum, pcum, e);
        item(g, g13, w, e);
      } else {
        item(g, g13, x);
      }
    }
  };
  if constexpr (MOE_FUSED_GEMM_BARRIER) {
    run_items(a.g13, true, n13);
    if constexpr (V == 3) {  // the fp8 down items' m-tiles of 256 rows
      __syncthreads();
      n2 = (long long)build_schedule(a.offsets, a.E, kF8Rows, cum, wsum) * per2;
    }
    grid_barrier(a.sync, 3 * G);
    run_items(a.g2, false, n2);
    set_wave_priority(0);
    grid_barrier(a.sync, 4 * G);
  } else {
    static_assert(V != 3, "the fp8 down items need the grid barrier between the GEMMs");
    for (long long w = lb; w < n13 + n2; w += G) {
      if (w < n13) {
        const int e = item(a.g13, true, w);
        if (tid == 0) __hip_atomic_fetch_add(&done13[e], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const long long w2 = w - n13;
        const int e = find_expert(cum, a.E, (int)(w2 / per2));
        if (tid == 0) spin_until_geq(&done13[e], (unsigned)((cum[e + 1] - cum[e]) * per13), &a.sync[2]);
        __syncthreads();
        item(a.g2, false, w2);
      }
    }
    grid_barrier(a.sync, 3 * G);
  }

  // 4. combine
  combine_range(a.y, a.wts, a.T, a.H, a.k, a.out, gtid, gstride);

  // the last block out clears the synchronisation words (the timeout flag stays)
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&a.sync[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {
      for (int e = 0; e < a.E; ++e) __hip_atomic_store(&done13[e], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

template <int DT>
static const void* fused_fn(int v) {
  if (v == 0) return reinterpret_cast<const void*>(fused_kernel<DT, 0>);
  if (v == 1) return reinterpret_cast<const void*>(fused_kernel<DT, 1>);
  if (v == 3) return reinterpret_cast<const void*>(fused_kernel<DT_MXFP8, 3>);
  return reinterpret_cast<const void*>(fused_kernel<DT, 2>);
}

static const void* fused_ptr(int dt, int v) {
  if (dt == DT_BF16) return fused_fn<DT_BF16>(v);
  if (dt == DT_MXFP8) return fused_fn<DT_MXFP8>(v);
  return fused_fn<DT_NVFP4>(v);
}

int fused_blocks_per_cu(int dt, int v) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_ptr(dt, v), kGemmThreads, 0) != hipSuccess || n < 1)
    return 0;
  return n;
}

hipError_t launch_fused(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                        const float* logits, const uint16_t* x, uint16_t* out, int* ids, float* wts, uint8_t* ws,
                        size_t ws_bytes, int max_tokens, int grid, hipStream_t s, float limit) {
  const WorkspaceLayout W = workspace_layout(dt, E, H, I, k, max_tokens);
  const PackedLayout L = packed_layout(dt, E, H, I, gated);
  FusedArgs f;
  f.logits = logits;
  f.x = x;
  f.out = out;
  f.ids = ids;
  f.wts = wts;
  f.offsets = reinterpret_cast<int*>(ws + W.offsets);
  f.sorted_pairs = reinterpret_cast<int*>(ws + W.sorted_pairs);
  f.pair_pos = reinterpret_cast<int*>(ws + W.pair_pos);
  uint8_t* xq = act_dt(dt) == DT_BF16 ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(x)) : ws + W.xq;
  uint8_t* hq = ws + W.hq;
  f.xq = xq;
  f.xq_scales = xq + act_scale_offset(dt, T, H);
  f.xq_deq = reinterpret_cast<uint16_t*>(xq + act_dequant_offset(dt, T, H));
  f.y = reinterpret_cast<uint16_t*>(ws + W.y);
  f.sync = reinterpret_cast<unsigned*>(ws + W.sync);
  f.quant_x = act_dt(dt) != DT_BF16;
  f.T = T;
  f.E = E;
  f.H = H;
  f.I = I;
  f.k = k;
  GemmArgs& g = f.g13;
  g.wcodes = packed + L.w13_codes;
  g.wscales = packed + L.w13_scales;
  g.walpha = reinterpret_cast<const float*>(packed + L.w13_alpha);
  g.offsets = f.offsets;
  g.sorted_pairs = f.sorted_pairs;
  g.act = xq + act_operand_offset(dt, T, H);
  g.out = hq;
  g.out_scales = hq + act_scale_offset(dt, T * k, I);
  g.out_deq = reinterpret_cast<uint16_t*>(hq + act_dequant_offset(dt, T * k, I));
  g.act_bf16 = dt == DT_BF16_MXFP8;
  g.gated = gated;
  g.E = E; g.K = H; g.G = L.G13; g.KG = L.KG13; g.k = k; g.n_out = I;
  GemmArgs& h = f.g2;
  h.wcodes = packed + L.w2_codes;
  h.wscales = packed + L.w2_scales;
  h.walpha = reinterpret_cast<const float*>(packed + L.w2_alpha);
  h.offsets = f.offsets;
  h.sorted_pairs = f.sorted_pairs;
  h.act = hq + act_operand_offset(dt, T * k, I);
  h.out = reinterpret_cast<uint8_t*>(f.y);
  h.out_scales = nullptr;
  h.out_deq = nullptr;
  h.act_bf16 = dt == DT_BF16_MXFP8;
  h.gated = gated;
  h.E = E; h.K = I; h.G = L.G2; h.KG = L.KG2; h.k = k; h.n_out = H;
  g.act_scales = h.act_scales = nullptr;
  g.limit = gated ? limit : 0.f;
  h.limit = 0.f;
  g.band = h.band = 0;
  g.balance = h.balance = 0;
  g.red = h.red = nullptr;
  g.wts = h.wts = nullptr;
  const int v = fused_variant(dt, T, k, E, H, I);
  if (v == 3) {  // the fp8 down items: fragment-order weights, e4m3 hq codes and e8m0 scales
    g.out_deq = nullptr;  // (hq's 16-bit copy is not read)
    h.wcodes = packed + L.w2_frag;
    h.act = hq;
    h.act_scales = hq + act_scale_offset(dt, T * k, I);
  }
  (void)ws_bytes;
  void* args[] = {&f};
  return hipLaunchCooperativeKernel(fused_ptr(weight_dt(dt), v), dim3(grid), dim3(kGemmThreads), args, 0, s);
}

hipError_t launch_zero_sync(uint8_t* ws, int dt, int E, int H, int I, int k, int max_tokens, hipStream_t s) {
  const WorkspaceLayout W = workspace_layout(dt, E, H, I, k, max_tokens);
  const int n = (int)(W.sync_bytes / 4);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, reinterpret_cast<unsigned*>(ws + W.sync),
                     n);
  return hipGetLastError();
}

}  // namespace moe
