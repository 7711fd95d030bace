// Grouped expert GEMMs (gate/up + SwiGLU + requant, and down), weight
// repacking and the top-k combine, for gfx950.
//
// GEMM work decomposition.  The pairs routed to expert e occupy sorted rows
// [offsets[e], offsets[e+1]); they are cut into m-tiles of kDecodeMT = 32 rows.
// One work item = (expert, m-tile, weight row group of 64 rows); items are
// numbered m-tile-major so neighbouring blocks share activation rows.  The
// grid is persistent (sized to the resident capacity) and each block walks
// items blockIdx.x, +gridDim.x, ...; every block derives the item -> expert
// map from `offsets` itself (a scan of per-expert m-tile counts in LDS), so
// no host synchronisation or extra launch is needed.  Inside a block the 4
// waves split K into quarters, each streaming its slice of the 4 weight
// tiles (16 rows each) through registers into MFMAs with the weights in the
// M slot and the (<= 16*NT) routed tokens in the N slot (an item of 17-32
// rows with NT = 1 runs as two halves of two waves each), then reduce through
// LDS.  This is the decode-shaped ("swap A/B") arrangement: weight rows fill
// the matrix unit's 16-row side so a handful of tokens per expert wastes no
// weight bandwidth [MegaMoE drop workflow, §1: the NVFP4 kernel package is
// the "swapab" variant].
#include "moe_gemm_item.h"
#include "moe_stages.h"

namespace moe {

// Every block gets the same number of items, so a compute unit finishes with
// its slowest resident block.  Measured on MI355X, the blocks placed later on
// a compute unit (higher block ids: the first 256 blocks take one unit each,
// the next 256 a second slot, ...) stream ~25 % slower than the first, as the
// older waves win the issue arbitration.  Each block therefore rotates its
// waves' priority by item, starting from its slot, so the blocks of one unit
// take turns at the top priority (3-4 % faster MXFP8 / NVFP4 decode GEMMs).
// Waves per SIMD the register allocation must allow.  Four resident blocks
// per compute unit keep more weight bytes in flight for NVFP4 (its steps are
// the smallest): measured 2-3 % faster gate/up GEMMs than the three the
// compiler picks by itself; the other formats keep the compiler's choice
// (MXFP8 would spill at four).
template <int DT, int NT>
constexpr int gemm_min_waves_per_simd() { return NT == 1 ? (DT == DT_NVFP4 ? 4 : (DT == DT_MXFP8 ? 3 : 2)) : 1; }

template <int DT, int NT, bool G13>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(gemm_min_waves_per_simd<DT, NT>())))
void gemm_kernel(GemmArgs a) {
  __shared__ int cum[1025];
  __shared__ int pcum[NT == 1 ? 1025 : 1];
  __shared__ int wsum[4];
  __shared__ f32x4_t red[3][4 * NT][64];
  int total_pairs;
  const int total_mt = build_decode_schedule<NT>(a.offsets, a.E, cum, pcum, wsum, total_pairs);
  const long long total = (long long)total_mt * a.G;
  int turn = (int)(blockIdx.x >> 8);
  if (total_pairs > 0) {
    const long long P = (long long)total_pairs * a.G;
    const long long rp = min(total % gridDim.x, total - P);
    for (long long x = blockIdx.x; x < total; x += gridDim.x, ++turn) {
      set_wave_priority(turn & 3);
      int e;
      const long long w = decode_item_at(x, rp, P, a, cum, pcum, e);
      gemm_item<DT, NT, G13>(a, w, cum, red, e);
    }
  } else {
    for (long long w = blockIdx.x; w < total; w += gridDim.x, ++turn) {
      set_wave_priority(turn & 3);
      gemm_item<DT, NT, G13>(a, w, cum, red);
    }
  }
}

// ------------------------------------------------------------------ prepare (repack)

template <int DT>
__global__ void prepare_kernel(const uint8_t* __restrict__ src, const uint8_t* __restrict__ src_s, int E, int R,
                               int K, int G, int KG, int I, int w13, uint8_t* __restrict__ dst,
                               uint8_t* __restrict__ dst_s) {
  const long long n = (long long)E * G * KG * 4 * 64;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const long long tile = idx >> 6;
    const int t = (int)(tile & 3);
    long long rest = tile >> 2;
    const int kg = (int)(rest % KG);
    rest /= KG;
    const int g = (int)(rest % G);
    const int e = (int)(rest / G);
    const int i = lane & 15, q = lane >> 4;
    const int row = w13 ? (t < 2 ? 32 * g + 16 * t + i : I + 32 * g + 16 * (t - 2) + i) : 64 * g + 16 * t + i;
    const size_t rb = (size_t)e * R + row;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(dst + tile * 4096 + c * 1024 + lane * 16) =
            *reinterpret_cast<const uint4*>(src + (rb * K + kg * 128 + 32 * c + 8 * q) * 2);
    } else if constexpr (DT == DT_MXFP8) {
#pragma unroll
      for (int c = 0; c < 4; ++c)  // half c/2, bytes 8*(c%2) of the lane's 16
        *reinterpret_cast<uint2*>(dst + tile * 2048 + (c >> 1) * 1024 + lane * 16 + 8 * (c & 1)) =
            *reinterpret_cast<const uint2*>(src + rb * K + kg * 128 + 32 * c + 8 * q);
      // row i's 4 scales of this kgroup, one byte per lane
      dst_s[tile * 64 + i * 4 + q] = src_s[rb * (K / 32) + kg * 4 + q];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint32_t*>(dst + tile * 1024 + lane * 16 + 4 * c) =
            *reinterpret_cast<const uint32_t*>(src + rb * (K / 2) + kg * 64 + 16 * c + 4 * q);
      // row i's 8 scales of this kgroup, two bytes per lane
      dst_s[tile * 128 + i * 8 + 2 * q] = src_s[rb * (K / 16) + kg * 8 + 2 * q];
      dst_s[tile * 128 + i * 8 + 2 * q + 1] = src_s[rb * (K / 16) + kg * 8 + 2 * q + 1];
    }
  }
}

// MXFP8 codes in the fp8 fragment order (see moe_layout.h): one thread per
// 16-byte unit (expert, row group, 64-K step, fragment, half, lane).  Used for
// W2 (w13 = 0); the SwiGLU W13 order (w13 = 1) is kept for completeness.
__global__ void prepare_frag_kernel(const uint8_t* __restrict__ src, int E, int R, int K, int G, int I, int w13,
                                    uint8_t* __restrict__ dst) {
  const int KS = K / 64;
  const long long n = (long long)E * G * KS * 4 * 64;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(idx & 63), q = (int)((idx >> 6) & 1), f = (int)((idx >> 7) & 1);
    long long rest = idx >> 8;
    const int s = (int)(rest % KS);
    rest /= KS;
    const int g = (int)(rest % G);
    const int e = (int)(rest / G);
    const int m = l & 31, h = l >> 5;
    // group row 32 f + m: gate rows then the matching up rows (SwiGLU W13), else 64 consecutive rows
    const int row = w13 ? (f == 0 ? 32 * g + m : I + 32 * g + m) : 64 * g + 32 * f + m;
    *reinterpret_cast<uint4*>(dst + idx * 16) =
        *reinterpret_cast<const uint4*>(src + ((size_t)e * R + row) * K + 64 * s + 32 * q + 16 * h);
  }
}

__global__ void copy_f32_kernel(const float* __restrict__ s, float* __restrict__ d, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = s[i];
}

// ------------------------------------------------------------------ combine
__global__ void combine_kernel(const uint16_t* __restrict__ y, const float* __restrict__ wts, int T, int H, int k,
                               uint16_t* __restrict__ out) {
  combine_range(y, wts, T, H, k, out, blockIdx.x * (long long)blockDim.x + threadIdx.x,
                (long long)gridDim.x * blockDim.x);
}

// ------------------------------------------------------------------ launchers

template <int DT, int NT, bool G13>
static hipError_t launch_gemm_t(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<DT, NT, G13>), dim3(grid), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

template <bool G13>
static hipError_t dispatch_gemm(int dt, int nt, const GemmArgs& a, int grid, hipStream_t s) {
  if (dt == DT_BF16) return nt == 1 ? launch_gemm_t<DT_BF16, 1, G13>(a, grid, s) : launch_gemm_t<DT_BF16, 2, G13>(a, grid, s);
  if (dt == DT_MXFP8) return nt == 1 ? launch_gemm_t<DT_MXFP8, 1, G13>(a, grid, s) : launch_gemm_t<DT_MXFP8, 2, G13>(a, grid, s);
  return nt == 1 ? launch_gemm_t<DT_NVFP4, 1, G13>(a, grid, s) : launch_gemm_t<DT_NVFP4, 2, G13>(a, grid, s);
}


int gemm_blocks_per_cu(int dt, bool g13, int nt) {
  int n = 0;
  hipError_t err = hipSuccess;
#define MOE_OCC(D, N, G)                                                                                  \
  if (dt == D && nt == N && g13 == G)                                                                     \
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(gemm_kernel<D, N, G>), \
                                                       kGemmThreads, 0);
  MOE_OCC(DT_BF16, 1, true) MOE_OCC(DT_BF16, 2, true) MOE_OCC(DT_BF16, 1, false) MOE_OCC(DT_BF16, 2, false)
  MOE_OCC(DT_MXFP8, 1, true) MOE_OCC(DT_MXFP8, 2, true) MOE_OCC(DT_MXFP8, 1, false) MOE_OCC(DT_MXFP8, 2, false)
  MOE_OCC(DT_NVFP4, 1, true) MOE_OCC(DT_NVFP4, 2, true) MOE_OCC(DT_NVFP4, 1, false) MOE_OCC(DT_NVFP4, 2, false)
#undef MOE_OCC
  if (err != hipSuccess || n < 1) n = 1;
  return n;
}

hipError_t launch_gemm13(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                         const int* offsets, const int* sorted_pairs, const uint8_t* xq, uint8_t* hq, int grid,
                         hipStream_t s, const GemmPlan& plan) {
  const PackedLayout L = packed_layout(dt, E, H, I, gated);
  GemmArgs a;
  a.wcodes = packed + L.w13_codes;
  a.wscales = packed + L.w13_scales;
  a.walpha = reinterpret_cast<const float*>(packed + L.w13_alpha);
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.act = xq + act_operand_offset(dt, T, H);
  a.out = hq;
  a.out_scales = hq + act_scale_offset(dt, T * k, I);
  a.out_deq = plan.skip_hq_deq ? nullptr : reinterpret_cast<uint16_t*>(hq + act_dequant_offset(dt, T * k, I));
  a.act_scales = nullptr;
  a.act_bf16 = dt == DT_BF16_MXFP8;
  a.gated = gated;
  a.limit = gated ? plan.limit : 0.f;
  a.band = plan.band;
  a.red = nullptr;
  a.wts = nullptr;
  a.E = E; a.K = H; a.G = L.G13; a.KG = L.KG13; a.k = k; a.n_out = I;
  a.balance = prefill_balance(true, plan.balance, a.G, grid);
  if (plan.variant == 2) return launch_prefill(weight_dt(dt), true, a, grid, s);
  return dispatch_gemm<true>(weight_dt(dt), plan.variant + 1, a, grid, s);
}

hipError_t launch_gemm2(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                        const int* offsets, const int* sorted_pairs, const uint8_t* hq, uint16_t* y, int grid,
                        hipStream_t s, const GemmPlan& plan) {
  const PackedLayout L = packed_layout(dt, E, H, I, gated);
  GemmArgs a;
  a.wcodes = packed + L.w2_codes;
  a.wscales = packed + L.w2_scales;
  a.walpha = reinterpret_cast<const float*>(packed + L.w2_alpha);
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.act = hq + act_operand_offset(dt, T * k, I);
  a.out = reinterpret_cast<uint8_t*>(y);
  a.out_scales = nullptr;
  a.out_deq = nullptr;
  a.act_scales = nullptr;
  a.act_bf16 = dt == DT_BF16_MXFP8;
  a.gated = gated;
  a.limit = 0.f;
  a.band = plan.band;
  a.red = plan.red;
  a.wts = plan.wts;
  a.E = E; a.K = I; a.G = L.G2; a.KG = L.KG2; a.k = k; a.n_out = H;
  a.balance = prefill_balance(false, plan.balance, a.G, grid);
  if (plan.variant == 2 && plan.down_fp8 && has_fp8_gemm(dt)) {
    a.wcodes = packed + L.w2_frag;
    a.act = hq;  // e4m3 codes
    a.act_scales = hq + act_scale_offset(dt, T * k, I);
    return launch_prefill_f8(false, a, grid, s);
  }
  if (plan.variant == 2) return launch_prefill(weight_dt(dt), false, a, grid, s);
  return dispatch_gemm<false>(weight_dt(dt), plan.variant + 1, a, grid, s);
}

__global__ void zero_f32_kernel(float* __restrict__ p, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n / 4; i += (long long)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ acc, uint16_t* __restrict__ out, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n / 4; i += (long long)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(acc)[i];
    reinterpret_cast<uint2*>(out)[i] = make_uint2(f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                                                  f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
  }
}

// (n is a multiple of 4: rows of H % 128 == 0 values)
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s) {
  const int blocks = (int)std::min((n / 4 + 255) / 256, 65536LL);
  hipLaunchKernelGGL(zero_f32_kernel, dim3(std::max(blocks, 1)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* acc, uint16_t* out, long long n, hipStream_t s) {
  const int blocks = (int)std::min((n / 4 + 255) / 256, 65536LL);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(std::max(blocks, 1)), dim3(256), 0, s, acc, out, n);
  return hipGetLastError();
}

hipError_t launch_dense_prepare(int N, int K, const uint8_t* codes, const uint8_t* scales, const float* alpha,
                                uint8_t* packed, hipStream_t s) {
  const DenseLayout D = dense_layout(N, K);
  const long long n = (long long)D.G * D.KG * 4 * 64;
  const int threads = 256;
  const int blocks = (int)std::min((n + threads - 1) / threads, 1LL << 20);
  // the W2 arrangement: 64-row groups, rows 64 g + 16 t + i
  hipLaunchKernelGGL(prepare_kernel<DT_NVFP4>, dim3(blocks), dim3(threads), 0, s, codes, scales, 1, N, K, D.G, D.KG,
                     K, 0, packed + D.codes, packed + D.scales);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(1), dim3(64), 0, s, alpha, reinterpret_cast<float*>(packed + D.alpha), 1);
  return hipGetLastError();
}

hipError_t launch_dense_gemm(int M, int N, int K, const uint8_t* packed, const int* offsets, const int* rows,
                             const uint8_t* xq, uint16_t* out, int grid, hipStream_t s) {
  const DenseLayout D = dense_layout(N, K);
  GemmArgs a;
  a.wcodes = packed + D.codes;
  a.wscales = packed + D.scales;
  a.walpha = reinterpret_cast<const float*>(packed + D.alpha);
  a.offsets = offsets;
  a.sorted_pairs = rows;
  a.act = xq + act_operand_offset(DT_NVFP4, M, K);
  a.act_scales = nullptr;
  a.out = reinterpret_cast<uint8_t*>(out);
  a.out_scales = nullptr;
  a.out_deq = nullptr;
  a.act_bf16 = 0;
  a.gated = 0;
  a.limit = 0.f;
  a.band = 0;
  a.red = nullptr;
  a.wts = nullptr;
  a.balance = 0;
  a.E = 1; a.K = K; a.G = D.G; a.KG = D.KG; a.k = 1; a.n_out = N;
  if (gemm_prefill(M, 1, 1)) return launch_prefill(DT_NVFP4, false, a, grid, s);
  return dispatch_gemm<false>(DT_NVFP4, gemm_nt(M, 1, 1), a, grid, s);
}

hipError_t launch_prepare(int dt, bool gated, int E, int H, int I, const uint8_t* w13, const uint8_t* w13s,
                          const float* w13a, const uint8_t* w2, const uint8_t* w2s, const float* w2a, uint8_t* packed,
                          hipStream_t s) {
  const PackedLayout L = packed_layout(dt, E, H, I, gated);
  const int layer_dt = dt;
  const int threads = 256;
  auto blocks = [&](long long n) { return (int)std::min((n + threads - 1) / threads, 1LL << 20); };
  long long n13 = (long long)E * L.G13 * L.KG13 * 4 * 64, n2 = (long long)E * L.G2 * L.KG2 * 4 * 64;
#define MOE_PREP(D)                                                                                              \
  hipLaunchKernelGGL(prepare_kernel<D>, dim3(blocks(n13)), dim3(threads), 0, s, w13, w13s, E, gated ? 2 * I : I, \
                     H, L.G13, L.KG13, I, gated ? 1 : 0, packed + L.w13_codes, packed + L.w13_scales);         \
  hipLaunchKernelGGL(prepare_kernel<D>, dim3(blocks(n2)), dim3(threads), 0, s, w2, w2s, E, H, I, L.G2, L.KG2, I, \
                     0, packed + L.w2_codes, packed + L.w2_scales);
  dt = weight_dt(dt);
  if (dt == DT_BF16) { MOE_PREP(DT_BF16) }
  else if (dt == DT_MXFP8) { MOE_PREP(DT_MXFP8) }
  else {
    MOE_PREP(DT_NVFP4)
    hipLaunchKernelGGL(copy_f32_kernel, dim3((E + 255) / 256), dim3(256), 0, s, w13a,
                       reinterpret_cast<float*>(packed + L.w13_alpha), E);
    hipLaunchKernelGGL(copy_f32_kernel, dim3((E + 255) / 256), dim3(256), 0, s, w2a,
                       reinterpret_cast<float*>(packed + L.w2_alpha), E);
  }
#undef MOE_PREP
  if (has_fp8_gemm(layer_dt)) {
    const long long f2 = (long long)E * L.G2 * (I / 64) * 256;
    hipLaunchKernelGGL(prepare_frag_kernel, dim3(blocks(f2)), dim3(threads), 0, s, w2, E, H, I, L.G2, I, 0,
                       packed + L.w2_frag);
  }
  return hipGetLastError();
}

hipError_t launch_combine(int T, int H, int k, const uint16_t* y, const float* wts, uint16_t* out, hipStream_t s) {
  const long long n = (long long)T * H / 8;
  const int threads = 256;
  int blocks = (int)std::min((n + threads - 1) / threads, 65536LL);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(threads), 0, s, y, wts, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
