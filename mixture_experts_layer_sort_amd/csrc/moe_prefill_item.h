// The prefill-shaped grouped-GEMM work item, shared by the stage kernel
// (moe_prefill.hip) and the fused single-launch kernel.
#pragma once

#include "moe_gemm_item.h"

namespace moe {

constexpr int kPfRows = 128;          // routed rows per item
constexpr int kPfSlots = 8 * 2 * 64;  // 16-byte slots per operand per stage: [8 tiles][2 chunks][64 lanes]

// Staging registers and LDS slots use plain vector types: copies of HIP's
// uint4 (a struct) keep the staging registers in private memory.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Global data of one K step held in registers between the load and the LDS store.
template <int DT>
struct PfRegs {
  u32x4_t a[DT == DT_BF16 ? 4 : 2];  // BF16: 4 slots of 16 B; MXFP8: 2 lane-slots of 16 fp8; NVFP4: 2 x 8 B in [0], [1]
  uint32_t as[2][DT == DT_NVFP4 ? 2 : 1];
  u32x4_t b[4];
};

// One prefill work item (see the kernel file for the decomposition).  `w`
// numbers items expert-major, then n-tile, m-tile fastest; `cum` holds the
// per-expert 128-row m-tile prefix from build_schedule.  `lds` is the block's
// two-stage operand buffer.  Returns the item's expert; ends with the block's
// LDS free for reuse.
template <int DT, bool G13>
__device__ __forceinline__ int prefill_item(const GemmArgs& a, long long w, const int* cum,
                                            u32x4_t (*lds)[2][kPfSlots]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wm = wv >> 1, wn = wv & 1;
  const int NB = a.G / 2;  // n-tiles of two row groups (G is even for supported shapes)
  const int KS = a.KG * 2;  // K steps of 64
  const size_t tcode = tile_code_bytes(DT), tscale = tile_scale_bytes(DT);
  const int e = find_expert(cum, a.E, (int)(w / NB));
  const int mts = cum[e + 1] - cum[e];
  const long long local = w - (long long)cum[e] * NB;
  const int nt = (int)(local / mts), mt = (int)(local % mts);
  const int r0 = a.offsets[e] + mt * kPfRows, r_end = a.offsets[e + 1];

  // B slots of this thread: slot = tid + 256 i -> subtile s, chunk c, lane (j, q)
  int brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = tid + 256 * i, s = slot >> 7, l = slot & 63;
    const int r = r0 + 16 * s + (l & 15);
    brow[i] = r < r_end ? (G13 ? a.sorted_pairs[r] / a.k : r) : -1;
  }
  // weight tile of slot-tile t (0..7): row group 2*nt + t/4, tile t%4
  auto tile_index = [&](int t, int kg) -> size_t {
    return ((size_t)(e * a.G + 2 * nt + (t >> 2)) * a.KG + kg) * 4 + (t & 3);
  };

  auto gload = [&](PfRegs<DT>& R, int step) {
    const int kg = step >> 1, h = step & 1;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = tid + 256 * i, t = slot >> 7, within = slot & 127;
        R.a[i] = *reinterpret_cast<const u32x4_t*>(a.wcodes + tile_index(t, kg) * tcode + h * 2048 + within * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int slot = tid + 256 * i, t = slot >> 6, l = slot & 63;
        const size_t ti = tile_index(t, kg);
        if constexpr (DT == DT_MXFP8) {
          R.a[i] = *reinterpret_cast<const u32x4_t*>(a.wcodes + ti * tcode + h * 1024 + l * 16);
          R.as[i][0] = *reinterpret_cast<const uint32_t*>(a.wscales + ti * tscale + (l & 15) * 4);
        } else {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(a.wcodes + ti * tcode + l * 16 + 8 * h);
          R.a[i] = u32x4_t{v[0], v[1], 0u, 0u};
          const u32x2_t sv = *reinterpret_cast<const u32x2_t*>(a.wscales + ti * tscale + (l & 15) * 8);
          R.as[i][0] = sv[0];
          R.as[i][1] = sv[1];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = tid + 256 * i, c = (slot >> 6) & 1, q = (slot & 63) >> 4;
      R.b[i] = brow[i] >= 0 ? *reinterpret_cast<const u32x4_t*>(
                                  a.act + ((size_t)brow[i] * a.K + step * 64 + 32 * c + 8 * q) * 2)
                            : u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  auto sstore = [&](const PfRegs<DT>& R, int buf, int step) {
    u32x4_t* A = lds[buf][0];
    u32x4_t* B = lds[buf][1];
    const int h = step & 1;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) A[tid + 256 * i] = R.a[i];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int slot = tid + 256 * i, t = slot >> 6, l = slot & 63, q = l >> 4;
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // chunk 2h + j of this kgroup -> LDS chunk j
          const int c = 2 * h + j;
          if constexpr (DT == DT_MXFP8) {
            const uint32_t lo = R.a[i][2 * j], hi = R.a[i][2 * j + 1];
            A[t * 128 + j * 64 + l] = (u32x4_t)mxfp8_dequant8(lo, hi, (R.as[i][0] >> (8 * c)) & 0xFF);
          } else {
            const int sb = 2 * c + (q >> 1);
            const uint32_t sw = sb < 4 ? R.as[i][0] : R.as[i][1];
            A[t * 128 + j * 64 + l] = (u32x4_t)nvfp4_dequant8(R.a[i][j], (sw >> (8 * (sb & 3))) & 0xFF);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) B[tid + 256 * i] = R.b[i];
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  {
    PfRegs<DT> R0;
    gload(R0, 0);
    sstore(R0, 0, 0);
  }
  __syncthreads();
  for (int step = 0; step < KS; ++step) {
    const int buf = step & 1;
    PfRegs<DT> R{};  // the next step's data, live only within this iteration
    if (step + 1 < KS) gload(R, step + 1);
    const u32x4_t* A = lds[buf][0];
    const u32x4_t* B = lds[buf][1];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4_t af[4], bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = A[(4 * wn + t) * 128 + c * 64 + lane];
#pragma unroll
      for (int s = 0; s < 4; ++s) bf[s] = B[(4 * wm + s) * 128 + c * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (DT == DT_NVFP4)
            acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16((f16x8_t)af[t], (f16x8_t)bf[s], acc[t][s], 0, 0, 0);
          else
            acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)af[t], (bf16x8_t)bf[s], acc[t][s], 0, 0, 0);
        }
    }
    if (step + 1 < KS) sstore(R, buf ^ 1, step + 1);
    __syncthreads();
  }
  gemm_epilogue<DT, 4, G13>(a, acc, r0 + 64 * wm, r_end, 2 * nt + wn, e, lane);
  return e;
}

}  // namespace moe
