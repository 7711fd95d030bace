// Grouped-GEMM building blocks shared by the stage kernels and the fused
// single-launch kernel (see moe_gemm.hip for the work decomposition).
#pragma once

#include "moe_kernels.h"

namespace moe {

constexpr int kGemmThreads = 256;

struct GemmArgs {
  const uint8_t* wcodes;
  const uint8_t* wscales;
  const float* walpha;
  const int* offsets;
  const int* sorted_pairs;
  const uint8_t* act;         // B operand rows, 16-bit: xq (gemm13, row = token) or hq (gemm2, row = sorted row);
                              // the fp8 prefill GEMM: their e4m3 codes
  const uint8_t* act_scales;  // the fp8 prefill GEMM: the e8m0 scales of those rows
  uint8_t* out;               // hq codes (gemm13) or y (gemm2)
  uint8_t* out_scales;        // hq scales (gemm13)
  uint16_t* out_deq;          // hq dequantised 16-bit copy (gemm13; MXFP8, NVFP4; null: not written, which
                              // only the prefill-shaped MXFP8 epilogue allows)
  int act_bf16;               // MXFP8 weights with bf16 activations: the intermediate is rounded to bf16
  int gated;                  // gate/up GEMM: 1 SwiGLU (gate/up row pairs), 0 ReLU^2 (64 W1 rows per group)
  float limit;                // SwiGLU gate/up clamp L (0: none): gate = min(gate, L), up = clamp(up, -L, L)
  int band;                   // prefill item order: token rows per band (0: the kernel's default, 1024)
  int balance;                // prefill item deal over the blocks (pf_chunk_slot)
  float* red;                 // down GEMM, in-kernel fc2 reduce: fp32 out [T, H] += wts[p] * y[p] (atomics);
                              // null: y rows are written
  const float* wts;           // the router weights of the pairs (with red)
  int E, K, G, KG, k, n_out;
};

// This wave's issue priority (0..3; s_setprio takes an immediate).
__device__ __forceinline__ void set_wave_priority(int p) {
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// Exclusive prefix over experts of count(rows of e), a 32-bit value or two
// packed into 64 bits: out(e, prefix) stores the prefix of expert e, and
// out(E, total) the total.  The first kGemmThreads threads do the scan (one
// load of the offsets, one wave scan, two barriers); a larger block only
// waits for it.  wsum holds kGemmThreads / 64 values.
template <typename V, typename CountFn, typename OutFn>
__device__ V build_prefix(const int* __restrict__ offsets, int E, CountFn count, OutFn out, V* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid >= kGemmThreads) {
    __syncthreads();
    V total = 0;
    for (int ww = 0; ww < kGemmThreads / 64; ++ww) total += wsum[ww];
    __syncthreads();
    return total;
  }
  const int per = (E + kGemmThreads - 1) / kGemmThreads;  // <= 4 (E <= 1024)
  const int e0 = tid * per;
  V cnt[4] = {0, 0, 0, 0}, local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = e0 + j;
    if (j < per && e < E) {
      cnt[j] = count(offsets[e + 1] - offsets[e]);
      local += cnt[j];
    }
  }
  V incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    V o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  V wbase = 0, total = 0;
  for (int ww = 0; ww < kGemmThreads / 64; ++ww) {
    if (ww < w) wbase += wsum[ww];
    total += wsum[ww];
  }
  V run = wbase + incl - local;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = e0 + j;
    if (j < per && e < E) {
      out(e, run);
      run += cnt[j];
    }
  }
  if (tid == 0) out(E, total);
  __syncthreads();
  return total;
}

// cum[e] = m-tiles of MT rows of experts < e (LDS); returns the total.
__device__ __forceinline__ int build_schedule(const int* __restrict__ offsets, int E, int MT, int* cum, int* wsum) {
  return build_prefix<int>(offsets, E, [MT](int c) { return (c + MT - 1) / MT; },
                           [cum](int e, int v) { cum[e] = v; }, wsum);
}

__device__ __forceinline__ int find_expert(const int* cum, int E, int mtg) {
  int lo = 0, hi = E;  // cum[lo] <= mtg < cum[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cum[mid] <= mtg) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint8_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// 8 e2m1 codes (one dword, element j in nibble j) times an e4m3 scale (one
// byte) -> 8 fp16, exactly: e2m1 (2 significant bits) x e4m3 (4 bits) fits
// fp16's 11 bits and its exponent range.  Hardware converts at scale 1 (pure
// conversion) and one packed fp16 multiply per pair.
__device__ __forceinline__ f16x8_t nvfp4_dequant8(uint32_t codes, uint32_t e4m3_byte) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 sc = __builtin_amdgcn_cvt_scalef32_f16_fp8(f16x2{}, e4m3_byte, 1.0f, 0, false);
  sc[1] = sc[0];
  f16x2 r[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc,
                __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc,
                __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc,
                __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc};
  f16x8_t o;
  __builtin_memcpy(&o, r, 16);
  return o;
}

// 8 e4m3 codes (two dwords, element j in byte j) times 2^(e - 127) (an e8m0
// scale byte) -> 8 bf16.  Exact: 4 significant bits, and the convert applies
// the power-of-two scale by exponent arithmetic.  (The gate/up GEMM does not
// use the gfx950 block-scaled fp8 matrix instruction: at K = 7168 its sums
// carry ~130x the error of fp32 accumulation of these exact bf16 products,
// measured, and flip ~70x more of the requantised intermediate codes.)
__device__ __forceinline__ bf16x8_t mxfp8_dequant8(uint32_t lo, uint32_t hi, uint32_t e8m0) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const float sc = __uint_as_float(e8m0 << 23);  // 2^(e8m0 - 127); byte 0 -> 0 (all-zero block)
  bf16x2 r[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true)};
  bf16x8_t o;
  __builtin_memcpy(&o, r, 16);
  return o;
}

// ------------------------------------------------------------------ K-slice fragments
// Raw bytes of one 128-wide K slice ("kgroup") for the 4 weight tiles of a
// work item and its NT token sub-tiles, as loaded from memory; converted and
// fed to the matrix unit by mma_kfrag.
template <int DT>
struct KW {  // words per lane per tile: codes (uint4) / scales (dwords)
  static constexpr int A = DT == DT_BF16 ? 4 : (DT == DT_MXFP8 ? 2 : 1);
  static constexpr int AS = DT == DT_NVFP4 ? 2 : 1;
};

template <int DT, int NT>
struct KFrag {
  uint4 ac[4][KW<DT>::A];
  // the 4 tiles' scale rows of the kgroup, one per lane: lane L holds tile
  // L / 16, row L % 16 (the tiles' scale blocks are contiguous); each lane
  // takes its own rows from the right lanes when it converts (one load per
  // kgroup instead of one per tile: the address unit's per-instruction cost
  // bounds the decode loads)
  uint32_t as[KW<DT>::AS];
  uint4 bc[NT][4];  // 16-bit activation operand, 4 chunks of 8
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NTLD>
__device__ __forceinline__ uint4 ld_w16(const uint8_t* p) {
  if constexpr (NTLD) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <int DT, int NT, bool G13, bool NTLD>
__device__ __forceinline__ void load_kfrag(KFrag<DT, NT>& f, const GemmArgs& a, size_t tile0, int kg,
                                           const int (&brow)[NT], int lane, int i16, int q) {
  const size_t tcode = tile_code_bytes(DT), tscale = tile_scale_bytes(DT);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint8_t* pc = a.wcodes + (tile0 + t) * tcode;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) f.ac[t][c] = ld_w16<NTLD>(pc + c * 1024 + lane * 16);
    } else if constexpr (DT == DT_MXFP8) {
      f.ac[t][0] = ld_w16<NTLD>(pc + lane * 16);
      f.ac[t][1] = ld_w16<NTLD>(pc + 1024 + lane * 16);
    } else {
      f.ac[t][0] = ld_w16<NTLD>(pc + lane * 16);
    }
  }
  if constexpr (DT == DT_MXFP8) {
    f.as[0] = *reinterpret_cast<const uint32_t*>(a.wscales + tile0 * tscale + lane * 4);
  } else if constexpr (DT == DT_NVFP4) {
    const uint2 sv = *reinterpret_cast<const uint2*>(a.wscales + tile0 * tscale + lane * 8);
    f.as[0] = sv.x;
    f.as[1] = sv.y;
  }
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    const bool ok = brow[s] >= 0;
    const uint8_t* p = a.act + ((size_t)(ok ? brow[s] : 0) * a.K + kg * 128 + 8 * q) * 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) f.bc[s][c] = ok ? *reinterpret_cast<const uint4*>(p + c * 64) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int DT, int NT>
__device__ __forceinline__ void mma_kfrag(f32x4_t (&acc)[4][NT], const KFrag<DT, NT>& f, int q) {
  // this lane's scale words of tile t (row lane % 16) from lane 16 t + lane % 16
  uint32_t st[4][KW<DT>::AS];
  if constexpr (DT != DT_BF16) {
    const int i16 = __lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int w = 0; w < KW<DT>::AS; ++w) st[t][w] = (uint32_t)__shfl((int)f.as[w], 16 * t + i16, 64);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DT == DT_NVFP4) {
        const int sb = 2 * c + (q >> 1);  // 16-block of this lane's 8 k's
        const uint32_t sw = sb < 4 ? st[t][0] : st[t][1];
        const f16x8_t A = nvfp4_dequant8(u4_word(f.ac[t][0], c), (sw >> (8 * (sb & 3))) & 0xFF);
#pragma unroll
        for (int s = 0; s < NT; ++s) {
          f16x8_t B;
          __builtin_memcpy(&B, &f.bc[s][c], 16);
          acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[t][s], 0, 0, 0);
        }
      } else {
        bf16x8_t A;
        if constexpr (DT == DT_BF16) {
          __builtin_memcpy(&A, &f.ac[t][c], 16);
        } else {
          const uint4& v = f.ac[t][c >> 1];
          A = (c & 1) ? mxfp8_dequant8(v.z, v.w, (st[t][0] >> (8 * c)) & 0xFF)
                      : mxfp8_dequant8(v.x, v.y, (st[t][0] >> (8 * c)) & 0xFF);
        }
#pragma unroll
        for (int s = 0; s < NT; ++s) {
          bf16x8_t B;
          __builtin_memcpy(&B, &f.bc[s][c], 16);
          acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t][s], 0, 0, 0);
        }
      }
    }
  }
}

// Compile-time tuning knobs of the grouped GEMMs.
#ifndef MOE_GEMM_PIPELINE  // 1: double-buffer K steps (prefetch the next while computing)
#define MOE_GEMM_PIPELINE 1
#endif
#ifndef MOE_GEMM_NTLOAD  // 1: non-temporal weight loads on the decode path
#define MOE_GEMM_NTLOAD 1
#endif
#ifndef MOE_GEMM_U_BF16  // kgroups per step, per weight format
#define MOE_GEMM_U_BF16 1
#endif
#ifndef MOE_GEMM_U_MXFP8
#define MOE_GEMM_U_MXFP8 1
#endif
#ifndef MOE_GEMM_U_NVFP4
#define MOE_GEMM_U_NVFP4 1
#endif

// kgroups per pipeline step: enough bytes in flight per wave for each format
template <int DT>
struct StepK {
  static constexpr int U = DT == DT_BF16 ? MOE_GEMM_U_BF16 : (DT == DT_MXFP8 ? MOE_GEMM_U_MXFP8 : MOE_GEMM_U_NVFP4);
};

// Epilogue of one wave's accumulators acc[4 tiles][NT token sub-tiles] for
// sorted rows r0 + 16s + (lane % 16) (valid below r_end) and weight row group
// g of expert e.  Gate/up GEMM: tiles 0,1 = gate rows 32g + 16tp + 4q + j,
// tiles 2,3 = the matching up rows; h = silu(g) * u (ReLU^2 experts: h =
// relu(v)^2 of all four tiles, 64 intermediates) is requantised into hq
// (codes, scales, exact 16-bit copy).  Down GEMM: y rows at the pair index.
template <int DT, int NT, bool G13>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, f32x4_t (&acc)[4][NT], int r0, int r_end, int g,
                                              int e, int lane) {
  const int i16 = lane & 15, q = lane >> 4;
  const float alpha = DT == DT_NVFP4 ? a.walpha[e] : 1.f;
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    const int r = r0 + 16 * s + i16;
    const bool ok = r < r_end;
    if constexpr (G13) {
      const int I = a.n_out;
      // requantise and store 32 intermediates: h[tp][j] is index 32gg + 16tp + 4q + j
      auto store_h = [&](const float(&h)[2][4], int gg) __attribute__((always_inline)) {
        if (DT == DT_BF16 || (DT == DT_MXFP8 && a.act_bf16)) {  // bf16 intermediate
          if (ok) {
            uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (size_t)r * I + 32 * gg + 4 * q;
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
              uint2 v;
              v.x = f32_to_bf16(h[tp][0]) | ((uint32_t)f32_to_bf16(h[tp][1]) << 16);
              v.y = f32_to_bf16(h[tp][2]) | ((uint32_t)f32_to_bf16(h[tp][3]) << 16);
              *reinterpret_cast<uint2*>(o + 16 * tp) = v;
            }
          }
        } else if constexpr (DT == DT_MXFP8) {
          // one block of 32 along I: [32g, 32g+32), spread over the 4 lanes sharing i16
          float amax = 0.f;
#pragma unroll
          for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(h[tp][j]));
          amax = wave_max_xor(amax, 16, 32);
          const int sx = mx_scale_exp(amax);
          if (ok) {
            uint8_t* o = a.out + (size_t)r * I + 32 * gg + 4 * q;
            uint16_t* od = a.out_deq + (size_t)r * I + 32 * gg + 4 * q;
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
              uint2 dq;
              const uint32_t v = mx_encode4(h[tp][0], h[tp][1], h[tp][2], h[tp][3], sx, dq);
              *reinterpret_cast<uint32_t*>(o + 16 * tp) = v;
              *reinterpret_cast<uint2*>(od + 16 * tp) = dq;
            }
            if (q == 0) a.out_scales[(size_t)r * (I / 32) + gg] = (uint8_t)(sx + 127);
          }
        } else if constexpr (DT == DT_NVFP4) {
          // two blocks of 16 along I: [32g + 16tp, +16)
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            float amax = fmaxf(fmaxf(fabsf(h[tp][0]), fabsf(h[tp][1])), fmaxf(fabsf(h[tp][2]), fabsf(h[tp][3])));
            amax = wave_max_xor(amax, 16, 32);
            const uint32_t sc_code = e4m3_from_f32(amax / 6.0f);
            const float sc = e4m3_to_f32(sc_code);
            uint32_t v = 0, d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint32_t c = sc > 0.f ? e2m1_from_f32(h[tp][j], sc) : ((__float_as_uint(h[tp][j]) >> 28) & 8u);
              v |= c << (4 * j);
              d[j] = f32_to_f16_bits(e2m1_to_f32(c) * sc);  // exact in fp16
            }
            if (ok) {
              *reinterpret_cast<uint16_t*>(a.out + (size_t)r * (I / 2) + 16 * gg + 8 * tp + 2 * q) = (uint16_t)v;
              if (q == 0) a.out_scales[(size_t)r * (I / 16) + 2 * gg + tp] = (uint8_t)sc_code;
              *reinterpret_cast<uint2*>(a.out_deq + (size_t)r * I + 32 * gg + 16 * tp + 4 * q) =
                  make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
            }
          }
        }
      };
      // SwiGLU: tiles 0,1 = gate rows 32g + 16tp + 4q + j, tiles 2,3 = the
      // matching up rows.  ReLU^2: the group's 64 W1 rows 64g + 16t + 4q + j
      // are the intermediates of half groups 2g + t / 2.  One copy of the
      // store code serves both (tiles are selected, not indexed).
      const int halves = a.gated ? 1 : 2;
#pragma unroll 1
      for (int hh = 0; hh < halves; ++hh) {
        float h[2][4];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (a.gated) {
              float gv = acc[tp][s][j] * alpha, uv = acc[2 + tp][s][j] * alpha;
              if (a.limit > 0.f) {
                gv = fminf(gv, a.limit);
                uv = fminf(fmaxf(uv, -a.limit), a.limit);
              }
              // silu with the hardware exp and reciprocal (~1 ulp each): h is requantised
              // to at most 8 significant bits, so a code moves only within a few ulps of a midpoint
              h[tp][j] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            } else {
              const float v = fmaxf((hh ? acc[2 + tp][s][j] : acc[tp][s][j]) * alpha, 0.f);
              h[tp][j] = v * v;
            }
          }
        store_h(h, a.gated ? g : 2 * g + hh);
      }
    } else {
      if (ok) {
        const int p = a.sorted_pairs[r];
        if (a.red) {  // in-kernel fc2 reduce: w * y added to the token's fp32 output row
          const float wp = a.wts[p];
          float* o = a.red + (size_t)(p / a.k) * a.n_out + 64 * g + 4 * q;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) unsafeAtomicAdd(o + 16 * t + j, wp * (acc[t][s][j] * alpha));
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (size_t)p * a.n_out + 64 * g + 4 * q;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            uint2 v;
            v.x = f32_to_bf16(acc[t][s][0] * alpha) | ((uint32_t)f32_to_bf16(acc[t][s][1] * alpha) << 16);
            v.y = f32_to_bf16(acc[t][s][2] * alpha) | ((uint32_t)f32_to_bf16(acc[t][s][3] * alpha) << 16);
            *reinterpret_cast<uint2*>(o + 16 * t) = v;
          }
        }
      }
    }
  }
}

// Routed rows per decode work item (m-tile), for both token-tile widths.
constexpr int kDecodeMT = 32;

// One work item (expert, m-tile of kDecodeMT sorted rows, 64-row weight
// group) of a grouped GEMM: the four waves stream their K slices into MFMAs,
// reduce through LDS, and run the epilogue (SwiGLU + requantisation for the
// gate/up GEMM, bf16 y rows for the down GEMM).  `w` numbers items
// m-tile-major; `cum` holds the per-expert m-tile prefix from
// build_schedule; `e_known` is the item's expert if the caller has it, else
// -1.  Returns the item's expert.  Ends with the block's LDS free for reuse.
//
// NT = 2: every wave covers the item's 32 rows (two 16-row token
// sub-tiles) and a quarter of K.  NT = 1: an item of at most 16 rows is
// split over K four ways as above; an item of 17-32 rows runs as two halves,
// waves 0-1 on rows r0.. and waves 2-3 on rows r0 + 16.., each pair
// splitting K two ways.  Both halves then read every weight tile at nearly
// the same time, so an expert with up to 32 rows fetches its weights from
// HBM once (two 16-row items had them read twice: measured +10 % HBM bytes
// on the MXFP8 decode layer, whose skewed routing gives a few experts
// 17-32 rows).
template <int DT, int NT, bool G13>
__device__ __forceinline__ int gemm_item(const GemmArgs& a, long long w, const int* cum,
                                         f32x4_t (*red)[4 * NT][64], int e_known = -1) {
  static_assert(16 * NT <= kDecodeMT, "token sub-tiles");
  constexpr int U = StepK<DT>::U;
  constexpr bool NTLD = MOE_GEMM_NTLOAD && NT == 1;  // decode: weights are streamed once
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int mtg = (int)(w / a.G), g = (int)(w % a.G);
  const int e = e_known >= 0 ? e_known : find_expert(cum, a.E, mtg);
  const int r0 = a.offsets[e] + (mtg - cum[e]) * kDecodeMT, r_end = a.offsets[e + 1];
  // halves (uniform across the block): nw waves share one set of rows starting at rs
  const bool pair = NT == 1 && r_end - r0 > 16;
  const int nw = pair ? 2 : 4, wl = pair ? (wv & 1) : wv;
  const int rs = pair ? r0 + 16 * (wv >> 1) : r0;
  // K slices are dealt to the nw waves in rounds of nw*U consecutive kgroups
  // (wave wl takes kgroups nw*U*j + U*wl .. +U), so the waves stream one
  // contiguous region; steps are double-buffered.
  const int nrounds = (a.KG + nw * U - 1) / (nw * U);
  int brow[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    int r = rs + 16 * s + i16;
    brow[s] = r < r_end ? (G13 ? a.sorted_pairs[r] / a.k : r) : -1;
  }
  f32x4_t acc[4][NT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < NT; ++s) acc[t][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const size_t tbase = (size_t)(e * a.G + g) * a.KG;
  KFrag<DT, NT> F0[U], F1[U];
  auto load_step = [&](KFrag<DT, NT>(&F)[U], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kg = nw * U * j + U * wl + u;
      if (kg < a.KG) load_kfrag<DT, NT, G13, NTLD>(F[u], a, (tbase + kg) * 4, kg, brow, lane, i16, q);
    }
  };
  auto mma_step = [&](const KFrag<DT, NT>(&F)[U], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kg = nw * U * j + U * wl + u;
      if (kg < a.KG) mma_kfrag<DT, NT>(acc, F[u], q);
    }
  };
  if constexpr (MOE_GEMM_PIPELINE) {
    load_step(F0, 0);
    for (int j = 0; j < nrounds; j += 2) {
      if (j + 1 < nrounds) load_step(F1, j + 1);
      mma_step(F0, j);
      if (j + 1 < nrounds) {
        if (j + 2 < nrounds) load_step(F0, j + 2);
        mma_step(F1, j + 1);
      }
    }
  } else {
    for (int j = 0; j < nrounds; ++j) {
      load_step(F0, j);
      mma_step(F0, j);
    }
  }

  // reduce the partial sums into the first wave of each set, in wave order
  if (pair) {
    if (wl == 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < NT; ++s) red[wv >> 1][t * NT + s][lane] = acc[t][s];
    }
  } else if (wv > 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < NT; ++s) red[wv - 1][t * NT + s][lane] = acc[t][s];
  }
  __syncthreads();
  if (wl == 0) {
    if (pair) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < NT; ++s) acc[t][s] += red[wv >> 1][t * NT + s][lane];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < NT; ++s)
          acc[t][s] += red[0][t * NT + s][lane] + red[1][t * NT + s][lane] + red[2][t * NT + s][lane];
    }
    gemm_epilogue<DT, NT, G13>(a, acc, rs, r_end, g, e, lane);
  }
  __syncthreads();
  return e;
}

// Paired m-tiles of an expert with `rows` routed rows (NT = 1 decode items
// of 17-32 rows, which take twice as long as the others): its full 32-row
// m-tiles and a last partial one of more than 16 rows.  Its other m-tile,
// if any, is the last one, of at most 16 rows.
__device__ __forceinline__ int paired_mtiles(int rows) { return rows / kDecodeMT + (rows % kDecodeMT > 16 ? 1 : 0); }

// Execution order of the NT = 1 decode items.  Blocks take positions
// blockIdx.x, + gridDim.x, ... (round-robin, so blocks running together
// stream neighbouring weight rows).  The N = q*B + r items leave blocks r..B-1
// one item short; the P paired items go to positions rp .. rp + P - 1, rp =
// min(r, N - P), i.e. to those blocks first, and the single items fill the
// other positions in order.  Within each kind the order is m-tile-major.
// cum / pcum: per-expert prefixes of m-tiles / paired m-tiles.
// Returns the item; `e` receives its expert.
__device__ __forceinline__ long long decode_item_at(long long x, long long rp, long long P, const GemmArgs& a,
                                                     const int* cum, const int* pcum, int& e) {
  const long long G = a.G;
  int lo = 0, hi = a.E;
  if (x >= rp && x < rp + P) {  // the k-th paired m-tile: expert lo with pcum[lo] <= k < pcum[lo + 1]
    const long long k = (x - rp) / G, g = (x - rp) % G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pcum[mid] <= k) lo = mid;
      else hi = mid;
    }
    e = lo;
    return ((long long)cum[lo] + (k - pcum[lo])) * G + g;
  }
  const long long y = x < rp ? x : x - P;  // the k-th single m-tile, its expert's last
  const long long k = y / G, g = y % G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] - pcum[mid] <= k) lo = mid;
    else hi = mid;
  }
  e = lo;
  return ((long long)cum[lo + 1] - 1) * G + g;
}

// Per-expert prefixes of the decode items' m-tiles (cum) and, for NT = 1,
// of their paired m-tiles (pcum), in one scan: the two counts are packed in
// 16-bit halves.  NT = 1 runs only for T * k <= 16 E <= 16384 routed rows,
// so both totals stay below 2^16; NT = 2 scans m-tiles alone.  Returns the
// m-tile total; total_pairs receives the paired total (0 for NT = 2).
template <int NT>
__device__ __forceinline__ int build_decode_schedule(const int* __restrict__ offsets, int E, int* cum, int* pcum,
                                                     int* wsum, int& total_pairs) {
  total_pairs = 0;
  if constexpr (NT == 1) {
    const int both = build_prefix<int>(
        offsets, E, [](int c) { return (c + kDecodeMT - 1) / kDecodeMT + (paired_mtiles(c) << 16); },
        [&](int e, int v) {
          cum[e] = v & 0xFFFF;
          pcum[e] = v >> 16;
        },
        wsum);
    total_pairs = both >> 16;
    return both & 0xFFFF;
  } else {
    return build_schedule(offsets, E, kDecodeMT, cum, wsum);
  }
}

hipError_t launch_prefill(int dt, bool g13, const GemmArgs& a, int grid, hipStream_t s);
// MXFP8 layers: the prefill-shaped down GEMM on the fp8 matrix instruction (a.wcodes: fragment
// region, a.act / a.act_scales: e4m3 codes / e8m0 scales of the hq rows); g13 must be false
hipError_t launch_prefill_f8(bool g13, const GemmArgs& a, int grid, hipStream_t s);
// The load-balance mode the prefill kernels run for moe_knobs.load_balance:
// mode 3 (the n-block split, pf_split_item) is for the gate/up GEMM and needs
// its n-block count (weight row groups G / 4) and the grid to be multiples of
// 8 (the XCDs), else the default chunked deal (0).
int prefill_balance(bool g13, int balance, int G, int grid);

}  // namespace moe
