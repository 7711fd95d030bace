// Device-side bodies of the routing, permutation, activation quantisation
// and combine stages, shared by the stage kernels and the fused kernel.
#pragma once

#include "moe_kernels.h"

namespace moe {

// ------------------------------------------------------------------ routing
// One wave per token.  Each lane holds experts lane, lane+64, ... (E <= 1024,
// up to 16 per lane).  k rounds of a wave-wide arg-max under the total order
// (logit descending, id ascending) pick the experts; slot j is the j-th pick.
// Weights: softmax over the k picked logits [vLLM PR 40082 report,
// "Implementation" item 1: routing inside the fused call].

// (v, i) <- the better of (v, i) and (ov, oi): larger value, then smaller id
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  const bool b = ov > v || (ov == v && oi < i);
  v = b ? ov : v;
  i = b ? oi : i;
}

// Row-local exchange through the DPP crossbar (a few cycles, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
  argmax_merge(v, i, ov, oi);
}

// Wave-wide arg-max; every lane receives the winner.  Within each row of 16
// lanes: swaps of neighbours (quad_perm 1,0,3,2), of pairs (2,3,0,1), then
// the half-row and row mirrors; the four row winners are then read from
// lanes 0, 16, 32, 48 and merged in row order.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<0xB1>(v, i);   // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4E>(v, i);   // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x141>(v, i);  // row_half_mirror
  argmax_dpp<0x140>(v, i);  // row_mirror
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    argmax_merge(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r)),
                 __builtin_amdgcn_readlane(i, 16 * r));
  v = bv;
  i = bi;
}

template <int NV>
__device__ __forceinline__ void route_token_n(const float* __restrict__ logits, int t, int E, int k,
                                              int* __restrict__ ids, float* __restrict__ wts, int lane) {
  const float* row = logits + (size_t)t * E;
  float v[NV];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int e = lane + 64 * i;
    float x = e < E ? row[e] : -INFINITY;
    v[i] = (x == x) ? x : -INFINITY;  // NaN never wins; results stay in range
    if (e >= E) taken |= 1u << i;
  }
  float my_val = 0.f, m0 = 0.f, sum = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int id = lane + 64 * i;
      bool better = !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && id < bi));
      bv = better ? v[i] : bv;
      bi = better ? id : bi;
    }
    wave_argmax(bv, bi);  // uniform across the wave from here
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) m0 = bv;
    sum += expf(bv - m0);  // the softmax denominator, in pick order
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = expf(my_val - m0) / sum;
  }
}

// One token's routing with NV = ceil(E / 64) rounded up to a power of two
// logits per lane (E <= 1024), so small expert counts skip empty slots.
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int* __restrict__ ids, float* __restrict__ wts, int lane) {
  if (E <= 64) route_token_n<1>(logits, t, E, k, ids, wts, lane);
  else if (E <= 128) route_token_n<2>(logits, t, E, k, ids, wts, lane);
  else if (E <= 256) route_token_n<4>(logits, t, E, k, ids, wts, lane);
  else if (E <= 512) route_token_n<8>(logits, t, E, k, ids, wts, lane);
  else route_token_n<16>(logits, t, E, k, ids, wts, lane);
}

// ------------------------------------------------------------------ permutation
// One block: stable counting sort of the P = T*k pairs by expert.  Each of
// the NWAVES waves owns a contiguous segment of pairs; pass 1 builds per-wave
// expert histograms in LDS, a scan turns them into per-(wave, expert) start
// positions, pass 2 walks each segment in order and ranks pairs of equal
// expert inside a 64-pair step with ballots on the id bits.  `hist` and
// `scan_tmp` are LDS of NWAVES*1024 and 64*NWAVES ints.
template <int NWAVES>
constexpr int permute_lds_ints() { return NWAVES * 1024 + 64 * NWAVES; }

template <int NWAVES>
__device__ void permute_block(const int* __restrict__ ids, int P, int E, int* __restrict__ offsets,
                              int* __restrict__ sorted_pairs, int* __restrict__ pair_pos, int (*hist)[1024],
                              int* scan_tmp) {
  constexpr int kPermWaves = NWAVES, kPermThreads = 64 * NWAVES, kPer = 1024 / kPermThreads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kPermWaves * 1024; i += kPermThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int S = ((P + kPermWaves * 64 - 1) / (kPermWaves * 64)) * 64;  // segment, multiple of 64
  const int seg0 = min(P, w * S), seg1 = min(P, (w + 1) * S);
  // ids outside [0, E) are clamped: results are then unspecified but every access stays in bounds.
  // Loads go kAhead chunks of 64 at a time, so the wave waits for memory once per group, not per chunk.
  // (Loads past the segment read a clamped in-bounds address and are discarded, so they need no branch.)
  constexpr int kAhead = 16;
  for (int p = seg0 + lane; p < seg1; p += 64 * kAhead) {
    int v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = ids[min(p + 64 * u, P - 1)];
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
      if (p + 64 * u < seg1) atomicAdd(&hist[w][min(max(v[u], 0), E - 1)], 1);
  }
  __syncthreads();
  // per-thread experts kPer*tid .. +kPer: totals, block exclusive scan
  int e0 = kPer * tid, local = 0;
  int tot[kPer] = {};
  for (int j = 0; j < kPer; ++j) {
    int e = e0 + j;
    if (e < E)
      for (int ww = 0; ww < kPermWaves; ++ww) tot[j] += hist[ww][e];
    local += tot[j];
  }
  scan_tmp[tid] = local;
  __syncthreads();
  for (int d = 1; d < kPermThreads; d <<= 1) {  // Hillis-Steele inclusive scan
    int add = tid >= d ? scan_tmp[tid - d] : 0;
    __syncthreads();
    scan_tmp[tid] += add;
    __syncthreads();
  }
  int base = scan_tmp[tid] - local;
  for (int j = 0; j < kPer; ++j) {
    int e = e0 + j;
    if (e < E) {
      offsets[e] = base;
      int b = base;
      for (int ww = 0; ww < kPermWaves; ++ww) {
        int c = hist[ww][e];
        hist[ww][e] = b;
        b += c;
      }
      base += tot[j];
    }
  }
  if (tid == 0) offsets[E] = P;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const unsigned long long lt = (1ull << lane) - 1ull;
  // chunk c's ids are loaded while chunk c - kAhead is ranked (a ring of kAhead registers)
  // (The wave's LDS operations complete in order, so each chunk sees the
  // previous chunk's hist update without a fence.)
  int ring[kAhead];
  if (seg0 < seg1) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) ring[u] = ids[min(seg0 + 64 * u + lane, P - 1)];
  }
  for (int p0 = seg0; p0 < seg1; p0 += 64 * kAhead) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int p = p0 + 64 * u + lane;
      if (p0 + 64 * u >= seg1) break;  // wave-uniform
      const bool valid = p < seg1;
      const int id = valid ? min(max(ring[u], 0), E - 1) : 0;
      ring[u] = ids[min(p + 64 * kAhead, P - 1)];
      unsigned long long m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        bool bit = (id >> b) & 1;
        unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        int pos = hist[w][id] + __popcll(m & lt);
        sorted_pairs[pos] = p;
        pair_pos[p] = pos;
        if (lane == 63 - __clzll(m)) hist[w][id] += __popcll(m);
      }
    }
  }
}

// The same with its own static LDS.
template <int NWAVES>
__device__ void permute_block(const int* __restrict__ ids, int P, int E, int* __restrict__ offsets,
                              int* __restrict__ sorted_pairs, int* __restrict__ pair_pos) {
  __shared__ int hist[NWAVES][1024];
  __shared__ int scan_tmp[64 * NWAVES];
  permute_block<NWAVES>(ids, P, E, offsets, sorted_pairs, pair_pos, hist, scan_tmp);
}

template <int DT>
__device__ void quantize_x_blocks(const uint16_t* __restrict__ x, long long n_elem, uint8_t* __restrict__ codes,
                                  uint8_t* __restrict__ scales, uint16_t* __restrict__ deq, long long gtid,
                                  long long gstride) {
  if constexpr (DT == DT_BF16) {
    // copy 8 bf16 per thread
    const uint4* src = reinterpret_cast<const uint4*>(x);
    uint4* dst = reinterpret_cast<uint4*>(codes);
    for (long long i = gtid; i < n_elem / 8; i += gstride) dst[i] = src[i];
  } else {
    // MXFP8: 8 lanes x 4 elements per block of 32; NVFP4: 4 lanes x 4 per 16
    constexpr int LPB = DT == DT_MXFP8 ? 8 : 4;
    const long long nthreads = n_elem / 4;
    for (long long i = gtid; i < ((nthreads + 63) / 64) * 64; i += gstride) {
      const bool ok = i < nthreads;
      uint2 raw = ok ? reinterpret_cast<const uint2*>(x)[i] : make_uint2(0, 0);
      float v[4] = {bf16_to_f32(raw.x & 0xFFFF), bf16_to_f32(raw.x >> 16), bf16_to_f32(raw.y & 0xFFFF),
                    bf16_to_f32(raw.y >> 16)};
      float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      amax = wave_max_xor(amax, 1, LPB / 2);
      const int sub = (int)(i % LPB);
      const long long blk = i / LPB;
      if constexpr (DT == DT_MXFP8) {
        int s = mx_scale_exp(amax);
        uint2 dq;
        const uint32_t out = mx_encode4(v[0], v[1], v[2], v[3], s, dq);
        if (ok) {
          reinterpret_cast<uint32_t*>(codes)[i] = out;
          if (sub == 0) scales[blk] = (uint8_t)(s + 127);
          reinterpret_cast<uint2*>(deq)[i] = dq;
        }
      } else {
        uint32_t sc_code = e4m3_from_f32(amax / 6.0f);
        float sc = e4m3_to_f32(sc_code);
        uint32_t out = 0, d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t c = sc > 0.f ? e2m1_from_f32(v[j], sc) : ((__float_as_uint(v[j]) >> 28) & 8u);
          out |= c << (4 * j);
          d[j] = f32_to_f16_bits(e2m1_to_f32(c) * sc);  // exact in fp16
        }
        if (ok) {
          reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)out;
          if (sub == 0) scales[blk] = (uint8_t)sc_code;
          reinterpret_cast<uint2*>(deq)[i] = make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine
// out[t, h] = bf16( sum_j w[t, j] * y[t*k + j, h] ), fp32, slot order.
__device__ __forceinline__ void combine_range(const uint16_t* __restrict__ y, const float* __restrict__ wts, int T,
                                              int H, int k, uint16_t* __restrict__ out, long long gtid,
                                              long long gstride) {
  const long long n = (long long)T * H / 8;
  for (long long i = gtid; i < n; i += gstride) {
    const long long e0 = i * 8;
    const int t = (int)(e0 / H), h = (int)(e0 % H);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const float wj = wts[(size_t)t * k + j];
      const uint4 v = *reinterpret_cast<const uint4*>(y + ((size_t)t * k + j) * H + h);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] += wj * bf16_to_f32(u[m] & 0xFFFF);
        acc[2 * m + 1] += wj * bf16_to_f32(u[m] >> 16);
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + e0) = o;
  }
}

}  // namespace moe
