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
//
// The order is carried by one 64-bit key per expert: the logit mapped to an
// unsigned integer of the same order (its high half; -0 counts as +0, NaN as
// -inf) and the complement of the id (low half, so the smaller id of two
// equal logits has the larger key); experts past E get key 0, below every
// real one.  Each lane sorts its own keys once; a round is then one
// wave-wide maximum of the lanes' first keys (DPP exchanges, no LDS), after
// which the winning lane drops its first key.

__device__ __forceinline__ uint64_t route_key(float v, int id) {
  v = (v == v) ? v + 0.0f : -INFINITY;  // NaN never wins; -0 -> +0 (equal logits tie on the id)
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ __forceinline__ int route_key_id(uint64_t key) { return (int)~(uint32_t)key; }

// x = max(x, the value DPP control CTRL brings from another lane); lanes
// outside ROW_MASK keep their own value
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max_dpp_u64(uint64_t& x) {
  const uint32_t hi = (uint32_t)(x >> 32), lo = (uint32_t)x;
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  x = o > x ? o : x;
}

// Wave-wide maximum of a 64-bit key; every lane receives it.  Within each row
// of 16 lanes: swaps of neighbours (quad_perm 1,0,3,2), of pairs (2,3,0,1),
// then the half-row and row mirrors; across rows: row 0's lane 15 into row 1
// and row 2's into row 3 (row_bcast:15), then row 1's lane 31 into rows 2
// and 3 (row_bcast:31); lane 63 then holds the wave's maximum.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  max_dpp_u64<0xB1, 0xF>(x);   // quad_perm [1, 0, 3, 2]
  max_dpp_u64<0x4E, 0xF>(x);   // quad_perm [2, 3, 0, 1]
  max_dpp_u64<0x141, 0xF>(x);  // row_half_mirror
  max_dpp_u64<0x140, 0xF>(x);  // row_mirror
  max_dpp_u64<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  max_dpp_u64<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  return ((uint64_t)hi << 32) | lo;
}

// Descending compare-exchange of keys a, b (a keeps the larger)
__device__ __forceinline__ void route_cx(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

template <int NV>
__device__ __forceinline__ void route_token_n(const float* __restrict__ logits, int t, int E, int k,
                                              int* __restrict__ ids, float* __restrict__ wts, int lane) {
  const float* row = logits + (size_t)t * E;
  uint64_t key[NV];
  // every load in bounds and unconditional (slots past E read logit E - 1
  // and get the lowest key), so the NV loads are in flight together rather
  // than one after another behind per-slot branches
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(v[i], e) : 0ull;
  }
  // this lane's keys in descending order (Batcher's odd-even merge sort
  // network for the next power of two, less the comparators that touch a
  // place >= NV: those places would hold the lowest keys, already last)
#pragma unroll
  for (int p = 1; p < NV; p <<= 1)
#pragma unroll
    for (int q = p; q >= 1; q >>= 1)
#pragma unroll
      for (int j = q % p; j + q < NV; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q && i + j + q < NV; ++i)
          if ((i + j) / (2 * p) == (i + j + q) / (2 * p)) route_cx(key[i + j], key[i + j + q]);
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t w = wave_max_u64(key[0]);  // uniform: pick j
    // the one lane that held it drops it: its keys move up one place.  The
    // move is written as masked bit operations on a mask the compiler cannot
    // see through; as selects it became a gather of every key from every
    // place (NV^2 selects per round).
    uint32_t m = key[0] == w ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(m));
    const uint64_t m64 = ((uint64_t)m << 32) | m;
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) key[i] ^= (key[i] ^ key[i + 1]) & m64;
    key[NV - 1] &= ~m64;
    mine = lane == j ? w : mine;
  }
  // slot `lane` < k: softmax over the picks, the denominator summed in pick order
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(route_key_value(mine)), 0));
  const float ex = expf(route_key_value(mine) - m0);
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = route_key_id(mine);
    wts[(size_t)t * k + lane] = ex / sum;
  }
}

// One token's routing with NV = ceil(E / 64) logits per lane (E <= 1024),
// rounded up to one of 1, 2, 4, 6, 8, 12, 16, so small expert counts skip
// empty slots (the sorting network and the key moves grow with NV; the
// 384-expert layers take 6).
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int* __restrict__ ids, float* __restrict__ wts, int lane) {
  if (E <= 64) route_token_n<1>(logits, t, E, k, ids, wts, lane);
  else if (E <= 128) route_token_n<2>(logits, t, E, k, ids, wts, lane);
  else if (E <= 256) route_token_n<4>(logits, t, E, k, ids, wts, lane);
  else if (E <= 384) route_token_n<6>(logits, t, E, k, ids, wts, lane);
  else if (E <= 512) route_token_n<8>(logits, t, E, k, ids, wts, lane);
  else if (E <= 768) route_token_n<12>(logits, t, E, k, ids, wts, lane);
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
__device__ __forceinline__ void permute_block(const int* __restrict__ ids, int P, int E, int* __restrict__ offsets,
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
  // The first group's ids stay in registers for the ranking pass below (a
  // segment of up to 64 kAhead pairs -- every decode batch -- is then read
  // from memory once).
  constexpr int kAhead = 16;
  int first[kAhead];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) first[u] = ids[min(seg0 + lane + 64 * u, P - 1)];
#pragma unroll
  for (int u = 0; u < kAhead; ++u)
    if (seg0 + lane + 64 * u < seg1) atomicAdd(&hist[w][min(max(first[u], 0), E - 1)], 1);
  for (int p = seg0 + lane + 64 * kAhead; p < seg1; p += 64 * kAhead) {
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
  // block exclusive scan of `local`: inclusive scans inside the waves, then
  // the waves' totals
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) scan_tmp[w] = incl;
  __syncthreads();
  int base = incl - local;
  for (int ww = 0; ww < w; ++ww) base += scan_tmp[ww];
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
#pragma unroll
  for (int u = 0; u < kAhead; ++u) ring[u] = first[u];
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

// Lanes of a 64-pair step (valid ones) that hold the same expert id as this
// lane: one ballot per id bit.
__device__ __forceinline__ unsigned long long same_expert_lanes(int id, bool valid, int nbits) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (id >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// The same sort split over several blocks, for large P.  Block c sorts the
// pairs of chunk [c0, c1): it counts the experts of all P pairs (each block
// redundantly: P ids from L2 against one block's serial ranking of all P),
// of the pairs before c0 and, per wave sub-segment, of its chunk; the
// exclusive scan of the totals gives offsets (written by the block with
// c0 == 0), offsets + the before-counts give the chunk's first position of
// each expert, and its waves rank their sub-segments as permute_block does.
// The result is the unique stable order, the same as permute_block's.
// c0 and the chunk length are multiples of 64 NWAVES except the last
// chunk's end (c1 == P).  LDS (ints): all[E], before[E], sub[NWAVES][E],
// scan_tmp[64 NWAVES].
template <int NWAVES>
__host__ __device__ constexpr int permute_chunk_lds_ints(int E) { return (2 + NWAVES) * E + 64 * NWAVES; }

template <int NWAVES>
__device__ __forceinline__ void permute_chunk(const int* __restrict__ ids, int P, int E, int c0, int c1,
                                              int* __restrict__ offsets, int* __restrict__ sorted_pairs,
                                              int* __restrict__ pair_pos, int* lds) {
  constexpr int kThreads = 64 * NWAVES, kAhead = 16;
  int* all = lds;
  int* before = lds + E;
  int* sub = lds + 2 * E;  // [NWAVES][E]
  int* scan_tmp = lds + (2 + NWAVES) * E;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < (2 + NWAVES) * E; i += kThreads) lds[i] = 0;
  __syncthreads();
  // 1. counts: wave w takes 64-aligned segment w of all P pairs, one LDS add
  //    per pair (a 64-pair step lies wholly before, inside or after the
  //    chunk, and inside one wave sub-segment of it)
  const int S = ((P + NWAVES * 64 - 1) / (NWAVES * 64)) * 64;
  const int SS = ((c1 - c0 + NWAVES * 64 - 1) / (NWAVES * 64)) * 64;  // chunk sub-segment per wave
  const int seg0 = min(P, w * S), seg1 = min(P, (w + 1) * S);
  for (int p0 = seg0; p0 < seg1; p0 += 64 * kAhead) {
    int v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = ids[min(p0 + 64 * u + lane, P - 1)];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int q0 = p0 + 64 * u;  // the step's first pair (wave-uniform)
      if (q0 >= seg1) break;
      if (q0 + lane < seg1) {
        const int id = min(max(v[u], 0), E - 1);
        atomicAdd(&all[id], 1);
        if (q0 < c0) atomicAdd(&before[id], 1);
        else if (q0 < c1) atomicAdd(&sub[((q0 - c0) / SS) * E + id], 1);
      }
    }
  }
  __syncthreads();
  // 2. offsets (exclusive scan of the totals over experts, kPer experts per
  //    thread), then the first position of each expert in each wave's
  //    sub-segment of the chunk
  constexpr int kPer = 1024 / kThreads;
  const int e0 = kPer * tid;
  int local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) local += e0 + j < E ? all[e0 + j] : 0;
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) scan_tmp[w] = incl;
  __syncthreads();
  int off = incl - local;
  for (int ww = 0; ww < w; ++ww) off += scan_tmp[ww];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = e0 + j;
    if (e < E) {
      if (c0 == 0) offsets[e] = off;
      int b = off + before[e];
      for (int ww = 0; ww < NWAVES; ++ww) {
        const int c = sub[ww * E + e];
        sub[ww * E + e] = b;
        b += c;
      }
      off += all[e];
    }
  }
  if (c0 == 0 && tid == 0) offsets[E] = P;
  __syncthreads();
  // 3. each wave ranks its sub-segment of the chunk in order (ballots on the
  //    id bits give each pair's place among the step's pairs of its expert)
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int* mine = sub + w * E;
  const int r0 = min(c1, c0 + w * SS), r1 = min(c1, c0 + (w + 1) * SS);
  for (int p0 = r0; p0 < r1; p0 += 64 * kAhead) {
    int v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = ids[min(p0 + 64 * u + lane, P - 1)];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      if (p0 + 64 * u >= r1) break;  // wave-uniform
      const int p = p0 + 64 * u + lane;
      const bool valid = p < r1;
      const int id = valid ? min(max(v[u], 0), E - 1) : 0;
      const unsigned long long m = same_expert_lanes(id, valid, nbits);
      if (valid) {
        const int pos = mine[id] + __popcll(m & lt);
        sorted_pairs[pos] = p;
        pair_pos[p] = pos;
        if (lane == 63 - __clzll(m)) mine[id] += __popcll(m);
      }
    }
  }
}

// The same with its own static LDS.
template <int NWAVES>
__device__ __forceinline__ void permute_block(const int* __restrict__ ids, int P, int E, int* __restrict__ offsets,
                              int* __restrict__ sorted_pairs, int* __restrict__ pair_pos) {
  __shared__ int hist[NWAVES][1024];
  __shared__ int scan_tmp[64 * NWAVES];
  permute_block<NWAVES>(ids, P, E, offsets, sorted_pairs, pair_pos, hist, scan_tmp);
}

template <int DT>
__device__ __forceinline__ void quantize_x_blocks(const uint16_t* __restrict__ x, long long n_elem,
                                                  uint8_t* __restrict__ codes,
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
    // U grid-stride steps per pass, their loads issued together (at clamped
    // in-bounds addresses, no branch): 8 bytes per lane per step are too
    // few bytes in flight to stream x at the memory's rate
    constexpr int U = 4;
    const long long nthreads = n_elem / 4;
    const long long lim = ((nthreads + 63) / 64) * 64;  // whole waves: the group maximum needs every lane
    for (long long i0 = gtid; i0 < lim; i0 += U * gstride) {
      uint2 rawu[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        rawu[u] = reinterpret_cast<const uint2*>(x)[min(i0 + u * gstride, nthreads - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
      const long long i = i0 + u * gstride;
      if (i >= lim) break;  // the same for the whole wave (gtid and gstride keep waves 64-aligned)
      const bool ok = i < nthreads;
      const uint2 raw = ok ? rawu[u] : make_uint2(0, 0);
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
    // slots in batches of 8: all loads of a batch are issued before the
    // first use, so a token's k rows cost one memory latency per batch
    // instead of one per slot; the sum keeps slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      float wj[8];
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = min(j0 + j, k - 1);  // slots past k reload the last one, unused
        wj[j] = wts[(size_t)t * k + jj];
        v[j] = *reinterpret_cast<const uint4*>(y + ((size_t)t * k + jj) * H + h);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j < k) {
          const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            acc[2 * m] += wj[j] * bf16_to_f32(u[m] & 0xFFFF);
            acc[2 * m + 1] += wj[j] * bf16_to_f32(u[m] >> 16);
          }
        }
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
