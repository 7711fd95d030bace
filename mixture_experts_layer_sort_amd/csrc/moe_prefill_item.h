// The prefill-shaped grouped-GEMM work item, shared by the stage kernel
// (moe_prefill.hip) and the fused single-launch kernel.
//
// Item = (expert, m-tile of 128 sorted rows, n-block of 4 weight row groups
// = 256 weight rows).  The block's 4 waves each own one row group (64 rows:
// for the gate/up GEMM 32 gate rows then the 32 matching up rows) and all
// 128 token rows: a 64 x 128 wave tile of 32x32x16 MFMAs (2 x 4 of them per
// 16-wide K slice), accumulated over K in order.  (From a single wave per
// SIMD the 32x32x16 instruction keeps the matrix unit much busier than
// 16x16x32: measured 2.1 vs 1.4 PFLOP/s on MI355X.)
//
//  * Weights stream from global memory straight into registers (each weight
//    element is used by exactly one wave): a ring of kPfStages K steps.
//    Fragments are gathered from the packed 16-row tiles: lane l of a
//    32-row fragment reads tile 2f + ((l >> 4) & 1), the lane position
//    (l & 15) + 16 * (2m + (l >> 5)) of the 16x16x32 layout.
//  * Token rows are shared by the 4 waves through LDS, filled by the 16-byte
//    direct global->LDS load (no register round trip) into a ring of
//    kPfStages stages of one 64-wide K step: per (32-row sub-tile, 32-wide
//    chunk) block, row-major with 64 B per row, the four 16-byte pieces of a
//    row XOR-swizzled so fragment reads are free of bank conflicts.
//  * One barrier per K step.  Loads for step s+kPfStages-1 are issued while
//    step s computes, spread between its MFMAs; the wait before the barrier
//    counts outstanding vector-memory operations explicitly.
#pragma once

#include <type_traits>

#include "moe_gemm_item.h"

namespace moe {

constexpr int kPfRows = 128;                  // routed rows per item of the single-launch kernel: 4 sub-tiles of 32
constexpr int kPfRowsStage = 256;             // routed rows per item of the stage kernel: 8 sub-tiles of 32
constexpr int kPfGroups = 4;                  // weight row groups per item, one per wave
// m-tiles per band of the item order (a band's token rows: 1024)
template <int ROWS>
constexpr int pf_band() { return 1024 / ROWS; }
// token part of a stage: ROWS / 32 sub-tiles x 2 chunks of 32 K, 32 rows x 64 B each, in 16-byte slots
template <int ROWS>
constexpr int pf_tok_slots() { return ROWS / 32 * 2 * 128; }
#ifndef MOE_PF_STAGES_Q
#define MOE_PF_STAGES_Q 4  // pipeline depth for MXFP8 / NVFP4 weights
#endif
constexpr int kPfMaxStages = 8;
// pipeline depth (K steps in flight + the one computed); 16-bit weights need
// twice the registers per step (the depth barely matters once loads are
// interleaved with the MFMAs: measured flat from 3 to 8 for MXFP8)
template <int DT, int ROWS>
constexpr int pf_stages() { return DT == DT_BF16 || (DT == DT_MXFP8 && ROWS > 128) ? 3 : MOE_PF_STAGES_Q; }

// Weights of MXFP8 items also go through LDS (direct loads in fragment
// order, shared by the two waves of a row group): the per-instruction cost of
// the address unit, not bytes, bounds the loads, and this halves their count.
template <int DT>
constexpr bool pf_alds() { return DT == DT_MXFP8; }
// 16-byte slots of one stage: tokens, then for LDS weights the codes
// [group 4][f 2][m 2][64 lanes] (16 KB) and per-wave scale copies [wave 8][64 words]
template <int DT, int ROWS>
constexpr int pf_stage_slots() { return pf_alds<DT>() ? pf_tok_slots<ROWS>() + 1024 + 128 : pf_tok_slots<ROWS>(); }
// weight loads per wave per K step (register path)
template <int DT>
constexpr int pf_a_ops() { return DT == DT_BF16 ? 8 : 6; }

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// One K step (64 wide = chunks 2h, 2h+1 of kgroup kg) of this wave's two
// 32-row weight fragments f, K slices m (16 wide) of each chunk, as loaded.
template <int DT>
struct PfA;
template <>
struct PfA<DT_BF16> {
  u32x4_t c[2][2][2];  // [f][chunk][m]: 8 bf16
};
template <>
struct PfA<DT_MXFP8> {
  u32x4_t c[2][2];  // [f][m]: 8 e4m3 of chunk 2h (words 0-1), of chunk 2h+1 (words 2-3)
  uint32_t s[2];    // [f]: the row's 4 e8m0 scales of the kgroup
};
template <>
struct PfA<DT_NVFP4> {
  u32x2_t c[2][2];  // [f][m]: 8 e2m1 of chunk 2h, of chunk 2h+1
  uint32_t s[2];    // [f]: the row's e4m3 scales of chunks 2h, 2h+1 (16 wide each)
};

// Blocks are dealt to the 8 XCDs (each with its own L2) round-robin by
// block index.  Renumbering so that each XCD holds a contiguous range of
// logical ids makes neighbouring items -- which share weight or token tiles
// -- run on the same L2.
__device__ __forceinline__ int xcd_logical_block() {
  const int b = blockIdx.x, g = gridDim.x;
  return g % 8 == 0 ? (b % 8) * (g / 8) + b / 8 : b;
}

// Slot of this block in chunk n of the persistent item order (chunks of
// gridDim.x consecutive items; the block takes item n gridDim.x + slot).
// The blocks of XCD x (b % 8 == x) take one contiguous slice of C =
// gridDim.x / 8 items of each chunk, so items that share weight or token
// tiles meet in one L2 (grids that are not a multiple of 8: block b takes
// place b).  `balance` (moe_knobs.load_balance) picks the slice and place:
// 0: slice x, place b / 8 every chunk (xcd_logical_block); 1: slice
// (x + n) % 8, place (b / 8 + n) % C; 2: slice (x + n / 4) % 8, place
// (b / 8 + n) % C.  Each is a permutation of the chunk's places.  (Mode 3
// does not use chunks: pf_split_item.)
__device__ __forceinline__ int pf_chunk_slot(long long n, int balance) {
  const int b = blockIdx.x, g = gridDim.x;
  if (g % 8 != 0) return b;
  const int C = g / 8, x = b % 8, j = b / 8, r = (int)(n % (32LL * C));
  if (balance == 1) return ((x + r) % 8) * C + (j + r) % C;
  if (balance == 2) return ((x + r / 4) % 8) * C + (j + r) % C;
  return x * C + j;
}

// Load-balance mode 3, the n-block split: XCD x takes the n-blocks
// [x NB/8, (x+1) NB/8) of every m-tile, so the eight XCDs get the same mix of
// full and ragged m-tiles (with the chunked deal the XCDs' sums differ by
// ~10 %, as each holds a fixed slice of every chunk).  Its blocks take the
// XCD's items i = b / 8 + n gridDim.x / 8 in round n, numbered m-tile-major (the
// NB / 8 n-blocks of one m-tile are neighbours, so they share its token
// rows); item i is w = (i / (NB/8)) NB + x NB/8 + i % (NB/8), decoded
// m-tile-major (pf_tile).  The host selects the mode only for the gate/up
// GEMM and only when NB and gridDim.x are multiples of 8, which makes it a
// permutation of the items.
__device__ __forceinline__ long long pf_split_item(long long i, int NB) {
  const int nx = NB / 8, x = (int)(blockIdx.x % 8);
  return (i / nx) * NB + x * nx + (int)(i % nx);
}

// This block's item in round n (rounds 0 .. total / gridDim.x, rounded up),
// or -1 for none: the chunked deal (pf_chunk_slot) or the n-block split.
// The split is built into the gate/up kernels only: the down kernels keep
// the plain chunked loop (their item bodies are at the edge of the register
// budget, and the extra branch there cost spills).
__device__ __forceinline__ long long pf_round_item(long long n, long long total, int NB, int balance) {
  if (balance == 3) {
    const long long i = blockIdx.x / 8 + n * (gridDim.x / 8);
    return i < total / 8 ? pf_split_item(i, NB) : -1;
  }
  const long long w = n * gridDim.x + pf_chunk_slot(n, balance);
  return w < total ? w : -1;
}

// m-tile (within expert e) and n-block of item w.  Modes 0-2 number the
// items expert-major, in bands of up to kBand m-tiles, n-block-major inside
// a band; mode 3 numbers them m-tile-major (w = global m-tile NB + n-block).
template <bool SPLIT>
__device__ __forceinline__ void pf_tile(long long w, int NB, int kBand, int balance, const int* cum, int e,
                                        int& mt, int& nb) {
  if (SPLIT && balance == 3) {
    const int wi = (int)w;  // item counts stay far below 2^31
    mt = wi / NB - cum[e];
    nb = wi % NB;
    return;
  }
  const int mts = cum[e + 1] - cum[e];
  const long long local = w - (long long)cum[e] * NB;
  const int band = (int)(local / (kBand * NB)), full = mts / kBand;
  const int bsize = band < full ? kBand : mts - full * kBand;
  const int inner = (int)(local - (long long)band * kBand * NB);
  nb = inner / bsize;
  mt = band * kBand + inner % bsize;
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS reads are done, then barrier.  No fence: the
// direct-to-LDS loads of later stages stay in flight across it.
template <int N>
__device__ __forceinline__ void pf_wait_barrier() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keep the uses of a K step's weight registers below the barrier that
// follows their wait (otherwise the register-only conversions are hoisted
// above it and the compiler inserts a full wait of its own).
template <int DT>
__device__ __forceinline__ void pf_pin(PfA<DT>& A) {
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    if constexpr (DT == DT_BF16) {
      asm volatile("" : "+v"(A.c[f][0][0]), "+v"(A.c[f][0][1]), "+v"(A.c[f][1][0]), "+v"(A.c[f][1][1]));
    } else {
      asm volatile("" : "+v"(A.c[f][0]), "+v"(A.c[f][1]), "+v"(A.s[f]));
    }
  }
}

// The token stages of one block: separate LDS objects, so the compiler's
// waits for the direct loads track each stage on its own.  Each index is
// one allocation per kernel, shared by every item the kernel runs.
template <int SLOTS>
struct PfStages {
  u32x4_t (*s[kPfMaxStages])[SLOTS];
};
template <int I, int SLOTS>
__device__ __forceinline__ u32x4_t (*pf_stage())[SLOTS] {
  __shared__ u32x4_t buf[SLOTS];
  return &buf;
}
template <int DT, int ROWS>
__device__ __forceinline__ PfStages<pf_stage_slots<DT, ROWS>()> pf_make_stages() {
  constexpr int NS = pf_stages<DT, ROWS>(), SL = pf_stage_slots<DT, ROWS>();
  static_assert(NS >= 3 && NS <= kPfMaxStages, "stages");
  PfStages<SL> st{};
  st.s[0] = pf_stage<0, SL>();
  st.s[1] = pf_stage<1, SL>();
  st.s[2] = pf_stage<2, SL>();
  if constexpr (NS > 3) st.s[3] = pf_stage<3, SL>();
  if constexpr (NS > 4) st.s[4] = pf_stage<4, SL>();
  if constexpr (NS > 5) st.s[5] = pf_stage<5, SL>();
  if constexpr (NS > 6) st.s[6] = pf_stage<6, SL>();
  if constexpr (NS > 7) st.s[7] = pf_stage<7, SL>();
  return st;
}

// Swizzle of the 16-byte pieces of token row r (0..31) in a stage block:
// piece p of the row sits in slot p ^ pf_swz(r).  Rows r, r+4, r+8, r+12
// (which the 64-byte row pitch puts on the same banks) get distinct slots;
// measured on MI355X, fragment reads with this swizzle are free of bank
// conflicts.
__device__ __forceinline__ int pf_swz(int r) { return (r >> 2) & 3; }

// Epilogue of a 64 x 32 NSA wave tile in the 32x32 accumulator layout: lane l,
// element e of acc[f][S] is weight row 32f + (e & 3) + 8 (e >> 2) + 4 (l >> 5)
// of row group g, routed row r0 + SSTR S + (l & 31).  Gate/up GEMM: SwiGLU of
// the f = 0 (gate) and f = 1 (up) values (ReLU^2 experts: relu(v)^2 of both
// fragments, 64 intermediates), requantised per token row; down GEMM: bf16 y
// rows of the pair.
template <int DT, bool G13, int NSA, int SW, int SSTR>
__device__ __forceinline__ void pf_epilogue(const GemmArgs& a, f32x16_t (&acc)[2][SW], int r0, int r_end, int g, int e,
                                            int lane) {
  const int hl = lane >> 5, l32 = lane & 31;
  const float alpha = DT == DT_NVFP4 ? a.walpha[e] : 1.f;
#pragma unroll
  for (int S = 0; S < NSA; ++S) {
    const int r = r0 + SSTR * S + l32;
    const bool ok = r < r_end;
    if constexpr (G13) {
      const int I = a.n_out;
      // requantise and store 32 intermediates of this token row
      auto store_h = [&](const float(&h)[16], int gg) __attribute__((always_inline)) {
        // h[4b + j] is intermediate index 32gg + 8b + 4hl + j
        if (DT == DT_BF16 || (DT == DT_MXFP8 && a.act_bf16)) {  // bf16 intermediate
          if (ok) {
            uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (size_t)r * I + 32 * gg + 4 * hl;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              *reinterpret_cast<uint2*>(o + 8 * b) =
                  make_uint2(f32_to_bf16(h[4 * b]) | ((uint32_t)f32_to_bf16(h[4 * b + 1]) << 16),
                             f32_to_bf16(h[4 * b + 2]) | ((uint32_t)f32_to_bf16(h[4 * b + 3]) << 16));
          }
        } else if constexpr (DT == DT_MXFP8) {
          // one block of 32 along I: this lane's 16 values and lane l ^ 32's
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(h[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
          const int sx = mx_scale_exp(amax);
          if (ok) {
            uint8_t* o = a.out + (size_t)r * I + 32 * gg + 4 * hl;
            uint16_t* od = a.out_deq + (size_t)r * I + 32 * gg + 4 * hl;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              uint2 dq;
              const uint32_t v = mx_encode4(h[4 * b], h[4 * b + 1], h[4 * b + 2], h[4 * b + 3], sx, dq);
              *reinterpret_cast<uint32_t*>(o + 8 * b) = v;
              if (a.out_deq) *reinterpret_cast<uint2*>(od + 8 * b) = dq;  // null: the copy is not read
            }
            if (hl == 0) a.out_scales[(size_t)r * (I / 32) + gg] = (uint8_t)(sx + 127);
          }
        } else if constexpr (DT == DT_NVFP4) {
          // two blocks of 16 along I: tp = 0 holds b = 0, 1; tp = 1 holds b = 2, 3
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            float amax = 0.f;
#pragma unroll
            for (int i = 8 * tp; i < 8 * tp + 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
            const uint32_t sc_code = e4m3_from_f32(amax / 6.0f);
            const float sc = e4m3_to_f32(sc_code);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
              const int b = 2 * tp + bb;
              uint32_t v = 0, d[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float x = h[4 * b + j];
                const uint32_t c = sc > 0.f ? e2m1_from_f32(x, sc) : ((__float_as_uint(x) >> 28) & 8u);
                v |= c << (4 * j);
                d[j] = f32_to_f16_bits(e2m1_to_f32(c) * sc);  // exact in fp16
              }
              if (ok) {
                *reinterpret_cast<uint16_t*>(a.out + (size_t)r * (I / 2) + 16 * gg + 4 * b + 2 * hl) = (uint16_t)v;
                *reinterpret_cast<uint2*>(a.out_deq + (size_t)r * I + 32 * gg + 8 * b + 4 * hl) =
                    make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
              }
            }
            if (ok && hl == 0) a.out_scales[(size_t)r * (I / 16) + 2 * gg + tp] = (uint8_t)sc_code;
          }
        }
      };
      // SwiGLU: one set of 32 intermediates (group g) from the gate (f = 0)
      // and up (f = 1) fragments.  ReLU^2: fragment f holds W1 rows 64g + 32f
      // + ..., the intermediates of half group 2g + f.  One copy of the store
      // code serves both (the fragment is selected, not indexed).
      const int halves = a.gated ? 1 : 2;
#pragma unroll 1
      for (int f = 0; f < halves; ++f) {
        float h[16];
        if (a.gated) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float gv = acc[0][S][i] * alpha, uv = acc[1][S][i] * alpha;
            if (a.limit > 0.f) {
              gv = fminf(gv, a.limit);
              uv = fminf(fmaxf(uv, -a.limit), a.limit);
            }
            // silu with the hardware exp and reciprocal (~1 ulp each): h is requantised
            // to at most 8 significant bits, so a code moves only within a few ulps of a midpoint
            h[i] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float t = fmaxf((f ? acc[1][S][i] : acc[0][S][i]) * alpha, 0.f);
            h[i] = t * t;
          }
        }
        store_h(h, a.gated ? g : 2 * g + f);
      }
    } else {
      if (ok) {
        const int p = a.sorted_pairs[r];
        if (a.red) {  // in-kernel fc2 reduce: w * y added to the token's fp32 output row
          const float wp = a.wts[p];
          float* o = a.red + (size_t)(p / a.k) * a.n_out + 64 * g + 4 * hl;
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
              for (int j = 0; j < 4; ++j) unsafeAtomicAdd(o + 32 * f + 8 * b + j, wp * (acc[f][S][4 * b + j] * alpha));
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (size_t)p * a.n_out + 64 * g + 4 * hl;
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const f32x16_t& v = acc[f][S];
              *reinterpret_cast<uint2*>(o + 32 * f + 8 * b) =
                  make_uint2(f32_to_bf16(v[4 * b] * alpha) | ((uint32_t)f32_to_bf16(v[4 * b + 1] * alpha) << 16),
                             f32_to_bf16(v[4 * b + 2] * alpha) | ((uint32_t)f32_to_bf16(v[4 * b + 3] * alpha) << 16));
            }
        }
      }
    }
  }
}

// One prefill work item.  `w` numbers items expert-major (pf_tile: bands of
// up to pf_band m-tiles, n-block-major inside a band, so that consecutive
// items share weight and token tiles; m-tile-major in load-balance mode 3,
// which only kernels instantiated with SPLIT run).  `cum` holds the
// per-expert ROWS-row m-tile prefix from build_schedule.  Returns the item's
// expert; ends with every load landed and the block's LDS free for reuse.
//
// TW (1 or 2) is the number of waves along the token dimension: the block
// has 4 TW waves; wave wv owns row group wv % 4 and every TW-th of the
// item's ROWS / 32 token sub-tiles, starting at wv / 4 (interleaved, so a
// partly filled m-tile still splits its rows evenly).  With TW = 2 and 256
// rows a wave's tile is 64 x 128 (128 accumulator registers) and two waves
// fit per SIMD, so one wave's LDS reads, loads and converts overlap the
// other's MFMAs; the 256-row tile halves the weight bytes loaded per flop.
template <int DT, bool G13, int TW, int ROWS, bool SPLIT = false>
__device__ __forceinline__ int prefill_item(const GemmArgs& a, long long w, const int* cum,
                                            const PfStages<pf_stage_slots<DT, ROWS>()>& st) {
  static_assert(TW == 1 || TW == 2, "waves along tokens");
  static_assert(ROWS == 128 || ROWS == 256, "rows per item");
  constexpr bool kALds = pf_alds<DT>();
  constexpr int kSlots = pf_stage_slots<DT, ROWS>();
  constexpr int kTokSlots = pf_tok_slots<ROWS>();
  constexpr int kSub = ROWS / 32;                   // token sub-tiles per item
  constexpr int kSW = kSub / TW;                    // token sub-tiles per wave
  constexpr int kDma = kSub / TW;                   // token loads per wave per K step (4 kSub per block)
  constexpr int kADma = 4 / TW;                     // LDS weights: code loads per wave per K step (16 per block)
  const int kBand = a.band > 0 ? max(1, a.band / ROWS) : pf_band<ROWS>();
  // vector-memory operations per wave per K step
  constexpr int kOps = kDma + (kALds ? kADma + 1 : pf_a_ops<DT>());
  constexpr int kPfStages = pf_stages<DT, ROWS>();
  const int tid = threadIdx.x, lane = tid & 63, i16 = lane & 15, hl = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wg = wv & 3, th = wv >> 2;
  const int NB = (a.G + kPfGroups - 1) / kPfGroups;
  const int KS = a.KG * 2;  // K steps of 64
  // w is the same for the whole block; said explicitly, else the compiler
  // takes the split deal's index for a per-lane value and builds the weight
  // buffer resources below in vector registers (a waterfall loop around
  // every load of the K loop).  Item counts stay far below 2^31.
  if constexpr (SPLIT) w = __builtin_amdgcn_readfirstlane((int)w);
  const int e = find_expert(cum, a.E, (int)(w / NB));
  int mt, nb;
  pf_tile<SPLIT>(w, NB, kBand, a.balance, cum, e, mt, nb);
  const int r0 = a.offsets[e] + mt * ROWS, r_end = a.offsets[e + 1];
  // this wave's row group; a group past the end (G not a multiple of 4) reads group G-1 and discards it
  const int g = kPfGroups * nb + wg, gl = min(g, a.G - 1);

  // Token loads: the block's 4 kSub per K step are (sub-tile d / 4, chunk
  // (d / 2) % 2, row half d % 2), d = 0..4 kSub - 1; this wave issues d =
  // wv kDma .. + kDma, all in sub-tile dS.  Load lane: row 16 half + lane / 4, the
  // row's 16-byte piece (lane % 4) ^ swizzle.  Rows past the expert's end
  // load its last row, whose results are discarded.
  // (byte offsets from a.act: the direct-to-LDS loads go through buffer
  // resources, see issue_op; the host keeps every offset below 2^31)
  const int dS = (wv * kDma) >> 2;
  uint32_t boff[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int rl = 16 * half + (lane >> 2);
    const int r = min(r0 + 32 * dS + rl, r_end - 1);
    const int row = G13 ? a.sorted_pairs[r] / a.k : r;
    const int piece = (lane & 3) ^ pf_swz(rl);
    boff[half] = ((uint32_t)row * (uint32_t)a.K + 8 * piece) * 2;
  }
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, 0x7FFFFFFF, 0x00020000);
  // fragment reads: row l32 of a block, piece 2m + hl
  int fro[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) fro[m] = 4 * l32 + ((2 * m + hl) ^ pf_swz(l32));

  // weights: lane part of the gathered fragment address
  constexpr size_t tcode = DT == DT_BF16 ? 4096 : DT == DT_MXFP8 ? 2048 : 1024;
  constexpr size_t tscale = DT == DT_MXFP8 ? 64 : 128;
  const int ltile = (lane >> 4) & 1, lpos = i16 + 16 * hl;  // lane position (l & 15) + 16 (2m + (l >> 5)), less 32m
  const size_t tile0 = (size_t)(e * a.G + gl) * a.KG * 4;  // tile index of (gl, kgroup 0, tile 0)
  const uint8_t* wc = a.wcodes + (tile0 + ltile) * tcode + lpos * 16;
  const uint8_t* ws = a.wscales + (tile0 + ltile) * tscale + i16 * (DT == DT_MXFP8 ? 4 : 8);
  // LDS-staged weights: buffer resources based at this row group's first tile (offsets within one group)
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.wcodes + tile0 * tcode), (short)0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t wsrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.wscales + tile0 * tscale), (short)0, 0x7FFFFFFF, 0x00020000);
  const uint32_t wlo = ltile * (uint32_t)tcode + lpos * 16;

  // Vector-memory operation k of K step `step`: k < kDma a token load into
  // `stage`; k >= kDma a piece of the weights into A.  The direct-to-LDS
  // loads use the buffer (MUBUF) form: the compiler tracks those with the
  // vector-memory counter alone, while the global form also counts as a
  // possible LDS access and made it wait for every LDS read before each
  // slice's MFMAs as long as one was in flight.
  auto issue_op = [&](int k, u32x4_t(&stage)[kSlots], PfA<DT>& A, int step) {
    if (k < kDma) {
      const int d = wv * kDma + k, cc = (d >> 1) & 1, half = k & 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          brs, (__attribute__((address_space(3))) void*)&stage[((2 * dS + cc) * 2 + half) * 64], 16,
          boff[half] + step * 128 + cc * 64, 0, 0, 0);
      return;
    }
    const int kg = step >> 1, h = step & 1, idx = k - kDma;
    const size_t tk = (size_t)kg * 4;  // tile offset of the kgroup
    if constexpr (kALds) {
      if (idx < kADma) {
        // codes of fragment pair (f, m) of this row group, in fragment-lane order
        const int f = TW == 2 ? th : (idx >> 1), m = TW == 2 ? idx : (idx & 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wrs, (__attribute__((address_space(3))) void*)&stage[kTokSlots + ((wg * 2 + f) * 2 + m) * 64], 16,
            wlo + (uint32_t)((tk + 2 * f) * tcode + h * 1024 + m * 512), 0, 0, 0);
      } else {
        // this wave's copy of the group's 4 tile scale blocks (256 contiguous bytes)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wsrs, (__attribute__((address_space(3))) void*)&stage[kTokSlots + 1024 + wv * 16], 4,
            (uint32_t)(tk * tscale) + lane * 4, 0, 0, 0);
      }
      return;
    }
    if constexpr (DT == DT_BF16) {
      const int f = idx >> 2, cc = (idx >> 1) & 1, m = idx & 1;
      A.c[f][cc][m] = *reinterpret_cast<const u32x4_t*>(wc + (tk + 2 * f) * tcode + (2 * h + cc) * 1024 + m * 512);
    } else if (idx < 4) {
      const int f = idx >> 1, m = idx & 1;
      if constexpr (DT == DT_MXFP8)
        A.c[f][m] = *reinterpret_cast<const u32x4_t*>(wc + (tk + 2 * f) * tcode + h * 1024 + m * 512);
      else
        A.c[f][m] = *reinterpret_cast<const u32x2_t*>(wc + (tk + 2 * f) * tcode + m * 512 + 8 * h);
    } else {
      const int f = idx - 4;
      A.s[f] = *reinterpret_cast<const uint32_t*>(ws + (tk + 2 * f) * tscale + (DT == DT_MXFP8 ? 0 : 4 * h));
    }
  };
  auto issue_all = [&](u32x4_t(&stage)[kSlots], PfA<DT>& A, int step) {
#pragma unroll
    for (int k = 0; k < kOps; ++k) issue_op(k, stage, A, step);
  };

  // The K loop with NSA of this wave's sub-tiles active (the rest of the
  // m-tile lies past the expert's rows and is skipped; its loads still
  // issue, clamped, so every wave keeps the same operation count per step).
  auto run = [&](auto nsa_tag) {
    constexpr int NSA = decltype(nsa_tag)::value;
    constexpr int kMfma = 8 * NSA;  // MFMAs per K step
    f32x16_t acc[2][kSW];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int S = 0; S < NSA; ++S)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][S][i] = 0.f;

    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short op_t;
    // weight fragments f = 0, 1 of K slice (chunk cc, m), converted
    auto convert = [&](op_t(&af)[2], const PfA<DT>& A, int h, int cc, int m) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if constexpr (DT == DT_BF16) {
          af[f] = (op_t)A.c[f][cc][m];
        } else if constexpr (DT == DT_MXFP8) {
          af[f] = (op_t)mxfp8_dequant8(A.c[f][m][2 * cc], A.c[f][m][2 * cc + 1], (A.s[f] >> (8 * (2 * h + cc))) & 0xFF);
        } else {
          af[f] = (op_t)nvfp4_dequant8(A.c[f][m][cc], (A.s[f] >> (8 * (2 * cc + m))) & 0xFF);
        }
      }
    };
    // token fragments of the active sub-tiles, K slice (chunk cc, m)
    auto read_b = [&](u32x4_t(&bf)[kSW], const u32x4_t(&stage)[kSlots], int cc, int m) {
#pragma unroll
      for (int S = 0; S < NSA; ++S) bf[S] = stage[(2 * (TW * S + th) + cc) * 128 + fro[m]];
    };

    // Operands of slice 0 of a step, read ahead across the step boundary:
    // the LDS weights (codes and scales) and the first token fragments.
    struct Carry {
      PfA<DT> AL;
      u32x4_t bf0[kSW];
    };
    auto prefetch = [&](Carry& cr, const u32x4_t(&stage)[kSlots]) {
      if constexpr (kALds) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
          for (int m = 0; m < 2; ++m) cr.AL.c[f][m] = stage[kTokSlots + ((wg * 2 + f) * 2 + m) * 64 + lane];
          cr.AL.s[f] = reinterpret_cast<const uint32_t*>(&stage[kTokSlots + 1024 + wv * 16])[(2 * f + ltile) * 16 + i16];
        }
      }
      read_b(cr.bf0, stage, 0, 0);
    };
    // loads issued before the mid-step barrier (interleave positions in slices 0..2)
    constexpr int kMidOps = [] {
      int n = 0;
      for (int k = 0; k < kOps; ++k)
        if (NSA == 0 || (k * kMfma) / kOps < 6 * NSA) ++n;
      return n;
    }();
    // Step t needs step t+1 landed (for every wave) at its mid barrier: at
    // most the NS-3 steps after t+1 and the part of step t+NS-1 issued so far
    // may still be in flight.
    constexpr int kMidWait = kOps * (kPfStages - 3) + kMidOps;

    // One K step: 4 K slices x 2 NSA MFMAs on `stage` / A, each slice's
    // operands fetched one slice ahead, the loads of step `nstep` spread
    // between the MFMAs so the memory pipeline accepts them while the matrix
    // unit is busy.  After slice 2: wait for step t+1, barrier, and read its
    // slice-0 operands (from `next`) while slice 3 computes.
    auto step_body = [&](const u32x4_t(&stage)[kSlots], const PfA<DT>& A, int step, Carry& cr,
                         const u32x4_t(&next)[kSlots], PfA<DT>& nextA, u32x4_t(&nstage)[kSlots], PfA<DT>& nA,
                         int nstep) {
      if constexpr (NSA == 0) {
        issue_all(nstage, nA, nstep);
        pf_wait_barrier<kMidWait>();
        return;
      }
      const int h = step & 1;
      op_t af[2][2];
      u32x4_t bf[2][kSW];
      const PfA<DT>& Aop = kALds ? cr.AL : A;
      convert(af[0], Aop, h, 0, 0);
#pragma unroll
      for (int S = 0; S < NSA; ++S) bf[0][S] = cr.bf0[S];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (sl < 3) {
          read_b(bf[(sl + 1) & 1], stage, (sl + 1) >> 1, (sl + 1) & 1);
          convert(af[(sl + 1) & 1], Aop, h, (sl + 1) >> 1, (sl + 1) & 1);
        } else {
          pf_wait_barrier<kMidWait>();
          if constexpr (!kALds) pf_pin(nextA);
          prefetch(cr, next);
        }
#pragma unroll
        for (int mm = 0; mm < 2 * NSA; ++mm) {
          const int f = mm / NSA, S = mm % NSA, gm = sl * 2 * NSA + mm;
          f32x16_t& c = acc[f][S];
          if constexpr (DT == DT_NVFP4)
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16((f16x8_t)af[sl & 1][f], (f16x8_t)bf[sl & 1][S], c, 0, 0, 0);
          else
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16((bf16x8_t)af[sl & 1][f], (bf16x8_t)bf[sl & 1][S], c, 0, 0, 0);
#pragma unroll
          for (int k = 0; k < kOps; ++k) {
            if (gm == (k * kMfma) / kOps) {
              __builtin_amdgcn_sched_barrier(0);
              issue_op(k, nstage, nA, nstep);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
    };

    // prologue: steps 0 .. NS-2 in flight (every wave issues the same number
    // of operations each step, clamped to the last step past the end), then
    // wait for step 0 and read its slice-0 operands
    PfA<DT> A[kPfStages];
#pragma unroll
    for (int i = 0; i < kPfStages - 1; ++i) {
      issue_all(*st.s[i], A[i], min(i, KS - 1));
      asm volatile("" ::: "memory");  // each step's operations issue after the previous step's
    }
    Carry cr;
    pf_wait_barrier<kOps * (kPfStages - 2)>();
    if constexpr (!kALds) pf_pin(A[0]);
    prefetch(cr, *st.s[0]);
    int s = 0;
    for (; s + kPfStages <= KS; s += kPfStages) {
#pragma unroll
      for (int u = 0; u < kPfStages; ++u) {
        const int nxt = (u + kPfStages - 1) % kPfStages;
        step_body(*st.s[u], A[u], s + u, cr, *st.s[(u + 1) % kPfStages], A[(u + 1) % kPfStages], *st.s[nxt], A[nxt],
                  min(s + u + kPfStages - 1, KS - 1));
      }
    }
    if (s < KS) {  // the last KS % NS steps; every body still issues its (clamped) operations and barrier
#pragma unroll
      for (int u = 0; u < kPfStages - 1; ++u) {
        const int nxt = (u + kPfStages - 1) % kPfStages;
        const int nstep = min(s + u + kPfStages - 1, KS - 1);
        if (s + u < KS) {
          step_body(*st.s[u], A[u], s + u, cr, *st.s[(u + 1) % kPfStages], A[(u + 1) % kPfStages], *st.s[nxt], A[nxt],
                    nstep);
        } else {
          issue_all(*st.s[nxt], A[nxt], nstep);
          pf_wait_barrier<kMidWait>();
        }
      }
    }
    pf_wait_barrier<0>();
    if constexpr (NSA > 0)
      if (g < a.G) pf_epilogue<DT, G13, NSA, kSW, 32 * TW>(a, acc, r0 + 32 * th, r_end, g, e, lane);
  };
  // this wave's active 32-row sub-tiles th, th + TW, ... (uniform across the wave)
  const int nact = min(kSub, (r_end - r0 + 31) >> 5);
  const int nsa = min(kSW, max(0, (nact - th + TW - 1) / TW));
  if constexpr (TW == 1) {
    switch (nsa) {
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  } else if constexpr (kSW == 2) {
    switch (nsa) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 2>{}); break;
    }
  } else {
    switch (nsa) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  }
  // Drain the epilogue's stores: with stores and loads both pending, the
  // shared vector-memory counter no longer counts loads in order, and the
  // compiler would wait for everything at the next item's K-loop head.
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
  return e;
}

}  // namespace moe
