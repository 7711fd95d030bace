// The prefill-shaped grouped-GEMM work item, shared by the stage kernel
// (moe_prefill.hip) and the fused single-launch kernel.
//
// Item = (expert, m-tile of 128 sorted rows, n-block of 4 weight row groups
// = 256 weight rows).  The block's 4 waves each own one row group (its 4
// packed 16-row tiles) and all 128 token rows: a 64 x 128 wave tile of
// 16x16x32 MFMAs, accumulated over K in order.
//
//  * Weights stream from global memory straight into registers (each weight
//    element is used by exactly one wave): a ring of kPfStages K steps.
//  * Token rows are shared by the 4 waves through LDS, filled by the 16-byte
//    direct global->LDS load (no register round trip) into a ring of
//    kPfStages stages, each one 64-wide K step in the matrix instruction's
//    lane order.
//  * One barrier per K step.  Loads for step s+kPfStages-1 are issued when
//    step s starts, so kPfStages-1 steps of MFMA work cover their latency;
//    the wait before the barrier counts outstanding vector-memory operations
//    explicitly.
#pragma once

#include "moe_gemm_item.h"

namespace moe {

constexpr int kPfRows = 128;                  // routed rows per item: 8 sub-tiles of 16
constexpr int kPfGroups = 4;                  // weight row groups per item, one per wave
constexpr int kPfBand = 8;                    // m-tiles per band of the item order
constexpr int kPfStageSlots = 8 * 2 * 64;     // token stage: [sub-tile][chunk][lane] x 16 B = 16 KB
constexpr int kPfStepOps = 12;                // vector-memory operations per wave per K step
constexpr int kPfStages = 4;                  // pipeline depth: K steps in flight + the one computed

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// One K step (64 wide) of this wave's 4 weight tiles, as loaded.
template <int DT>
struct PfA;
template <>
struct PfA<DT_BF16> {
  u32x4_t c[4][2];  // [tile][chunk]: 8 bf16 per lane
};
template <>
struct PfA<DT_MXFP8> {
  u32x4_t c[4];   // [tile]: chunk 0 in words 0-1, chunk 1 in words 2-3 (8 e4m3 each)
  uint32_t s[4];  // [tile]: the row's 4 e8m0 scales of the kgroup
};
template <>
struct PfA<DT_NVFP4> {
  u32x2_t c[4];   // [tile]: 8 e2m1 of chunk 0, of chunk 1
  uint32_t s[4];  // [tile]: the row's 4 e4m3 scales of this half kgroup
};

// Blocks are dealt to the 8 XCDs (each with its own L2) round-robin by
// block index.  Renumbering so that each XCD holds a contiguous range of
// logical ids makes neighbouring items -- which share weight or token tiles
// -- run on the same L2.
__device__ __forceinline__ int xcd_logical_block() {
  const int b = blockIdx.x, g = gridDim.x;
  return g % 8 == 0 ? (b % 8) * (g / 8) + b / 8 : b;
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
  for (int t = 0; t < 4; ++t) {
    if constexpr (DT == DT_BF16) {
      asm volatile("" : "+v"(A.c[t][0]), "+v"(A.c[t][1]));
    } else {
      asm volatile("" : "+v"(A.c[t]), "+v"(A.s[t]));
    }
  }
}

// The token stages of one block (separate LDS objects, so the compiler's
// waits for the direct loads track each stage on its own).
struct PfStages {
  u32x4_t (*s[kPfStages])[kPfStageSlots];
};

// One prefill work item.  `w` numbers items expert-major; within an expert,
// bands of up to kPfBand m-tiles, n-block-major inside a band, so kPfBand^2
// consecutive items form a square of weight x token tiles.  `cum` holds the
// per-expert 128-row m-tile prefix from build_schedule.  Returns the item's
// expert; ends with every load landed and the block's LDS free for reuse.
template <int DT, bool G13>
__device__ __forceinline__ int prefill_item(const GemmArgs& a, long long w, const int* cum, const PfStages& st) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, i16 = lane & 15, q = lane >> 4;
  const int NB = (a.G + kPfGroups - 1) / kPfGroups;
  const int KS = a.KG * 2;  // K steps of 64
  const int e = find_expert(cum, a.E, (int)(w / NB));
  const int mts = cum[e + 1] - cum[e];
  const long long local = w - (long long)cum[e] * NB;
  const int band = (int)(local / (kPfBand * NB)), full = mts / kPfBand;
  const int bsize = band < full ? kPfBand : mts - full * kPfBand;
  const int inner = (int)(local - (long long)band * kPfBand * NB);
  const int nb = inner / bsize, mt = band * kPfBand + inner % bsize;
  const int r0 = a.offsets[e] + mt * kPfRows, r_end = a.offsets[e + 1];
  // this wave's row group; a group past the end (G not a multiple of 4) reads group G-1 and discards it
  const int g = kPfGroups * nb + wv, gl = min(g, a.G - 1);

  // token rows of the two sub-tiles this wave loads (2wv, 2wv+1); rows past
  // the expert's end load its last row, whose results are discarded
  const uint8_t* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = min(r0 + 16 * (2 * wv + j) + i16, r_end - 1);
    const int row = G13 ? a.sorted_pairs[r] / a.k : r;
    bsrc[j] = a.act + ((size_t)row * a.K + 8 * q) * 2;
  }
  const size_t tile0 = (size_t)(e * a.G + gl) * a.KG * 4;  // tile index of (gl, kgroup 0, tile 0)
  // Vector-memory operation k (0..11) of K step `step`: k < 4 the token
  // rows of sub-tile 2wv + k/2, chunk k%2 into `stage`; k >= 4 a piece of
  // weight tile (k-4)/2 into A.
  auto issue_op = [&](int k, u32x4_t(&stage)[kPfStageSlots], PfA<DT>& A, int step) {
    if (k < 4) {
      const int j = k >> 1, c = k & 1;
      __builtin_amdgcn_global_load_lds(bsrc[j] + step * 128 + c * 64, &stage[((2 * wv + j) * 2 + c) * 64], 16, 0, 0);
      return;
    }
    const int t = (k - 4) >> 1, part = (k - 4) & 1, kg = step >> 1, h = step & 1;
    const size_t ti = tile0 + (size_t)kg * 4 + t;
    if constexpr (DT == DT_BF16) {
      A.c[t][part] = *reinterpret_cast<const u32x4_t*>(a.wcodes + ti * 4096 + (2 * h + part) * 1024 + lane * 16);
    } else if constexpr (DT == DT_MXFP8) {
      if (part == 0) A.c[t] = *reinterpret_cast<const u32x4_t*>(a.wcodes + ti * 2048 + h * 1024 + lane * 16);
      else A.s[t] = *reinterpret_cast<const uint32_t*>(a.wscales + ti * 64 + i16 * 4);
    } else {
      if (part == 0) A.c[t] = *reinterpret_cast<const u32x2_t*>(a.wcodes + ti * 1024 + lane * 16 + 8 * h);
      else A.s[t] = *reinterpret_cast<const uint32_t*>(a.wscales + ti * 128 + i16 * 8 + 4 * h);
    }
  };
  auto issue_all = [&](u32x4_t(&stage)[kPfStageSlots], PfA<DT>& A, int step) {
#pragma unroll
    for (int k = 0; k < kPfStepOps; ++k) issue_op(k, stage, A, step);
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[t][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short op_t;
  // matrix operands of chunk j (0, 1) of a step: the 4 weight tiles, converted
  auto convert = [&](op_t(&af)[4], const PfA<DT>& A, int h, int j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DT == DT_BF16) {
        af[t] = (op_t)A.c[t][j];
      } else if constexpr (DT == DT_MXFP8) {
        af[t] = (op_t)mxfp8_dequant8(A.c[t][2 * j], A.c[t][2 * j + 1], (A.s[t] >> (8 * (2 * h + j))) & 0xFF);
      } else {
        af[t] = (op_t)nvfp4_dequant8(A.c[t][j], (A.s[t] >> (8 * (2 * j + (q >> 1)))) & 0xFF);
      }
    }
  };
  // token operands of chunk j, sub-tiles 4sh .. 4sh+3
  auto read_b = [&](u32x4_t(&bf)[4], const u32x4_t(&stage)[kPfStageSlots], int j, int sh) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) bf[s4] = stage[((4 * sh + s4) * 2 + j) * 64 + lane];
  };

  // One K step: 64 MFMAs on `stage` / A in four quarters (chunk j, sub-tile
  // half sh), the next quarter's token fragments read ahead, and the 12
  // loads of step `nstep` spread one per five MFMAs so the memory pipeline
  // accepts them while the matrix unit is busy.
  auto step_body = [&](const u32x4_t(&stage)[kPfStageSlots], const PfA<DT>& A, int step,
                       u32x4_t(&nstage)[kPfStageSlots], PfA<DT>& nA, int nstep) {
    const int h = step & 1;
    op_t af[2][4];
    u32x4_t bf[2][4];
    convert(af[0], A, h, 0);
    read_b(bf[0], stage, 0, 0);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int j = qq >> 1, sh = qq & 1;
      if (qq < 3) read_b(bf[(qq + 1) & 1], stage, (qq + 1) >> 1, (qq + 1) & 1);
      if (qq == 1) convert(af[1], A, h, 1);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int s4 = m >> 2, t = m & 3, gm = qq * 16 + m;
        f32x4_t& c = acc[t][4 * sh + s4];
        if constexpr (DT == DT_NVFP4)
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16((f16x8_t)af[j][t], (f16x8_t)bf[qq & 1][s4], c, 0, 0, 0);
        else
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)af[j][t], (bf16x8_t)bf[qq & 1][s4], c, 0, 0, 0);
        if (gm % 5 == 4 && gm / 5 < kPfStepOps) {
          __builtin_amdgcn_sched_barrier(0);
          issue_op(gm / 5, nstage, nA, nstep);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // prologue: steps 0 .. NS-2 in flight (every wave issues the same number
  // of operations each step, clamped to the last step past the end)
  PfA<DT> A[kPfStages];
#pragma unroll
  for (int i = 0; i < kPfStages - 1; ++i) {
    issue_all(*st.s[i], A[i], min(i, KS - 1));
    asm volatile("" ::: "memory");  // each step's operations issue after the previous step's
  }
  int s = 0;
  for (; s + kPfStages <= KS; s += kPfStages) {
#pragma unroll
    for (int u = 0; u < kPfStages; ++u) {
      // step s+u has landed once at most the NS-2 newer steps are in flight
      pf_wait_barrier<kPfStepOps * (kPfStages - 2)>();
      pf_pin(A[u]);
      const int nxt = (u + kPfStages - 1) % kPfStages;
      step_body(*st.s[u], A[u], s + u, *st.s[nxt], A[nxt], min(s + u + kPfStages - 1, KS - 1));
    }
  }
  if (s < KS) {  // the last KS % NS steps; every body still issues its 12 (clamped) operations
#pragma unroll
    for (int u = 0; u < kPfStages - 1; ++u) {
      pf_wait_barrier<kPfStepOps * (kPfStages - 2)>();
      pf_pin(A[u]);
      const int nxt = (u + kPfStages - 1) % kPfStages;
      const int nstep = min(s + u + kPfStages - 1, KS - 1);
      if (s + u < KS) step_body(*st.s[u], A[u], s + u, *st.s[nxt], A[nxt], nstep);
      else issue_all(*st.s[nxt], A[nxt], nstep);
    }
  }
  pf_wait_barrier<0>();
  if (g < a.G) gemm_epilogue<DT, 8, G13>(a, acc, r0, r_end, g, e, lane);
  // Drain the epilogue's stores: with stores and loads both pending, the
  // shared vector-memory counter no longer counts loads in order, and the
  // compiler would wait for everything at the next item's K-loop head.
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
  return e;
}

}  // namespace moe
