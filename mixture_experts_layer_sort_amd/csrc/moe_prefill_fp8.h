// The prefill-shaped grouped-GEMM work item of MXFP8 layers on the gfx950
// block-scaled fp8 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3
// operands, one e8m0 scale per 32 along K per row and per token), shared by
// the stage kernel (moe_prefill.hip) and the single-launch kernel.
//
// The instruction applies the MX block scales itself, so the e4m3 codes of
// the weights (packed in fragment order by moe_prepare_weights) and of the
// quantised activations (xq / hq rows as the quantisers wrote them) feed the
// matrix unit without any conversion, at twice the bf16 rate and half the
// operand bytes.  Operand layout of one 32-row x 64-K fragment (measured on
// MI355X): lane l = m + 32h holds row m, K bytes [16h, 16h+16) in VGPRs 0-3
// and [32+16h, 32+16h+16) in VGPRs 4-7; the scale of row m's K block b (32
// wide) is read from lane m + 32b.  Measured accuracy: a 7168-long dot product
// of MX-quantised N(0,1) x N(0,0.02) data has relative L2 error 1.4e-5 against
// the exact sum (the fp32 accumulation into C is exact-rounded; the error is
// inside the 64-product sum), so the requantised intermediate differs from
// the oracle's only where a value sits next to a rounding midpoint.
//
// Item = (expert, m-tile of 256 sorted rows, n-block of 4 weight row groups
// = 256 weight rows).  Each of the block's 4 waves owns one 64-row group
// (gate/up GEMM: 32 gate rows then the matching 32 up rows) and all 256
// routed rows: a 64 x 256 wave tile, 2 x 8 fragments, 256 fp32 accumulators.
//  * Weights go from global memory straight into registers (each weight row
//    is used by exactly one wave): a ring of 3 kgroups (128 K), loads issued
//    two kgroups ahead.  Each 1 KB load is one contiguous wave-wide dwordx4.
//  * Token codes and their scale words are shared by the 4 waves through
//    LDS, filled by direct global->LDS loads into a ring of 3 stages of one
//    kgroup: per (32-row sub-tile, 64-K step) block, 64 B rows with their
//    16-byte pieces XOR-swizzled by (row >> 2) & 3 (conflict-free fragment
//    reads), then each token's 4 e8m0 scales of the kgroup.
//  * One barrier per kgroup, after an explicit wait for this wave's loads of
//    the kgroup (the loads of the next two kgroups stay in flight).
#pragma once

#include <type_traits>

#include "moe_prefill_item.h"

namespace moe {

constexpr int kF8Rows = 256;    // routed rows per item
constexpr int kF8Sub = 8;       // 32-row token sub-tiles per item
constexpr int kF8Stages = 3;    // token stages (kgroups) in LDS
constexpr int kF8ARing = 3;     // weight kgroups in registers
// 16-byte slots of one stage: token codes [sub-tile 8][step 2][row 32][4 pieces], then [token 256][4 e8m0]
constexpr int kF8TokSlots = kF8Sub * 2 * 32 * 4;
constexpr int kF8StageSlots = kF8TokSlots + kF8Rows * 4 / 16;
// vector-memory operations per wave per kgroup: weights 2 steps x 2 fragments x 2 halves + 2 scale
// words; token codes 8 (of the block's 32) + 1 scale load (of 4)
constexpr int kF8AOps = 10;
constexpr int kF8TOps = 9;

// Byte offset of the fragment-order weight unit (expert e, row group g, 64-K
// step s, fragment f, half q, lane l) in the fp8 fragment region: groups of
// KS = K / 64 steps, 4 KB per (group, step).
__host__ __device__ inline size_t f8_unit_offset(int e, int G, int g, int KS, int s, int f, int q, int l) {
  return (((((size_t)e * G + g) * KS + s) * 2 + f) * 2 + q) * 1024 + (size_t)l * 16;
}

template <int I>
__device__ __forceinline__ u32x4_t (*f8_stage())[kF8StageSlots] {
  __shared__ u32x4_t buf[kF8StageSlots];
  return &buf;
}

// Pair index of each routed row of the item (down GEMM epilogue).
__device__ __forceinline__ int (*f8_pidx())[kF8Rows] {
  __shared__ int buf[kF8Rows];
  return &buf;
}

struct F8Stages {
  u32x4_t (*s[kF8Stages])[kF8StageSlots];
};

__device__ __forceinline__ F8Stages f8_make_stages() {
  static_assert(kF8Stages == 3, "stages");
  F8Stages st{};
  st.s[0] = f8_stage<0>();
  st.s[1] = f8_stage<1>();
  st.s[2] = f8_stage<2>();
  return st;
}

typedef int f8op_t __attribute__((ext_vector_type(8)));

// Weight operands of one kgroup: [step][fragment] 32 code bytes (two 16-byte
// halves) and the fragment rows' 4 scale bytes.
struct F8A {
  u32x4_t c[2][2][2];  // [step][f][q]
  uint32_t s[2];       // [f]
};

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS operations are done, then barrier.
template <int N>
__device__ __forceinline__ void f8_wait_barrier() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Down-GEMM epilogue: bf16 y rows of the pairs of the item's `nrows` routed
// rows; pidx (LDS, filled at the start of the item so the loads' latency
// hides behind the K loop) holds the pair index of each.  Lane l, element i
// of acc[f][S] is weight row 32 f + (i & 3) + 8 (i >> 2) + 4 (l >> 5) of row
// group g, routed row 32 S + (l & 31) (the 32x32 accumulator layout).
//
// The accumulator layout gives each lane 16-byte pieces of 32 different y
// rows per store; written straight out, every store instruction touches 32
// cache lines.  Instead each wave turns its 64-column slice around in LDS
// (the token stages are free once the K loop is done): up to 4 sub-tiles at
// a time, 128 rows x 128 bytes in the wave's own 16 KB, 16-byte chunk j of
// row r at slot j ^ (r & 7) (conflict-free writes of 8-byte pieces and reads
// of whole rows), then each store instruction writes 8 whole 128-byte row
// segments (one cache line each).  The caller ends the item with a block
// barrier before the next item's loads refill the stages.
template <int NSA>
__device__ __forceinline__ void f8_down_epilogue(const GemmArgs& a, f32x16_t (&acc)[2][kF8Sub], const int* pidx,
                                                 int nrows, int g, int lane, int wv, const F8Stages& st) {
  const int hl = lane >> 5, m = lane & 31;
  if (a.red) {  // in-kernel fc2 reduce: w * y added to the token's fp32 output row
#pragma unroll
    for (int S = 0; S < NSA; ++S) {
      if (32 * S + m < nrows) {
        const int p = pidx[32 * S + m];
        const float wp = a.wts[p];
        float* o = a.red + (size_t)(p / a.k) * a.n_out + 64 * g + 4 * hl;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int i = 0; i < 16; ++i) unsafeAtomicAdd(o + 32 * f + 8 * (i >> 2) + (i & 3), wp * acc[f][S][i]);
      }
    }
    return;
  }
  // (a select, not an indexed load: indexing st would place it in memory)
  u32x4_t* buf = &(*(wv < 2 ? st.s[0] : st.s[1]))[(wv & 1) * 1024];  // 1024 slots of 16 bytes
  uint2* b64 = reinterpret_cast<uint2*>(buf);
  // Lane-dependent address parts, opaque to the compiler here so that the
  // per-store addresses are formed in place rather than hoisted out of the
  // item loop (dozens of loop-invariant registers, spilled across the K loop)
  int xm = m & 7, rl = lane >> 3, c8 = lane & 7;
  asm volatile("" : "+v"(xm), "+v"(rl), "+v"(c8));
  const int rslot = rl * 8 + (c8 ^ rl);  // read slot of chunk c8 of row rl
  uint16_t* y = reinterpret_cast<uint16_t*>(a.out) + 64 * g + 8 * c8;
#pragma unroll
  for (int p = 0; p < (NSA + 3) / 4; ++p) {
    constexpr int kPass = 4;
#pragma unroll
    for (int S = kPass * p; S < NSA && S < kPass * p + kPass; ++S) {
      uint2* wrow = b64 + (256 * (S - kPass * p) + 8 * m) * 2 + hl;  // row 32 (S - kPass p) + m
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x16_t& v = acc[f][S];
          wrow[((4 * f + b) ^ xm) * 2] =
              make_uint2(f32_to_bf16(v[4 * b]) | ((uint32_t)f32_to_bf16(v[4 * b + 1]) << 16),
                         f32_to_bf16(v[4 * b + 2]) | ((uint32_t)f32_to_bf16(v[4 * b + 3]) << 16));
        }
    }
    // 8 rows per store: lane l reads chunk l % 8 of row 8 j + l / 8 (all
    // reads first, so their latencies overlap; then the stores)
    const int nj = 4 * (NSA - kPass * p < kPass ? NSA - kPass * p : kPass);  // a constant once unrolled
    u32x4_t v[4 * kPass];
    int pid[4 * kPass];
#pragma unroll
    for (int j = 0; j < nj; ++j) {
      v[j] = buf[64 * j + rslot];
      pid[j] = pidx[32 * kPass * p + 8 * j + rl];
    }
#pragma unroll
    for (int j = 0; j < nj; ++j)
      if (32 * kPass * p + 8 * j + rl < nrows) *reinterpret_cast<u32x4_t*>(y + (size_t)pid[j] * a.n_out) = v[j];
  }
}

// One fp8 prefill work item.  `w` numbers items as the 128-row prefill items
// do (expert-major, bands of m-tiles, n-block-major inside a band); `cum`
// holds the per-expert 256-row m-tile prefix.  a.wcodes is the fragment-order
// weight region, a.act the e4m3 activation codes (row = token for the gate/up
// GEMM, sorted row for the down GEMM), a.act_scales their e8m0 scales.
// Returns the item's expert; ends with every load landed and the block's LDS
// free for reuse.
template <bool G13>
__device__ __forceinline__ int f8_item(const GemmArgs& a, long long w, const int* cum, const F8Stages& st) {
  const int kBand = a.band > 0 ? max(1, a.band / kF8Rows) : pf_band<kF8Rows>();
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 31, hl = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NB = (a.G + kPfGroups - 1) / kPfGroups;
  const int KG = a.KG, KS = 2 * a.KG;
  const int e = find_expert(cum, a.E, (int)(w / NB));
  int mt, nb;
  pf_tile<false>(w, NB, kBand, a.balance, cum, e, mt, nb);
  const int r0 = a.offsets[e] + mt * kF8Rows, r_end = a.offsets[e + 1];
  // this wave's row group; a group past the end (G not a multiple of 4) reads group G-1 and discards it
  const int g = kPfGroups * nb + wv, gl = min(g, a.G - 1);

  // Token code loads: the block's 32 per kgroup are (sub-tile S, step s, row
  // half) = (c / 4, (c / 2) % 2, c % 2), c = 0..31; this wave issues c = 8 wv
  // .. 8 wv + 7 (sub-tiles 2 wv, 2 wv + 1).  Lane L loads row 16 half + L / 4
  // of the sub-tile, piece (L % 4) ^ swizzle.  Rows past the expert's end
  // load its last row (results discarded).
  // (byte offsets from a.act / a.act_scales: the loads go through buffer
  // resources, see issue_t; the host keeps every offset below 2^31)
  uint32_t toff[2][2];
#pragma unroll
  for (int S2 = 0; S2 < 2; ++S2)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int rl = 16 * half + (lane >> 2);
      const int r = min(r0 + 32 * (2 * wv + S2) + rl, r_end - 1);
      const int row = G13 ? a.sorted_pairs[r] / a.k : r;
      toff[S2][half] = (uint32_t)row * (uint32_t)a.K + 16 * ((lane & 3) ^ pf_swz(rl));
    }
  // token scale words: this wave loads tokens 64 wv .. +64 of the item, 4 bytes each
  uint32_t soff;
  {
    const int r = min(r0 + 64 * wv + lane, r_end - 1);
    const int row = G13 ? a.sorted_pairs[r] / a.k : r;
    soff = (uint32_t)row * (uint32_t)(a.K / 32);
  }
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act_scales, (short)0, 0x7FFFFFFF, 0x00020000);
  // down GEMM: the pair index of each routed row of the item, straight into
  // LDS for the epilogue (issued before the kgroup loads, so the K loop's
  // waits cover it); rows past the expert's end repeat its last row
  int* pidx = *f8_pidx();
  if constexpr (!G13) {
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.sorted_pairs, (short)0, 0x7FFFFFFF, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (__attribute__((address_space(3))) void*)&pidx[64 * wv], 4,
                                             (uint32_t)min(r0 + 64 * wv + lane, r_end - 1) * 4u, 0, 0, 0);
  }
  // weights: this lane's unit of (gl, step 0, f 0, q 0), and its scale word of (gl, kgroup 0, f 0)
  const uint8_t* wsrc = a.wcodes + f8_unit_offset(e, a.G, gl, KS, 0, 0, 0, lane);
  const uint8_t* wssrc = a.wscales + ((size_t)e * a.G + gl) * KG * 256 + m * 4;

  auto issue_a = [&](F8A& A, int kg) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          A.c[s][f][q] = *reinterpret_cast<const u32x4_t*>(wsrc + ((size_t)(2 * kg + s) * 4 + f * 2 + q) * 1024);
#pragma unroll
    for (int f = 0; f < 2; ++f) A.s[f] = *reinterpret_cast<const uint32_t*>(wssrc + (size_t)kg * 256 + f * 128);
  };
  // Token loads straight into LDS through buffer resources (the MUBUF form:
  // the compiler then tracks them with the vector-memory counter alone; the
  // global form is also counted as a possible LDS access, which made it wait
  // for every LDS read before each MFMA while any of these were in flight).
  auto issue_t = [&](u32x4_t(&stage)[kF8StageSlots], int kg) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * wv + i, S = c >> 2, s = (c >> 1) & 1, half = c & 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          trs, (__attribute__((address_space(3))) void*)&stage[((S * 2 + s) * 2 + half) * 64], 16,
          toff[i >> 2][half] + kg * 128 + s * 64, 0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        srs, (__attribute__((address_space(3))) void*)&stage[kF8TokSlots + 16 * wv], 4, soff + 4 * kg, 0, 0, 0);
  };

  auto run = [&](auto nsa_tag) {
    constexpr int NSA = decltype(nsa_tag)::value;
    f32x16_t acc[2][kF8Sub];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int S = 0; S < NSA; ++S)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][S][i] = 0.f;

    F8A A[kF8ARing];
    // prologue: weights and tokens of kgroups 0 and 1 in flight
    issue_a(A[0], 0);
    issue_t(*st.s[0], 0);
    issue_a(A[1], min(1, KG - 1));
    issue_t(*st.s[1], min(1, KG - 1));

    // Keep the uses of a kgroup's weight registers below the wait + barrier
    // that guarantees them (otherwise the register-only scale shifts are
    // hoisted above it and the compiler adds a full wait of its own).
    auto pin = [&](F8A& Ak) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
#pragma unroll
        for (int f = 0; f < 2; ++f) asm volatile("" : "+v"(Ak.c[ss][f][0]), "+v"(Ak.c[ss][f][1]));
      asm volatile("" : "+v"(Ak.s[0]), "+v"(Ak.s[1]));
    };
    auto body = [&](const F8A& Ak, const u32x4_t(&stage)[kF8StageSlots]) {
      // this lane's scale bytes: weights (row 32f + m) and tokens (sub-tile S, row m), K block 2s + hl
      uint32_t wsc[2], tsc[NSA];
#pragma unroll
      for (int f = 0; f < 2; ++f) wsc[f] = Ak.s[f] >> (8 * hl);
#pragma unroll
      for (int S = 0; S < NSA; ++S)
        tsc[S] = reinterpret_cast<const uint32_t*>(&stage[kF8TokSlots])[32 * S + m] >> (8 * hl);
      // token fragment i = (step i / NSA, sub-tile i % NSA): pieces hl and 2 + hl of row m
      auto read_b = [&](int i) {
        const int base = (((i % NSA) * 2 + i / NSA) * 32 + m) * 4;
        const u32x4_t lo = stage[base + (hl ^ pf_swz(m))];
        const u32x4_t hi = stage[base + ((2 + hl) ^ pf_swz(m))];
        return f8op_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      f8op_t af[2][2];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const u32x4_t lo = Ak.c[ss][f][0], hi = Ak.c[ss][f][1];
          af[ss][f] = f8op_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      // Software pipeline with one wave per SIMD: token fragment i + 2 is read
      // while the two MFMAs of fragment i (and those of i + 1) run, so the LDS
      // latency hides behind 256 cycles of matrix work.  The scheduling
      // groups keep that order (the register allocator would otherwise reuse
      // one fragment register set and serialise reads behind the MFMAs).
      constexpr int NF = 2 * NSA;
      f8op_t B[NF];
      B[0] = read_b(0);
      if constexpr (NF > 1) B[1] = read_b(1);
      // the scale words and the first two fragments before any MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, NSA + 4, 0);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int s = i / NSA, S = i % NSA;
        const int sb = (int)((tsc[S] >> (16 * s)) & 0xFF);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int sa = (int)((wsc[f] >> (16 * s)) & 0xFF);
          acc[f][S] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s][f], B[i], acc[f][S], 0, 0, 0, sa, 0, sb);
        }
        if (i + 2 < NF) B[i + 2] = read_b(i + 2);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // the pair's two MFMAs
        if (i + 2 < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // then the reads of fragment i + 2
      }
    };

    // kgroup kg: wait for this wave's loads of kg (those of kg + 1 may stay in
    // flight), barrier (every wave's token loads of kg landed; every wave done
    // with kg - 1, whose stage and weight slot are refilled next), issue kg + 2
    // (clamped to the last kgroup past the end, so the counts stay uniform),
    // compute kg
    int kg = 0;
    for (; kg + kF8Stages <= KG; kg += kF8Stages) {
#pragma unroll
      for (int u = 0; u < kF8Stages; ++u) {
        f8_wait_barrier<kF8AOps + kF8TOps>();
        pin(A[u]);
        const int nk = min(kg + u + 2, KG - 1);
        issue_a(A[(u + 2) % kF8ARing], nk);
        issue_t(*st.s[(u + 2) % kF8Stages], nk);
        __builtin_amdgcn_sched_barrier(0);  // the direct-to-LDS loads stay ahead of the MFMAs
        body(A[u], *st.s[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kF8Stages - 1; ++u) {
      if (kg + u < KG) {
        f8_wait_barrier<kF8AOps + kF8TOps>();
        pin(A[u]);
        const int nk = min(kg + u + 2, KG - 1);
        issue_a(A[(u + 2) % kF8ARing], nk);
        issue_t(*st.s[(u + 2) % kF8Stages], nk);
        __builtin_amdgcn_sched_barrier(0);  // the direct-to-LDS loads stay ahead of the MFMAs
        body(A[u], *st.s[u]);
      }
    }
    // drain the clamped loads (L2 hits of the last kgroup, issued a kgroup of
    // matrix work ago); every wave done with the stages before the epilogue
    // and the next item reuse them
    f8_wait_barrier<0>();
    if constexpr (NSA > 0)
      if (g < a.G) {
        if constexpr (G13) pf_epilogue<DT_MXFP8, G13, NSA, kF8Sub, 32>(a, acc, r0, r_end, g, e, lane);
        else f8_down_epilogue<NSA>(a, acc, pidx, r_end - r0, g, lane, wv, st);
      }
    // every wave done reading its staged rows (the stores may stay in flight:
    // a full __syncthreads would wait for all of them)
    if constexpr (!G13) f8_wait_barrier<63>();
  };
  const int nsa = min(kF8Sub, (r_end - r0 + 31) >> 5);
  switch (nsa) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 4: run(std::integral_constant<int, 4>{}); break;
    case 5: run(std::integral_constant<int, 5>{}); break;
    case 6: run(std::integral_constant<int, 6>{}); break;
    case 7: run(std::integral_constant<int, 7>{}); break;
    default: run(std::integral_constant<int, 8>{}); break;
  }
  return e;
}

}  // namespace moe
