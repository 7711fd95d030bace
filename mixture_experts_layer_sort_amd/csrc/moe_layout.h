// Byte layouts shared by the host entry points and the kernels: the packed
// (MFMA-ready) weight buffer, the quantised activation buffers and the
// forward workspace.
//
// Packed weights.  K is cut into 128-wide slices ("kgroups").  A "tile" is 16
// weight rows x one kgroup, stored in the per-lane operand order of the CDNA4
// matrix instruction that consumes it (lane l = 16*q + i holds row i):
//   BF16  (v_mfma_f32_16x16x32_bf16, 4 per kgroup): [chunk c<4][lane][8 bf16],
//         lane (i,q) of chunk c holds k = 32c + 8q .. +8           (4096 B)
//   MXFP8 (converted exactly to bf16 in registers, then bf16 MFMA):
//         [half h<2][lane][2 chunks x 8 B], lane (i,q) of chunk c = 2h + j
//         holds k = 32c + 8q .. +8 (so every element of chunk c lies in scale
//         block c); each half is one contiguous 1 KB wave load;
//         scales [row i][4 e8m0 bytes]                  (2048 B + 64 B)
//   NVFP4 (dequantised exactly to fp16 in registers, then fp16 MFMA):
//         [lane][4 chunks x 4 B] of e2m1 nibbles, lane (i,q) of chunk c holds
//         k = 32c + 8q .. +8; scales [row i][8 e4m3 bytes] in K order, lane
//         (i,q) of chunk c uses byte 2c + q/2            (1024 B + 128 B)
// MXFP8 layers (not bf16 x MXFP8) also hold their W2 codes in fragment order
// for the prefill-shaped down GEMM on the block-scaled fp8 matrix
// instruction: per (expert, row group of 64, 64-wide K step) 4 KB =
// [fragment f<2 (group rows 32f..32f+32)][half q<2][lane 64][16 B], lane
// l = m + 32h holding row m's K bytes 64s + 32q + 16h .. +16 (the
// instruction's operand order); that GEMM reads the scales of the tile region
// above.
// Row groups: W13 group g = gate rows 32g..32g+32 (tiles 0,1) and up rows
// I+32g..I+32g+32 (tiles 2,3), so SwiGLU pairs sit in the same lanes;
// W2 group g = rows 64g..64g+64 (tiles 0..3).  Block (e, g, kgroup) holds its
// 4 tiles contiguously: index ((e * G + g) * KG + kg) * 4 + t.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__ inline
#else
#define MOE_HD inline
#endif

namespace moe {

// Layer formats (moe_dtype).  DT_BF16_MXFP8 keeps activations in bf16 (no
// quantisation of x, intermediate rounded to bf16) over MXFP8 weights.
enum { DT_BF16 = 0, DT_MXFP8 = 1, DT_NVFP4 = 2, DT_BF16_MXFP8 = 3 };
// the format of the weights / of the activations (x, the intermediate) of a layer format
MOE_HD int weight_dt(int dt) { return dt == DT_BF16_MXFP8 ? DT_MXFP8 : dt; }
MOE_HD int act_dt(int dt) { return dt == DT_BF16_MXFP8 ? DT_BF16 : dt; }

constexpr int kKGroup = 128;   // K slice of one tile
constexpr int kTileRows = 16;  // rows of one tile
constexpr int kTilesPerGroup = 4;

MOE_HD size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bytes of one weight tile's codes / scales (dt: a layer format)
MOE_HD size_t tile_code_bytes(int dt) {
  dt = weight_dt(dt);
  return dt == DT_BF16 ? 4096 : (dt == DT_MXFP8 ? 2048 : 1024);
}
MOE_HD size_t tile_scale_bytes(int dt) {
  dt = weight_dt(dt);
  return dt == DT_BF16 ? 0 : (dt == DT_MXFP8 ? 64 : 128);
}

// activation row bytes (x2 for nvfp4: half a byte) and scale block (dt: a layer format)
MOE_HD size_t row_code_bytes(int dt, int K) {
  dt = act_dt(dt);
  return dt == DT_BF16 ? (size_t)K * 2 : (dt == DT_MXFP8 ? (size_t)K : (size_t)K / 2);
}
MOE_HD int scale_block(int dt) { return dt == DT_MXFP8 ? 32 : (dt == DT_NVFP4 ? 16 : 0); }
MOE_HD size_t row_scale_bytes(int dt, int K) {
  dt = act_dt(dt);
  return dt == DT_BF16 ? 0 : (size_t)K / scale_block(dt);
}

struct PackedLayout {
  int G13, KG13, G2, KG2;
  size_t w13_codes, w13_scales, w2_codes, w2_scales, w13_alpha, w2_alpha, w2_frag, total;
};

// The layer formats whose prefill-shaped down GEMM runs on the fp8 matrix
// instruction (its output is not requantised: the instruction's ~1e-5
// relative accumulation error stays far below the bf16 rounding of y; the
// gate/up GEMM keeps exact products with fp32 accumulation, as its
// requantised output turns such errors into code flips).
MOE_HD bool has_fp8_gemm(int dt) { return dt == DT_MXFP8; }

// gated: SwiGLU experts, W13 row group g = 32 gate rows + the matching 32 up
// rows; otherwise (ReLU^2) W1 of I rows in groups of 64.
MOE_HD PackedLayout packed_layout(int dt, int E, int H, int I, bool gated = true) {
  PackedLayout L;
  L.G13 = gated ? I / 32 : I / 64;
  L.KG13 = H / kKGroup;
  L.G2 = H / 64;
  L.KG2 = I / kKGroup;
  size_t n13 = (size_t)E * L.G13 * L.KG13 * kTilesPerGroup;  // tiles of W13
  size_t n2 = (size_t)E * L.G2 * L.KG2 * kTilesPerGroup;     // tiles of W2
  size_t off = 0;
  L.w13_codes = off; off = align256(off + n13 * tile_code_bytes(dt));
  L.w13_scales = off; off = align256(off + n13 * tile_scale_bytes(dt));
  L.w2_codes = off; off = align256(off + n2 * tile_code_bytes(dt));
  L.w2_scales = off; off = align256(off + n2 * tile_scale_bytes(dt));
  L.w13_alpha = off; off = align256(off + (weight_dt(dt) == DT_NVFP4 ? (size_t)E * 4 : 0));
  L.w2_alpha = off; off = align256(off + (weight_dt(dt) == DT_NVFP4 ? (size_t)E * 4 : 0));
  L.w2_frag = off; off = align256(off + (has_fp8_gemm(dt) ? n2 * tile_code_bytes(dt) : 0));
  L.total = off;
  return L;
}

// Quantised activation rows (xq: rows = tokens, K = H; hq: rows = pairs, K = I):
// codes [rows, row_code_bytes] at 0, scales [rows, row_scale_bytes] after,
// then (MXFP8, NVFP4) the exact dequantised values as 16-bit floats [rows, K]
// (bf16 for MXFP8, fp16 for NVFP4), the matrix-unit operand of the next GEMM.
MOE_HD size_t act_scale_offset(int dt, int rows, int K) { return align256((size_t)rows * row_code_bytes(dt, K)); }
MOE_HD size_t act_dequant_offset(int dt, int rows, int K) {
  return act_scale_offset(dt, rows, K) + align256((size_t)rows * row_scale_bytes(dt, K));
}
MOE_HD size_t act_bytes(int dt, int rows, int K) {
  return act_dequant_offset(dt, rows, K) + (act_dt(dt) == DT_BF16 ? 0 : align256((size_t)rows * K * 2));
}
// 16-bit operand rows of an activation buffer: the codes for BF16, else the dequantised copy
MOE_HD size_t act_operand_offset(int dt, int rows, int K) {
  return act_dt(dt) == DT_BF16 ? 0 : act_dequant_offset(dt, rows, K);
}

// moe_forward workspace, sized for max_tokens.  It opens with the fused
// kernel's synchronisation words (kSyncHeader words, then one per expert),
// which must be zero before the first forward and are left zero by it.
constexpr int kSyncHeader = 4;

struct WorkspaceLayout {
  size_t sync, sync_bytes, ids, wts, offsets, sorted_pairs, pair_pos, xq, hq, y, total;
};

MOE_HD WorkspaceLayout workspace_layout(int dt, int E, int H, int I, int k, int max_tokens) {
  WorkspaceLayout W;
  size_t P = (size_t)max_tokens * k, off = 0;
  W.sync = off;
  W.sync_bytes = align256((size_t)(kSyncHeader + E) * 4);
  off += W.sync_bytes;
  W.ids = off; off = align256(off + P * 4);
  W.wts = off; off = align256(off + P * 4);
  W.offsets = off; off = align256(off + (size_t)(E + 1) * 4);
  W.sorted_pairs = off; off = align256(off + P * 4);
  W.pair_pos = off; off = align256(off + P * 4);
  W.xq = off; off = align256(off + (act_dt(dt) == DT_BF16 ? 0 : act_bytes(dt, max_tokens, H)));
  W.hq = off; off = align256(off + act_bytes(dt, (int)P, I));
  W.y = off; off = align256(off + P * (size_t)H * 2);
  W.total = off;
  return W;
}

// Dense NVFP4 linear layer: weights [N, K] in the W2 tile layout (row groups
// of 64, 128-wide kgroups), then the fp32 alpha.
struct DenseLayout {
  int G, KG;
  size_t codes, scales, alpha, total;
};

MOE_HD DenseLayout dense_layout(int N, int K) {
  DenseLayout D;
  D.G = N / 64;
  D.KG = K / kKGroup;
  const size_t n = (size_t)D.G * D.KG * kTilesPerGroup;
  size_t off = 0;
  D.codes = off; off = align256(off + n * tile_code_bytes(DT_NVFP4));
  D.scales = off; off = align256(off + n * tile_scale_bytes(DT_NVFP4));
  D.alpha = off; off = align256(off + 4);
  D.total = off;
  return D;
}

// Its workspace for M rows: offsets {0, M}, the identity row map, the NVFP4-quantised rows of x.
struct DenseWorkspace {
  size_t offsets, rows, xq, total;
};

MOE_HD DenseWorkspace dense_workspace(int M, int K) {
  DenseWorkspace W;
  size_t off = 0;
  W.offsets = off; off = align256(off + 8);
  W.rows = off; off = align256(off + (size_t)M * 4);
  W.xq = off; off = align256(off + act_bytes(DT_NVFP4, M, K));
  W.total = off;
  return W;
}

// moe_batched_experts workspace: E experts of up to M rows each.
struct BatchedLayout {
  size_t offsets, rows, xq, hq, total;
};

MOE_HD BatchedLayout batched_layout(int dt, int E, int H, int I, int M) {
  BatchedLayout B;
  const size_t R = (size_t)E * M;
  size_t off = 0;
  B.offsets = off; off = align256(off + (size_t)(E + 1) * 4);
  B.rows = off; off = align256(off + R * 4);
  B.xq = off; off = align256(off + (act_dt(dt) == DT_BF16 ? 0 : act_bytes(dt, (int)R, H)));
  B.hq = off; off = align256(off + act_bytes(dt, (int)R, I));
  B.total = off;
  return B;
}

}  // namespace moe
