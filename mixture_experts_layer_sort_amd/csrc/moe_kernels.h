// Launchers of the library's kernels (internal).  Each returns the result of
// hipGetLastError() after enqueueing on stream `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_layout.h"

namespace moe {

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* wts, hipStream_t s);

hipError_t launch_permute(int dt, const int* ids, int T, int k, int E, int H, int* offsets, int* sorted_pairs,
                          int* pair_pos, const uint16_t* x, uint8_t* xq, hipStream_t s);

// Routing and permutation (+ x quantisation) in one launch, for T up to
// route_permute_max_tokens(): the results of launch_route + launch_permute.
int route_permute_max_tokens();
hipError_t launch_route_permute(int dt, const float* logits, int T, int k, int E, int H, int* ids, float* wts,
                                int* offsets, int* sorted_pairs, int* pair_pos, const uint16_t* x, uint8_t* xq,
                                hipStream_t s);

// Batched activation format: offsets and rows of the valid rows of x [E, M, H]
// (counts clamped to [0, M]), and x quantised into xq (all E M rows; BF16
// activations are used in place and xq is ignored).
hipError_t launch_batched_prep(int dt, const int* counts, int E, int M, int H, int* offsets, int* rows,
                               const uint16_t* x, uint8_t* xq, hipStream_t s);

// Dense NVFP4 linear layer: repack weights [N, K] (W2 arrangement) and alpha;
// offsets / identity rows / NVFP4 quantisation of x [M, K]; the down-GEMM kernels
// with one expert of M rows writing out [M, N].
hipError_t launch_dense_prepare(int N, int K, const uint8_t* codes, const uint8_t* scales, const float* alpha,
                                uint8_t* packed, hipStream_t s);
hipError_t launch_dense_prep(int M, int K, int* offsets, int* rows, const uint16_t* x, uint8_t* xq, hipStream_t s);
hipError_t launch_dense_gemm(int M, int N, int K, const uint8_t* packed, const int* offsets, const int* rows,
                             const uint8_t* xq, uint16_t* out, int grid, hipStream_t s);

hipError_t launch_quantize_weights(int dt, int count, int rows, int K, const float* w, void* codes, void* scales,
                                   float* alpha, hipStream_t s);

// gated: SwiGLU experts (W13 of 2I rows); otherwise ReLU^2 (W1 of I rows)
// NVFP4: scales_out = e4m3(fp32(e4m3(scales_in) * alpha_in[matrix])), then alpha_out = 1
hipError_t launch_fold_global_scale(int count, long long scales_per_matrix, const uint8_t* scales_in,
                                    const float* alpha_in, uint8_t* scales_out, float* alpha_out, hipStream_t s);

hipError_t launch_prepare(int dt, bool gated, int E, int H, int I, const uint8_t* w13, const uint8_t* w13s,
                          const float* w13a, const uint8_t* w2, const uint8_t* w2s, const float* w2a, uint8_t* packed,
                          hipStream_t s);

// How the grouped GEMMs of one call run: the kernel variant (0: decode items
// with 16-row token tiles, 1: 32-row token tiles, 2: prefill items), whether
// an MXFP8 layer's prefill-shaped down GEMM runs on the fp8 instruction (only
// where fp8_down_fits), the
// prefill item band (token rows per band of weight reuse; 0: the kernel's
// default), the persistent blocks per compute unit (0: the occupancy limit), the SwiGLU clamp and
// the optional in-kernel fc2 reduce of the down GEMM (red: fp32 [T, H] output
// rows, wts: the router weights of the pairs), and whether the gate/up GEMM
// may leave out the 16-bit copy of hq (only the bf16-product down GEMMs read
// it; the fp8 one reads the codes).
struct GemmPlan {
  int variant = 0;
  bool down_fp8 = true;
  bool skip_hq_deq = false;
  int band = 0;
  int blocks_per_cu = 0;
  int balance = 0;  // prefill item deal (moe_knobs.load_balance)
  float limit = 0.f;
  float* red = nullptr;
  const float* wts = nullptr;
};

// Grouped GEMMs.  `grid` is the persistent grid size (blocks) of the plan's variant.
hipError_t launch_gemm13(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                         const int* offsets, const int* sorted_pairs, const uint8_t* xq, uint8_t* hq, int grid,
                         hipStream_t s, const GemmPlan& plan);

hipError_t launch_gemm2(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                        const int* offsets, const int* sorted_pairs, const uint8_t* hq, uint16_t* y, int grid,
                        hipStream_t s, const GemmPlan& plan);

// fp32 rows [n] = 0 (a fill kernel: safe under graph capture); bf16 out [n] = rne(acc [n])
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* acc, uint16_t* out, long long n, hipStream_t s);

hipError_t launch_combine(int T, int H, int k, const uint16_t* y, const float* wts, uint16_t* out, hipStream_t s);

// Blocks of the GEMM kernels that fit on one compute unit at once.
int gemm_blocks_per_cu(int dt, bool gemm13, int nt);

// Token sub-tiles (of 16) per decode GEMM work item: 1 while experts see
// about 16 routed rows or fewer on average, else 2.
inline int gemm_nt(int T, int k, int E) { return (long long)T * k > 16LL * E ? 2 : 1; }
// The prefill-shaped GEMM (LDS-staged, 128-row tiles) once experts see 64 or
// more routed rows on average.
inline bool gemm_prefill(int T, int k, int E) { return (long long)T * k >= 64LL * E; }
// GEMM variant index for caches: 0 decode NT=1, 1 decode NT=2, 2 prefill.
inline int gemm_variant(int T, int k, int E) { return gemm_prefill(T, k, E) ? 2 : gemm_nt(T, k, E) - 1; }
// The prefill-shaped GEMMs load activation rows straight into LDS through
// buffer resources with 32-bit offsets below 2^31: rows13 rows of the gate/up
// GEMM's 16-bit activations (H wide) and rows2 rows of the down GEMM's (I
// wide); the fp8 down GEMM reads the latter's I-byte codes.
inline bool prefill_fits(long long rows13, int H, long long rows2, int I) {
  return rows13 * H * 2 < (1LL << 31) && rows2 * I * 2 < (1LL << 31);
}
inline bool fp8_down_fits(int T, int k, int I) { return (long long)T * k * I < (1LL << 31); }
// GEMM variant of the single-launch kernel (layer format dt): as gemm_variant
// (the 32-row decode items where the prefill-shaped ones do not fit), and 3
// for the prefill-shaped GEMMs of MXFP8 layers (fp8 matrix instruction).
inline int fused_variant(int dt, int T, int k, int E, int H, int I) {
  int v = gemm_variant(T, k, E);
  if (v == 2 && !prefill_fits(T, H, (long long)T * k, I)) v = 1;
  return v == 2 && has_fp8_gemm(dt) && fp8_down_fits(T, k, I) ? 3 : v;
}
int prefill_blocks_per_cu(int dt, bool g13);
int prefill_f8_blocks_per_cu(bool g13);

// The whole layer in one cooperative launch; `grid` must not exceed the
// co-resident capacity (fused_blocks_per_cu * compute units).
hipError_t launch_fused(int dt, bool gated, int E, int H, int I, int k, int T, const uint8_t* packed,
                        const float* logits,
                        const uint16_t* x, uint16_t* out, int* ids, float* wts, uint8_t* ws, size_t ws_bytes,
                        int max_tokens, int grid, hipStream_t s, float limit = 0.f);
int fused_blocks_per_cu(int dt, int variant);  // variant as fused_variant
// Zero the workspace's synchronisation words.
hipError_t launch_zero_sync(uint8_t* ws, int dt, int E, int H, int I, int k, int max_tokens, hipStream_t s);

}  // namespace moe
