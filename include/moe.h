/*
 * moe.h — C ABI of libmoe_mi355x.so, a fused Mixture-of-Experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (one GPU's share, all experts local):
 *   top-k routing -> permutation of (token, slot) pairs by expert (+ in-kernel
 *   activation quantisation) -> gate/up grouped GEMM -> SwiGLU (+ dynamic
 *   per-block requantisation of the intermediate) -> down grouped GEMM ->
 *   weighted top-k combine.
 * It is the computation the pages describe for the FlashInfer b12x fused MoE
 * (one call does routing, W1 GEMM, SwiGLU, W2 GEMM and the reduction; bf16
 * hidden states are quantised inside) [vLLM PR 40082 report, "Implementation"
 * item 1 and "Key source excerpts"] and for the MegaMoE NVFP4 / MXFP8 / BF16
 * kernels [MegaMoE drop workflow, §1].
 *
 * Weight formats (canonical, caller-facing):
 *   MOE_BF16  : W13 bf16 [E, 2I, H], W2 bf16 [E, H, I].
 *   MOE_MXFP8 : e4m3fn codes, one e8m0 scale byte per 32 along K:
 *               W13 u8 [E, 2I, H] + u8 [E, 2I, H/32]; W2 u8 [E, H, I] + u8 [E, H, I/32].
 *   MOE_NVFP4 : e2m1 codes packed two per byte (element 2i in the low nibble),
 *               one e4m3fn scale per 16 along K, one fp32 dequant multiplier
 *               alpha per expert and tensor (= 1 / global scale) [vLLM PR
 *               40082 report, "Key source excerpts": block scale = amax *
 *               global scale / fp4 max, alpha = 1 / global scale]:
 *               W13 u8 [E, 2I, H/2] + u8 [E, 2I, H/16] + f32 [E];
 *               W2  u8 [E, H, I/2]  + u8 [E, H, I/16]  + f32 [E].
 *   MOE_BF16_MXFP8 : MXFP8 weights (as MOE_MXFP8) with bf16 activations: the
 *               hidden states are not quantised and the intermediate is
 *               rounded to bf16, as for MOE_BF16 (the pages list a bf16 x
 *               MXFP8 MegaMoE entry, bf16_mxfp8_mega_moe, beside the three
 *               formats [MegaMoE drop workflow, §1, the package exports]).
 *               Weight buffers, moe_quantize_weights and moe_prepare_weights
 *               are those of MOE_MXFP8; xq and hq are those of MOE_BF16.
 *   W13 rows [0, I) are the gate projection, rows [I, 2I) the up projection.
 *   With MOE_RELU2 experts W13 holds I rows (W1) instead of 2I: [E, I, H]
 *   codes (and [E, I, H/32] / [E, I, H/16] scales); W2 is unchanged.
 *
 * Conventions of every entry point:
 *   - Buffers are device pointers owned by the caller; the library never
 *     allocates device memory, never synchronises the stream, never reads
 *     device data on the host, and never writes its inputs.  Outputs are
 *     written in place into the caller's buffers.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous;
 *     device-side faults surface at the caller's next synchronisation.
 *   - Arguments are checked on the host before anything is enqueued; on error
 *     nothing is enqueued and a negative moe_status is returned.  T == 0 is a
 *     successful no-op.  No exception or abort crosses the ABI.
 *   - Expert ids are local ids in [0, E) (E = experts resident on this GPU).
 *   - Calls are reentrant; the only library state is a per-device cache of
 *     the compute-unit count and occupancy.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum { MOE_BF16 = 0, MOE_MXFP8 = 1, MOE_NVFP4 = 2, MOE_BF16_MXFP8 = 3 } moe_dtype;

/* Expert activation.  MOE_SWIGLU: gated, h = silu(gate) * up with W13 rows
 * [0, I) gate and [I, 2I) up.  MOE_RELU2: non-gated, h = relu(W1 x)^2 with
 * W1 = W13 of I rows (the squared-ReLU experts of Nemotron-style models,
 * which the pages note the b12x backend rejects [vLLM PR 40082 report,
 * "Risks" item 4]).  Everything else -- formats, requantisation of h, the
 * down GEMM and the combine -- is the same. */
typedef enum { MOE_SWIGLU = 0, MOE_RELU2 = 1 } moe_activation;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, T out of range, bad size */
  MOE_ERR_UNSUPPORTED = -2, /* shape or dtype outside the supported set */
  MOE_ERR_WORKSPACE = -3,   /* workspace or packed buffer too small */
  MOE_ERR_LAUNCH = -4       /* a kernel launch failed (hipGetLastError) */
} moe_status;

/* Layer shape.  Supported: hidden % 128 == 0, inter % 128 == 0,
 * 1 <= num_experts <= 1024, 1 <= top_k <= min(num_experts, 32),
 * 1 <= max_tokens and max_tokens * top_k <= 2^24, dtype a moe_dtype,
 * activation a moe_activation, gate_up_limit finite and >= 0 (0 with
 * MOE_RELU2 experts).
 * gate_up_limit: the SwiGLU experts' gate/up clamp L (the pages name a
 * resolve_gate_up_clamp step and no rule [MegaMoE drop workflow, §2, the
 * adaptation layer's comm.py]; reading: before the activation the gate is
 * min(gate, L) and the up value clamp(up, -L, L)); 0 = no clamp. */
typedef struct {
  int32_t hidden;      /* H */
  int32_t inter;       /* I, per expert */
  int32_t num_experts; /* E, local */
  int32_t top_k;       /* k */
  int32_t max_tokens;  /* workspace capacity in tokens */
  int32_t dtype;       /* moe_dtype of weights and activations */
  int32_t activation;  /* moe_activation of the experts */
  float gate_up_limit; /* gate/up clamp L of SwiGLU experts, 0 = none */
} moe_shape;

/* Text of a status code (static storage). */
MOE_API const char* moe_status_string(int32_t status);

/* MOE_OK if the shape is supported, else MOE_ERR_UNSUPPORTED / INVALID_ARG. */
MOE_API moe_status moe_check_shape(const moe_shape* shape);

/* Sizes in bytes (0 for an unsupported shape). */
MOE_API size_t moe_packed_weight_bytes(const moe_shape* shape);
/* Workspace of moe_forward for any T <= max_tokens. */
MOE_API size_t moe_workspace_bytes(const moe_shape* shape);
/* Quantised activations of T tokens (moe_permute's xq): codes [T, H*b] at
 * offset 0, then scales [T, H/blk] at moe_xq_scale_offset(shape, T), then
 * (MXFP8, NVFP4) the exact dequantised values [T, H] as bf16 (MXFP8) or
 * fp16 (NVFP4) at moe_xq_dequant_offset(shape, T) — the operand the grouped
 * GEMM reads, produced once per token instead of once per expert tile.
 *   BF16, BF16_MXFP8: bf16 [T, H], no scales;  MXFP8: u8 [T, H] + e8m0 [T, H/32] + bf16;
 *   NVFP4: packed e2m1 [T, H/2] + e4m3 [T, H/16] + fp16. */
MOE_API size_t moe_xq_bytes(const moe_shape* shape, int32_t T);
MOE_API size_t moe_xq_scale_offset(const moe_shape* shape, int32_t T);
MOE_API size_t moe_xq_dequant_offset(const moe_shape* shape, int32_t T);
/* Requantised intermediate of the T*k pairs in expert-sorted order
 * (moe_gemm13_swiglu_quant's hq), same scheme along I:
 *   BF16, BF16_MXFP8: bf16 [P, I];  MXFP8: u8 [P, I] + e8m0 [P, I/32] + bf16 [P, I];
 *   NVFP4: packed e2m1 [P, I/2] + e4m3 [P, I/16] + fp16 [P, I]  (P = T * k). */
MOE_API size_t moe_hq_bytes(const moe_shape* shape, int32_t T);
MOE_API size_t moe_hq_scale_offset(const moe_shape* shape, int32_t T);
MOE_API size_t moe_hq_dequant_offset(const moe_shape* shape, int32_t T);

/* Quantise fp32 master weights of `count` stacked matrices [count, rows, K]
 * into the canonical format of `dtype` (the load-time preprocessing step the
 * pages describe for turning canonical weights into the kernel format
 * [MegaMoE drop workflow, §3, preprocess_mega_weights]).
 *   BF16 : codes = bf16 [count, rows, K]; scales, alpha unused (may be NULL).
 *   MXFP8: codes u8 [count, rows, K], scales e8m0 [count, rows, K/32]; the
 *          OCP MX rule s = floor(log2 amax) - 8 per block of 32.
 *   NVFP4: codes packed [count, rows, K/2], scales e4m3 [count, rows, K/16],
 *          alpha f32 [count] = amax(matrix) / (6 * 448) (1 if all zero);
 *          block scale = e4m3(fp32(amax_blk / 6) / alpha), code =
 *          e2m1(w / fp32(scale * alpha)), all fp32 operations correctly rounded.
 * rows >= 1, K % 32 == 0 (MXFP8) / % 16 == 0 (NVFP4) / % 2 == 0 (BF16). */
MOE_API moe_status moe_quantize_weights(int32_t dtype, int32_t count, int32_t rows, int32_t K,
                                const float* w, void* codes, void* scales, float* alpha,
                                hipStream_t stream);

/* Fold the NVFP4 per-tensor weight alpha into the block scales, as the pages'
 * weight preprocessing does [vLLM PR 40082 report, "Key source excerpts",
 * process_weights_after_loading: the weight global scale is baked into the
 * block scales and the weight alpha becomes 1]: for `count` matrices of
 * `rows` x `K` NVFP4 weights,
 *   scales_out[e, r, b] = e4m3_rne_satfinite( fp32(e4m3(scales_in[e, r, b]) * alpha_in[e]) ),
 *   alpha_out[e] = 1.
 * The codes are unchanged.  Every block scale is re-rounded in e4m3, and
 * products below 2^-6 land in e4m3's subnormal range (quantum 2^-9), so
 * the folded weights are a coarser quantisation of the same masters; the
 * layer then runs with alpha = 1.  Buffers: scales u8 [count, rows, K/16],
 * alpha f32 [count]; out may equal in (in place).  K % 16 == 0. */
MOE_API moe_status moe_nvfp4_fold_global_scale(int32_t count, int32_t rows, int32_t K, const void* scales_in,
                                               const float* alpha_in, void* scales_out, float* alpha_out,
                                               hipStream_t stream);

/* Repack canonical weights into the MFMA-ready tile layout in `packed`
 * (moe_packed_weight_bytes bytes): per expert, W13 is cut into groups of 32
 * gate rows + the matching 32 up rows (MOE_RELU2: W1 into groups of 64
 * rows), W2 into groups of 64 rows; each
 * (row group, 128-wide K slice) is one contiguous block laid out in the
 * per-lane operand order of the CDNA4 MFMA that consumes it, with scales in
 * the matching per-lane order.  A pure byte permutation; done once at load
 * time, not per forward [vLLM PR 40082 report, "Key source excerpts" and
 * "Review highlights": the MMA-layout scale conversion is cached at load
 * time; vLLM PR 38050 report, "Implementation": scale conversion and
 * interleave when preparing weights for the CuteDSL kernel].
 * MOE_MXFP8 layers also get a second copy of the W2 codes in the operand
 * order of the block-scaled fp8 matrix instruction (32-row x 64-K fragments)
 * for the down GEMM of prefill-sized batches (moe_packed_weight_bytes
 * includes it; E * H * I bytes more).
 * Scales / alpha are NULL for BF16; alpha is NULL for MXFP8. */
MOE_API moe_status moe_prepare_weights(const moe_shape* shape,
                               const void* w13_codes, const void* w13_scales, const float* w13_alpha,
                               const void* w2_codes, const void* w2_scales, const float* w2_alpha,
                               void* packed, size_t packed_bytes, hipStream_t stream);

/* Top-k routing of T tokens [vLLM PR 40082 report, "Implementation" item 1].
 * logits fp32 [T, E] -> topk_ids int32 [T, k], topk_w fp32 [T, k].
 * Experts are picked by logit descending, ties to the lower id (-0 == +0);
 * slot j holds the j-th pick; weights are the softmax over the k picked
 * logits (= full softmax restricted to the picks and renormalised).
 * Non-finite logits give unspecified (but in-bounds) results. */
MOE_API moe_status moe_route(const moe_shape* shape, int32_t T, const float* logits,
                     int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Token dispatch: permutation of the P = T*k pairs p = t*k + j by expert
 * [vLLM PR 40082 report, "Key source excerpts": token dispatch fused with the
 * GEMMs], plus the in-kernel quantisation of the bf16 hidden states x [T, H]
 * into xq (layout of moe_xq_bytes; for BF16, xq may equal x: then nothing is
 * copied) [same report: bf16 hidden states are quantised inside].
 * Outputs: offsets int32 [E+1] (exclusive prefix of per-expert counts,
 * offsets[E] = P), sorted_pairs int32 [P] (pairs in (expert, p) order),
 * pair_pos int32 [P] (inverse: sorted_pairs[pair_pos[p]] == p).
 * Expert ids must lie in [0, E) (undefined results otherwise).
 * ws / ws_bytes: unused, may be NULL / 0. */
MOE_API moe_status moe_permute(const moe_shape* shape, int32_t T, const int32_t* topk_ids, const uint16_t* x,
                       int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos, void* xq,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Gate/up grouped GEMM + SwiGLU + requantisation [vLLM PR 40082 report,
 * "Implementation" item 1; "Key source excerpts": the intermediate uses
 * dynamic per-block quantisation with global scale 1].
 * For each expert e and sorted row r in [offsets[e], offsets[e+1]):
 *   g, u = W13[e] . xq[sorted_pairs[r] / k]  (fp32 accumulation; NVFP4 scaled
 *   by the W13 alpha; with gate_up_limit L > 0: g = min(g, L),
 *   u = clamp(u, -L, L)), h = silu(g) * u, hq[r] = requant(h) (layout of
 *   moe_hq_bytes).  MOE_RELU2: g = W1[e] . xq[...], h = relu(g)^2.  ws / ws_bytes: unused, may be NULL / 0. */
MOE_API moe_status moe_gemm13_swiglu_quant(const moe_shape* shape, int32_t T, const void* packed,
                                   const int32_t* offsets, const int32_t* sorted_pairs, const void* xq,
                                   void* hq, void* ws, size_t ws_bytes, hipStream_t stream);

/* Down grouped GEMM: for each expert e and sorted row r of it,
 * y[sorted_pairs[r]] = bf16(W2[e] . hq[r]) (fp32 accumulation, NVFP4 scaled
 * by the W2 alpha).  y is bf16 [T*k, H], row p = t*k + j (slot-major).
 * MOE_MXFP8 layers with 64 or more routed rows per expert on average run it
 * on the block-scaled fp8 matrix instruction (e4m3 x e4m3 with the e8m0
 * block scales applied by the hardware; its 64-product sums carry a relative
 * error of ~1e-5, far below the bf16 rounding of y).
 * ws / ws_bytes: unused, may be NULL / 0. */
MOE_API moe_status moe_gemm2(const moe_shape* shape, int32_t T, const void* packed,
                     const int32_t* offsets, const int32_t* sorted_pairs, const void* hq,
                     uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted top-k reduction [vLLM PR 40082 report, "Implementation" item 1]:
 * out[t] = bf16( sum_{j=0..k-1} topk_w[t, j] * y[t*k + j] ), fp32, slot order
 * (deterministic: the pages note that an in-kernel atomic fc2 reduce makes the
 * order non-deterministic [MegaMoE drop workflow, §6]). */
MOE_API moe_status moe_combine(const moe_shape* shape, int32_t T, const uint16_t* y, const float* topk_w,
                       uint16_t* out, hipStream_t stream);

/* The whole layer: route -> permute (+quant) -> gemm13 -> gemm2 -> combine
 * [vLLM PR 40082 report, "Implementation" item 1: one call does routing, W1
 * GEMM, SwiGLU, W2 GEMM and the reduction], enqueued as the five stage
 * kernels back to back on `stream` (bitwise the same results as the staged
 * entry points).  Every intermediate lives in `ws` (moe_workspace_bytes(shape)
 * bytes, sized once for max_tokens; any T <= max_tokens reuses it [MegaMoE
 * drop workflow, §6: buffers are sized once by the token capacity]).
 * out bf16 [T, H].  topk_ids / topk_w: optional outputs (NULL = keep them in
 * the workspace). */
MOE_API moe_status moe_forward(const moe_shape* shape, int32_t T, const void* packed, const float* logits,
                       const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* The same layer in ONE cooperative launch of a persistent kernel: grid
 * barriers separate routing, the permutation, the two GEMMs and the combine;
 * results are bitwise equal to moe_forward.  On MI355X a device-wide barrier
 * costs ~10 us (measured), more than a kernel boundary on one stream, so
 * moe_forward is the faster entry; this one serves callers that need a
 * single dispatch.  The workspace opens with synchronisation words that must
 * be zero before the first call (moe_workspace_init, or a zeroed allocation)
 * and are left zero by every call; calls on one workspace must be
 * stream-ordered.  Spin-waits are bounded: a timeout (a bug, never expected)
 * sets the third synchronisation word and lets the kernel finish.
 * MOE_ERR_UNSUPPORTED if the device cannot host the cooperative grid. */
MOE_API moe_status moe_forward_fused(const moe_shape* shape, int32_t T, const void* packed, const float* logits,
                                     const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace of moe_batched_experts for up to max_rows rows per expert
 * (0 for an unsupported shape or num_experts * max_rows > 2^24). */
MOE_API size_t moe_batched_workspace_bytes(const moe_shape* shape, int32_t max_rows);

/* The expert MLPs on tokens that arrive already bucketed per expert -- the
 * batched activation format of the CuteDSL batched-experts class [vLLM PR
 * 38050 report, "Implementation": FlashInferCuteDSLBatchedExperts, batched
 * activation format with workspace_shapes] -- with no routing and no
 * combine (the dispatch and the weighted combine live outside, e.g. in an
 * expert-parallel exchange).
 *   x      bf16 [E, max_rows, H]: row r of expert e is valid for r < counts[e];
 *   counts int32 [E] on the device (values clamped to [0, max_rows]);
 *   y      bf16 [E, max_rows, H]: y[e, r] = W2[e] . requant(act(W13[e] . quant(x[e, r])))
 *          for the valid rows (the same arithmetic as moe_forward's expert
 *          outputs); other rows of y are not written.
 * The weights are those of moe_prepare_weights for `shape` (top_k and
 * max_tokens are not used).  ws: moe_batched_workspace_bytes(shape,
 * max_rows) bytes.  The GEMM shapes (decode- or prefill-shaped) follow
 * max_rows as the expected rows per expert. */
MOE_API moe_status moe_batched_experts(const moe_shape* shape, int32_t max_rows, const int32_t* counts,
                                       const uint16_t* x, const void* packed, uint16_t* y, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Dense NVFP4 linear layer, the pages' second b12x kernel: bf16 activations
 * quantised to NVFP4 inside and multiplied by NVFP4 weights [vLLM PR 40082
 * report, "Implementation" item 2: FlashInferB12xNvFp4LinearKernel quantises
 * the input (scaled_fp4_quant) and calls the scaled fp4 matrix product].
 *   out[m, n] = bf16( alpha * sum_k xq[m, k] * w[n, k] )  (fp32 accumulation),
 * xq = the NVFP4 quantisation of x's rows (per 16, global scale 1: the
 * layer's activation rule), w = e2m1 codes [N, K/2] (element 2i in the low
 * nibble) times e4m3 scales [N, K/16] (moe_quantize_weights(MOE_NVFP4, 1, N,
 * K, ...) produces them and alpha).  N % 64 == 0, K % 128 == 0 (else
 * MOE_ERR_UNSUPPORTED).  The weights are repacked once by
 * moe_nvfp4_linear_prepare into moe_nvfp4_linear_packed_bytes(N, K) bytes;
 * a call on M rows needs moe_nvfp4_linear_workspace_bytes(M, K) bytes of
 * workspace (sizes are 0 for unsupported arguments).  x bf16 [M, K],
 * out bf16 [M, N]; M == 0 is a no-op.  It runs the MoE down-GEMM kernels
 * with one expert holding all M rows. */
MOE_API size_t moe_nvfp4_linear_packed_bytes(int32_t N, int32_t K);
MOE_API size_t moe_nvfp4_linear_workspace_bytes(int32_t max_M, int32_t K);
MOE_API moe_status moe_nvfp4_linear_prepare(int32_t N, int32_t K, const void* codes, const void* scales,
                                            const float* alpha, void* packed, size_t packed_bytes,
                                            hipStream_t stream);
MOE_API moe_status moe_nvfp4_linear(int32_t M, int32_t N, int32_t K, const void* packed, const uint16_t* x,
                                    uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Size of the device scratch array behind moe_forward_noalloc (64 MiB per
 * device, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the layer
 * of moe_forward (same kernels, bitwise the same results) with its
 * intermediates in a library-owned static device array instead of a caller
 * workspace.  Nothing is allocated, freed or synchronised.  The intermediates
 * of T tokens must fit: moe_workspace_bytes of `shape` with max_tokens = T
 * must not exceed MOE_NOALLOC_SCRATCH_BYTES, else MOE_ERR_WORKSPACE (nothing
 * enqueued) -- decode-sized batches fit (e.g. T = 128, H = 7168, I = 2048,
 * top-8 NVFP4 needs ~21 MiB), prefill-sized ones do not.  All calls on one
 * device share that device's array, which keeps the last call's contents:
 * calls that may overlap on one device (different streams or host threads
 * without ordering) race and give undefined results; stream-ordered calls
 * are safe.  MOE_ERR_LAUNCH if the array's device address cannot be
 * obtained. */
MOE_API moe_status moe_forward_noalloc(const moe_shape* shape, int32_t T, const void* packed, const float* logits,
                                       const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w,
                                       hipStream_t stream);

/* Knobs of one layer call: how the grouped GEMMs run (the pages separate
 * correctness knobs, which change the code path or the output bits, from
 * performance knobs, which leave the output unchanged, and resolve knobs once
 * per buffer capacity from a persistent knob cache with a default heuristic
 * as fallback, a plain lookup with no compilation [MegaMoE drop workflow,
 * §4 step 3 (the knob split of the tuner) and §6 (knob resolution, the fc2
 * reduce)]).  Every kernel variant is compiled into the library; knobs only
 * choose among them.
 *   gemm       0: by the rows per expert (T k / E; the default heuristic);
 *              1: decode-shaped items with 16-row token tiles; 2: decode-shaped
 *              items with 32-row token tiles; 3: prefill-shaped items (128
 *              rows, LDS-staged; 256 rows on the fp8 instruction).
 *              Correctness knob: the fp32 accumulation order of the
 *              contractions differs between variants.
 *   down_fp8   MXFP8 layers, prefill-shaped down GEMM: 1 (default) on the
 *              block-scaled fp8 matrix instruction, 0 on bf16 products of the
 *              widened codes.  Correctness knob (accumulation order); ignored
 *              by other formats.
 *   band_rows  prefill-shaped items: token rows of one band of the item order
 *              (consecutive items share weight tiles within a band); 0 = 1024.
 *              Performance knob: the output bits do not change.
 *   fc2_reduce 1: the down GEMM adds w * y into an fp32 accumulator of the
 *              token's output row with atomics and no y rows are written; the
 *              summation order then depends on scheduling, so outputs are
 *              not bitwise reproducible.  0 (default): y rows and the
 *              deterministic slot-order combine.  Needs top_k >= 2 (the
 *              accumulator lives in the y region of the workspace).
 *   blocks_per_cu  persistent grid of the grouped GEMMs, blocks per compute
 *              unit (0: as many as fit at once; 1..16 otherwise; blocks past
 *              the resident capacity start as earlier ones finish).
 *              Performance knob.
 *   load_balance  prefill-shaped items: how the persistent blocks deal the
 *              item order, chunk by chunk of (grid) consecutive items, each
 *              XCD taking one slice of 1/8 of a chunk.  0 (default): XCD x
 *              always takes slice x (its L2 keeps the same weight n-blocks
 *              from chunk to chunk); 1: the slice rotates over the XCDs every
 *              chunk and each block's place in it every chunk (item costs
 *              follow the expert-major order, so a fixed slice can leave one
 *              XCD the costlier places chunk after chunk); 2: the slice
 *              rotates every fourth chunk, the place every chunk; 3: no
 *              chunks -- XCD x takes the n-blocks [x NB/8, (x+1) NB/8) of
 *              every m-tile (NB = the GEMM's n-blocks of 256 weight rows), so
 *              every XCD gets the same mix of full and ragged m-tiles; used
 *              where NB and the grid are multiples of 8, else mode 0.
 *              Performance knob (each item is computed the same way wherever
 *              it runs); ignored by the decode-shaped items. */
typedef struct moe_knobs {
  int32_t gemm;
  int32_t down_fp8;
  int32_t band_rows;
  int32_t fc2_reduce;
  int32_t blocks_per_cu;
  int32_t load_balance;
} moe_knobs;

/* The default knobs: {0, 1, 0, 0, 0, 0}. */
MOE_API void moe_default_knobs(moe_knobs* knobs);

/* moe_forward with explicit knobs (NULL = the defaults).  Same arguments and
 * workspace as moe_forward; with the default knobs the results are bitwise
 * those of moe_forward.  MOE_ERR_INVALID_ARG for a knob out of range (gemm
 * outside [0, 3], down_fp8 / fc2_reduce outside {0, 1}, band_rows outside
 * [0, 2^20], blocks_per_cu outside [0, 16], load_balance outside [0, 3]);
 * MOE_ERR_UNSUPPORTED for fc2_reduce with top_k == 1, for
 * gemm = 1 with more than 16 (65535 - num_experts) routed rows (T top_k), and
 * for gemm = 3 where T hidden or T top_k inter reaches 2^30 (the prefill-shaped
 * GEMMs address activation rows with 31-bit byte offsets; the default knobs
 * then use the 32-row decode items). */
MOE_API moe_status moe_forward_knobs(const moe_shape* shape, int32_t T, const void* packed, const float* logits,
                                     const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w,
                                     void* ws, size_t ws_bytes, const moe_knobs* knobs, hipStream_t stream);

/* Persistent knob cache lookup (host only, no device work).  The cache is a
 * text file of lines
 *     dtype act hidden inter experts top_k t_min t_max : gemm down_fp8 band_rows fc2_reduce blocks_per_cu
 *                                                         load_balance
 * (dtype: bf16 | mxfp8 | nvfp4 | bf16_mxfp8; act: swiglu | relu2; '#' starts
 * a comment).  The first line whose shape matches `shape` and whose token
 * range t_min <= T <= t_max holds T fills *knobs and sets *found = 1;
 * otherwise *knobs = the defaults and *found = 0.  Pass T = the buffer
 * capacity (max_tokens) to resolve knobs once per workspace, as the pages
 * do, or the call's own T.  A missing file is no error (*found = 0);
 * MOE_ERR_INVALID_ARG for NULL arguments or a malformed line (*found = 0,
 * *knobs = the defaults). */
MOE_API moe_status moe_knob_cache_lookup(const char* path, const moe_shape* shape, int32_t T, moe_knobs* knobs,
                                         int32_t* found);

/* Zero the synchronisation words at the start of a workspace (enqueued on
 * `stream`); needed once per workspace before moe_forward_fused. */
MOE_API moe_status moe_workspace_init(const moe_shape* shape, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
