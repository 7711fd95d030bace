// C ABI entry points: host-side argument checks, then kernel launches on the
// caller's stream.  Nothing here allocates device memory, synchronises, or
// reads device data.
#include <atomic>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

constexpr int kMaxDevices = 64;

// Per-device cache of the compute-unit count (the library's only state).
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// occupancy of each GEMM variant, per device: [dev][dt][g13][variant], variant 3 = the fp8 prefill GEMM
std::atomic<int> g_occ[kMaxDevices][3][2][4];

// Persistent grid of one grouped GEMM under plan p.
int gemm_grid(int layer_dt, bool g13, const GemmPlan& p) {
  const int dt = weight_dt(layer_dt);  // the kernels are those of the weight format
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  int v = p.variant;
  if (v == 2 && !g13 && p.down_fp8 && has_fp8_gemm(layer_dt)) v = 3;
  if (p.blocks_per_cu > 0) return device_cu_count() * p.blocks_per_cu;
  int occ = 1;
  if (dev >= 0 && dev < kMaxDevices) {
    occ = g_occ[dev][dt][g13][v].load(std::memory_order_relaxed);
    if (occ <= 0) {
      occ = v == 3 ? prefill_f8_blocks_per_cu(g13) : v == 2 ? prefill_blocks_per_cu(dt, g13)
                                                             : gemm_blocks_per_cu(dt, g13, v + 1);
      g_occ[dev][dt][g13][v].store(occ, std::memory_order_relaxed);
    }
  }
  return device_cu_count() * occ;
}

// The plan of the default knobs for T tokens x k slots: the GEMM variant
// follows the rows per expert (32-row decode items where the prefill-shaped
// ones do not fit), the fp8 down GEMM is on where its offsets fit.
GemmPlan default_plan(int T, int k, int E, int H, int I, float limit) {
  GemmPlan p;
  p.variant = gemm_variant(T, k, E);
  if (p.variant == 2 && !prefill_fits(T, H, (long long)T * k, I)) p.variant = 1;
  p.down_fp8 = fp8_down_fits(T, k, I);
  p.limit = limit;
  return p;
}

// co-resident blocks of the fused kernel, per device: [dev][dt][variant]; -1 = unusable
std::atomic<int> g_fused_occ[kMaxDevices][3][4];

int fused_grid(int layer_dt, int T, int k, int E, int H, int I) {
  const int dt = weight_dt(layer_dt);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int v = fused_variant(layer_dt, T, k, E, H, I);
  int occ = g_fused_occ[dev][dt][v].load(std::memory_order_relaxed);
  if (occ == 0) {
    occ = fused_blocks_per_cu(dt, v);
    g_fused_occ[dev][dt][v].store(occ > 0 ? occ : -1, std::memory_order_relaxed);
  }
  return occ > 0 ? occ * device_cu_count() : 0;
}

static bool gated(const moe_shape* s) { return s->activation == MOE_SWIGLU; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->dtype < MOE_BF16 || s->dtype > MOE_BF16_MXFP8) return MOE_ERR_UNSUPPORTED;
  if (s->hidden <= 0 || s->inter <= 0 || s->hidden % 128 || s->inter % 128) return MOE_ERR_UNSUPPORTED;
  if (s->hidden > (1 << 20) || s->inter > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (s->num_experts < 1 || s->num_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (s->top_k < 1 || s->top_k > 32 || s->top_k > s->num_experts) return MOE_ERR_UNSUPPORTED;
  if (s->max_tokens < 1 || (long long)s->max_tokens * s->top_k > (1LL << 24)) return MOE_ERR_UNSUPPORTED;
  if (s->activation != MOE_SWIGLU && s->activation != MOE_RELU2) return MOE_ERR_UNSUPPORTED;
  if (!(s->gate_up_limit >= 0.f) || s->gate_up_limit > 3.0e38f) return MOE_ERR_INVALID_ARG;  // NaN, < 0, inf
  if (s->activation == MOE_RELU2 && s->gate_up_limit != 0.f) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_T(const moe_shape* s, int32_t T) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (T < 0 || T > s->max_tokens) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

// Device scratch of moe_forward_noalloc: the staged layer's intermediates for
// callers that cannot allocate.  Each device holds its own copy for the life
// of the process; in host code only the per-device address from
// hipGetSymbolAddress is used (the array's name is a host-side stand-in).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<uint8_t*> g_scratch[kMaxDevices];

// Address of this device's scratch array (looked up once per device, with the
// device current); nullptr if the lookup fails.
uint8_t* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(static_cast<uint8_t*>(q), std::memory_order_release);
  return static_cast<uint8_t*>(q);
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace or packed buffer too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape); }

size_t moe_packed_weight_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return packed_layout(s->dtype, s->num_experts, s->hidden, s->inter, gated(s)).total;
}

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return workspace_layout(s->dtype, s->num_experts, s->hidden, s->inter, s->top_k, s->max_tokens).total;
}

size_t moe_xq_bytes(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_bytes(s->dtype, T, s->hidden);
}

size_t moe_xq_scale_offset(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_scale_offset(s->dtype, T, s->hidden);
}

size_t moe_xq_dequant_offset(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_dequant_offset(s->dtype, T, s->hidden);
}

size_t moe_hq_dequant_offset(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_dequant_offset(s->dtype, T * s->top_k, s->inter);
}

size_t moe_hq_bytes(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_bytes(s->dtype, T * s->top_k, s->inter);
}

size_t moe_hq_scale_offset(const moe_shape* s, int32_t T) {
  if (check_T(s, T) != MOE_OK) return 0;
  return act_scale_offset(s->dtype, T * s->top_k, s->inter);
}

moe_status moe_nvfp4_fold_global_scale(int32_t count, int32_t rows, int32_t K, const void* scales_in,
                                       const float* alpha_in, void* scales_out, float* alpha_out, hipStream_t stream) {
  if (count < 0 || rows < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 16) return MOE_ERR_UNSUPPORTED;
  if ((long long)count * rows * (K / 16) > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (count == 0) return MOE_OK;
  if (!scales_in || !alpha_in || !scales_out || !alpha_out) return MOE_ERR_INVALID_ARG;
  return launched(launch_fold_global_scale(count, (long long)rows * (K / 16), (const uint8_t*)scales_in, alpha_in,
                                           (uint8_t*)scales_out, alpha_out, stream));
}

moe_status moe_quantize_weights(int32_t dtype, int32_t count, int32_t rows, int32_t K, const float* w, void* codes,
                                void* scales, float* alpha, hipStream_t stream) {
  if (dtype < MOE_BF16 || dtype > MOE_BF16_MXFP8) return MOE_ERR_UNSUPPORTED;
  dtype = weight_dt(dtype);  // MOE_BF16_MXFP8 weights are MXFP8
  if (count < 0 || rows < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  const int blk = dtype == MOE_MXFP8 ? 32 : (dtype == MOE_NVFP4 ? 16 : 8);
  if (K % blk) return MOE_ERR_UNSUPPORTED;
  if ((long long)count * rows * K > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (count == 0) return MOE_OK;
  if (!w || !codes) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && !scales) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_NVFP4 && !alpha) return MOE_ERR_INVALID_ARG;
  return launched(launch_quantize_weights(dtype, count, rows, K, w, codes, scales, alpha, stream));
}

moe_status moe_prepare_weights(const moe_shape* s, const void* w13_codes, const void* w13_scales,
                               const float* w13_alpha, const void* w2_codes, const void* w2_scales,
                               const float* w2_alpha, void* packed, size_t packed_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!w13_codes || !w2_codes || !packed) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_BF16 && (!w13_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
  if (s->dtype == MOE_NVFP4 && (!w13_alpha || !w2_alpha)) return MOE_ERR_INVALID_ARG;
  if (packed_bytes < moe_packed_weight_bytes(s)) return MOE_ERR_WORKSPACE;
  return launched(launch_prepare(s->dtype, gated(s), s->num_experts, s->hidden, s->inter, (const uint8_t*)w13_codes,
                                 (const uint8_t*)w13_scales, w13_alpha, (const uint8_t*)w2_codes,
                                 (const uint8_t*)w2_scales, w2_alpha, (uint8_t*)packed, stream));
}

moe_status moe_workspace_init(const moe_shape* s, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_workspace_bytes(s)) return MOE_ERR_WORKSPACE;
  return launched(launch_zero_sync((uint8_t*)ws, s->dtype, s->num_experts, s->hidden, s->inter, s->top_k,
                                   s->max_tokens, stream));
}

moe_status moe_route(const moe_shape* s, int32_t T, const float* logits, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream) {
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  return launched(launch_route(logits, T, s->num_experts, s->top_k, topk_ids, topk_w, stream));
}

moe_status moe_permute(const moe_shape* s, int32_t T, const int32_t* topk_ids, const uint16_t* x, int32_t* offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos, void* xq, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !x || !offsets || !sorted_pairs || !pair_pos || !xq) return MOE_ERR_INVALID_ARG;
  return launched(launch_permute(s->dtype, topk_ids, T, s->top_k, s->num_experts, s->hidden, offsets, sorted_pairs,
                                 pair_pos, x, (uint8_t*)xq, stream));
}

moe_status moe_gemm13_swiglu_quant(const moe_shape* s, int32_t T, const void* packed, const int32_t* offsets,
                                   const int32_t* sorted_pairs, const void* xq, void* hq, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!packed || !offsets || !sorted_pairs || !xq || !hq) return MOE_ERR_INVALID_ARG;
  const GemmPlan p = default_plan(T, s->top_k, s->num_experts, s->hidden, s->inter, s->gate_up_limit);
  return launched(launch_gemm13(s->dtype, gated(s), s->num_experts, s->hidden, s->inter, s->top_k, T, (const uint8_t*)packed,
                                offsets, sorted_pairs, (const uint8_t*)xq, (uint8_t*)hq, gemm_grid(s->dtype, true, p),
                                stream, p));
}

moe_status moe_gemm2(const moe_shape* s, int32_t T, const void* packed, const int32_t* offsets,
                     const int32_t* sorted_pairs, const void* hq, uint16_t* y, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!packed || !offsets || !sorted_pairs || !hq || !y) return MOE_ERR_INVALID_ARG;
  const GemmPlan p = default_plan(T, s->top_k, s->num_experts, s->hidden, s->inter, s->gate_up_limit);
  return launched(launch_gemm2(s->dtype, gated(s), s->num_experts, s->hidden, s->inter, s->top_k, T, (const uint8_t*)packed,
                               offsets, sorted_pairs, (const uint8_t*)hq, y, gemm_grid(s->dtype, false, p), stream, p));
}

moe_status moe_combine(const moe_shape* s, int32_t T, const uint16_t* y, const float* topk_w, uint16_t* out,
                       hipStream_t stream) {
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!y || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  return launched(launch_combine(T, s->hidden, s->top_k, y, topk_w, out, stream));
}

// Shared argument checks of the two whole-layer entry points.
static moe_status check_forward(const moe_shape* s, int32_t T, const void* packed, const float* logits,
                                const uint16_t* x, uint16_t* out, void* ws, size_t ws_bytes) {
  moe_status st = check_T(s, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!packed || !logits || !x || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_workspace_bytes(s)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// The five stage kernels of the layer on `stream`, intermediates in the
// workspace at `base` laid out for `cap` tokens (cap >= T), the GEMMs as plan
// p says.  With fc2 (the in-kernel fc2 reduce, top_k >= 2) the down GEMM
// adds w * y into an fp32 [T, H] accumulator in the y region (T H 4 bytes <=
// cap k H 2 bytes), zeroed first, and the combine becomes a conversion to bf16.
static moe_status forward_staged(const moe_shape* s, int32_t T, int cap, const void* packed, const float* logits,
                                 const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w, uint8_t* base,
                                 GemmPlan p, bool fc2, hipStream_t stream) {
  const int dt = s->dtype, E = s->num_experts, H = s->hidden, I = s->inter, k = s->top_k;
  const WorkspaceLayout W = workspace_layout(dt, E, H, I, k, cap);
  int32_t* ids = topk_ids ? topk_ids : (int32_t*)(base + W.ids);
  float* wts = topk_w ? topk_w : (float*)(base + W.wts);
  int32_t* offsets = (int32_t*)(base + W.offsets);
  int32_t* sorted_pairs = (int32_t*)(base + W.sorted_pairs);
  int32_t* pair_pos = (int32_t*)(base + W.pair_pos);
  uint8_t* xq = act_dt(dt) == DT_BF16 ? (uint8_t*)x : base + W.xq;  // bf16 activations are used in place
  uint8_t* hq = base + W.hq;
  uint16_t* y = (uint16_t*)(base + W.y);
  float* acc = fc2 ? (float*)(base + W.y) : nullptr;
  p.red = acc;
  p.wts = acc ? wts : nullptr;
  // the fp8 down GEMM reads the hq codes: the gate/up GEMM skips hq's 16-bit copy
  p.skip_hq_deq = p.variant == 2 && p.down_fp8 && has_fp8_gemm(dt);
  // a handful of tokens: routing and the sort in one launch
  hipError_t e = T <= route_permute_max_tokens()
                     ? launch_route_permute(dt, logits, T, k, E, H, ids, wts, offsets, sorted_pairs, pair_pos, x,
                                            xq, stream)
                     : launch_route(logits, T, E, k, ids, wts, stream);
  if (e == hipSuccess && T > route_permute_max_tokens())
    e = launch_permute(dt, ids, T, k, E, H, offsets, sorted_pairs, pair_pos, x, xq, stream);
  if (e == hipSuccess)
    e = launch_gemm13(dt, gated(s), E, H, I, k, T, (const uint8_t*)packed, offsets, sorted_pairs, xq, hq,
                      gemm_grid(dt, true, p), stream, p);
  if (e == hipSuccess && acc) e = launch_zero_f32(acc, (long long)T * H, stream);
  if (e == hipSuccess)
    e = launch_gemm2(dt, gated(s), E, H, I, k, T, (const uint8_t*)packed, offsets, sorted_pairs, hq, y,
                     gemm_grid(dt, false, p), stream, p);
  if (e == hipSuccess) e = acc ? launch_f32_to_bf16(acc, out, (long long)T * H, stream)
                               : launch_combine(T, H, k, y, wts, out, stream);
  return launched(e);
}

moe_status moe_forward(const moe_shape* s, int32_t T, const void* packed, const float* logits, const uint16_t* x,
                       uint16_t* out, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status st = check_forward(s, T, packed, logits, x, out, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  return forward_staged(s, T, s->max_tokens, packed, logits, x, out, topk_ids, topk_w, (uint8_t*)ws,
                        default_plan(T, s->top_k, s->num_experts, s->hidden, s->inter, s->gate_up_limit), false, stream);
}

void moe_default_knobs(moe_knobs* kn) {
  if (kn) *kn = moe_knobs{0, 1, 0, 0, 0, 0};
}

static bool knobs_valid(const moe_knobs& kn) {
  return kn.gemm >= 0 && kn.gemm <= 3 && (kn.down_fp8 | 1) == 1 && (kn.fc2_reduce | 1) == 1 && kn.band_rows >= 0 &&
         kn.band_rows <= (1 << 20) && kn.blocks_per_cu >= 0 && kn.blocks_per_cu <= 16 && kn.load_balance >= 0 &&
         kn.load_balance <= 3;
}

moe_status moe_forward_knobs(const moe_shape* s, int32_t T, const void* packed, const float* logits,
                             const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w, void* ws,
                             size_t ws_bytes, const moe_knobs* knobs, hipStream_t stream) {
  moe_knobs kn;
  moe_default_knobs(&kn);
  if (knobs) kn = *knobs;
  if (!knobs_valid(kn)) return MOE_ERR_INVALID_ARG;
  moe_status st = check_forward(s, T, packed, logits, x, out, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (kn.fc2_reduce && s->top_k < 2) return MOE_ERR_UNSUPPORTED;
  // the 16-row decode schedule packs two m-tile prefixes into 16-bit halves
  if (kn.gemm == 1 && (long long)T * s->top_k > 16LL * (65535 - s->num_experts)) return MOE_ERR_UNSUPPORTED;
  if (kn.gemm == 3 && !prefill_fits(T, s->hidden, (long long)T * s->top_k, s->inter)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  GemmPlan p = default_plan(T, s->top_k, s->num_experts, s->hidden, s->inter, s->gate_up_limit);
  if (kn.gemm > 0) p.variant = kn.gemm - 1;
  p.down_fp8 = p.down_fp8 && kn.down_fp8 != 0;
  p.band = kn.band_rows;
  p.blocks_per_cu = kn.blocks_per_cu;
  p.balance = kn.load_balance;
  return forward_staged(s, T, s->max_tokens, packed, logits, x, out, topk_ids, topk_w, (uint8_t*)ws, p,
                        kn.fc2_reduce != 0, stream);
}

moe_status moe_forward_noalloc(const moe_shape* s, int32_t T, const void* packed, const float* logits,
                               const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w,
                               hipStream_t stream) {
  moe_status st = check_T(s, T);
  if (st != MOE_OK || T == 0) return st;
  if (!packed || !logits || !x || !out) return MOE_ERR_INVALID_ARG;
  const size_t need = workspace_layout(s->dtype, s->num_experts, s->hidden, s->inter, s->top_k, T).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  uint8_t* base = scratch_address();
  if (!base) return MOE_ERR_LAUNCH;
  // every intermediate is written before it is read: nothing needs clearing
  return forward_staged(s, T, T, packed, logits, x, out, topk_ids, topk_w, base,
                        default_plan(T, s->top_k, s->num_experts, s->hidden, s->inter, s->gate_up_limit), false, stream);
}

size_t moe_batched_workspace_bytes(const moe_shape* s, int32_t max_rows) {
  if (check_shape(s) != MOE_OK || max_rows < 1 || (long long)s->num_experts * max_rows > (1LL << 24)) return 0;
  return batched_layout(s->dtype, s->num_experts, s->hidden, s->inter, max_rows).total;
}

moe_status moe_batched_experts(const moe_shape* s, int32_t max_rows, const int32_t* counts, const uint16_t* x,
                               const void* packed, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (max_rows < 1 || (long long)s->num_experts * max_rows > (1LL << 24)) return MOE_ERR_INVALID_ARG;
  if (!counts || !x || !packed || !y || !ws) return MOE_ERR_INVALID_ARG;
  const int dt = s->dtype, E = s->num_experts, H = s->hidden, I = s->inter, R = E * max_rows;
  const BatchedLayout B = batched_layout(dt, E, H, I, max_rows);
  if (ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  int32_t* offsets = (int32_t*)(base + B.offsets);
  int32_t* rows = (int32_t*)(base + B.rows);
  uint8_t* xq = act_dt(dt) == DT_BF16 ? (uint8_t*)x : base + B.xq;  // bf16 activations are used in place
  uint8_t* hq = base + B.hq;
  // one "pair" per valid row (k = 1, R rows of capacity): the GEMM variants follow the rows per expert
  const GemmPlan p = default_plan(R, 1, E, H, I, s->gate_up_limit);
  hipError_t e = launch_batched_prep(dt, counts, E, max_rows, H, offsets, rows, x, xq, stream);
  if (e == hipSuccess)
    e = launch_gemm13(dt, gated(s), E, H, I, 1, R, (const uint8_t*)packed, offsets, rows, xq, hq,
                      gemm_grid(dt, true, p), stream, p);
  if (e == hipSuccess)
    e = launch_gemm2(dt, gated(s), E, H, I, 1, R, (const uint8_t*)packed, offsets, rows, hq, y,
                     gemm_grid(dt, false, p), stream, p);
  return launched(e);
}

static bool dense_shape_ok(int32_t N, int32_t K) {
  return N >= 64 && K >= 128 && N % 64 == 0 && K % 128 == 0 && N <= (1 << 20) && K <= (1 << 20);
}

size_t moe_nvfp4_linear_packed_bytes(int32_t N, int32_t K) {
  return dense_shape_ok(N, K) ? dense_layout(N, K).total : 0;
}

size_t moe_nvfp4_linear_workspace_bytes(int32_t max_M, int32_t K) {
  if (max_M < 1 || max_M > (1 << 24) || K < 128 || K % 128 || K > (1 << 20)) return 0;
  return dense_workspace(max_M, K).total;
}

moe_status moe_nvfp4_linear_prepare(int32_t N, int32_t K, const void* codes, const void* scales, const float* alpha,
                                    void* packed, size_t packed_bytes, hipStream_t stream) {
  if (!dense_shape_ok(N, K)) return MOE_ERR_UNSUPPORTED;
  if (!codes || !scales || !alpha || !packed) return MOE_ERR_INVALID_ARG;
  if (packed_bytes < dense_layout(N, K).total) return MOE_ERR_WORKSPACE;
  return launched(launch_dense_prepare(N, K, (const uint8_t*)codes, (const uint8_t*)scales, alpha, (uint8_t*)packed,
                                       stream));
}

moe_status moe_nvfp4_linear(int32_t M, int32_t N, int32_t K, const void* packed, const uint16_t* x, uint16_t* out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dense_shape_ok(N, K)) return MOE_ERR_UNSUPPORTED;
  if (M < 0 || M > (1 << 24)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!packed || !x || !out || !ws) return MOE_ERR_INVALID_ARG;
  const DenseWorkspace W = dense_workspace(M, K);
  if (ws_bytes < W.total) return MOE_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  int32_t* offsets = (int32_t*)(base + W.offsets);
  int32_t* rows = (int32_t*)(base + W.rows);
  uint8_t* xq = base + W.xq;
  hipError_t e = launch_dense_prep(M, K, offsets, rows, x, xq, stream);
  if (e == hipSuccess)
    e = launch_dense_gemm(M, N, K, (const uint8_t*)packed, offsets, rows, xq, out,
                          gemm_grid(MOE_NVFP4, false, default_plan(M, 1, 1, K, K, 0.f)), stream);
  return launched(e);
}

moe_status moe_forward_fused(const moe_shape* s, int32_t T, const void* packed, const float* logits,
                             const uint16_t* x, uint16_t* out, int32_t* topk_ids, float* topk_w, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_forward(s, T, packed, logits, x, out, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const int dt = s->dtype, E = s->num_experts, H = s->hidden, I = s->inter, k = s->top_k;
  const WorkspaceLayout W = workspace_layout(dt, E, H, I, k, s->max_tokens);
  uint8_t* base = (uint8_t*)ws;
  int32_t* ids = topk_ids ? topk_ids : (int32_t*)(base + W.ids);
  float* wts = topk_w ? topk_w : (float*)(base + W.wts);
  const int grid = fused_grid(dt, T, k, E, H, I);
  if (grid <= 0) return MOE_ERR_UNSUPPORTED;
  return launched(launch_fused(dt, gated(s), E, H, I, k, T, (const uint8_t*)packed, logits, x, out, ids, wts, base, ws_bytes,
                               s->max_tokens, grid, stream, s->gate_up_limit));
}

static int parse_dtype(const char* t) {
  static const char* names[] = {"bf16", "mxfp8", "nvfp4", "bf16_mxfp8"};
  for (int i = 0; i < 4; ++i)
    if (!strcmp(t, names[i])) return i;
  return -1;
}

moe_status moe_knob_cache_lookup(const char* path, const moe_shape* s, int32_t T, moe_knobs* knobs,
                                 int32_t* found) {
  if (!path || !s || !knobs || !found) return MOE_ERR_INVALID_ARG;
  moe_default_knobs(knobs);
  *found = 0;
  FILE* f = fopen(path, "r");
  if (!f) return MOE_OK;
  char line[512];
  moe_status st = MOE_OK;
  while (fgets(line, sizeof line, f)) {
    if (char* c = strchr(line, '#')) *c = 0;
    constexpr int kKeys = 8, kKnobs = 6, kTok = kKeys + 1 + kKnobs;
    char* tok[kTok];
    int n = 0;
    char* save = nullptr;
    for (char* t = strtok_r(line, " \t\r\n", &save); t; t = strtok_r(nullptr, " \t\r\n", &save)) {
      if (n == kTok) { n = kTok + 1; break; }
      tok[n++] = t;
    }
    if (n == 0) continue;
    long v[kKeys + kKnobs] = {};  // v[2..7]: hidden inter experts top_k t_min t_max; v[8..]: the knobs
    bool ok = n == kTok && !strcmp(tok[kKeys], ":");
    for (int i = 2; ok && i < kTok; ++i) {
      if (i == kKeys) continue;
      char* end = nullptr;
      const long x = strtol(tok[i], &end, 10);
      ok = end != tok[i] && *end == 0 && x >= INT_MIN && x <= INT_MAX;
      v[i < kKeys ? i : i - 1] = x;
    }
    const int dt = ok ? parse_dtype(tok[0]) : -1;
    const int act = ok ? (!strcmp(tok[1], "swiglu") ? MOE_SWIGLU : !strcmp(tok[1], "relu2") ? MOE_RELU2 : -1) : -1;
    const moe_knobs kn{(int32_t)v[8],  (int32_t)v[9],  (int32_t)v[10],
                       (int32_t)v[11], (int32_t)v[12], (int32_t)v[13]};
    if (!ok || dt < 0 || act < 0 || !knobs_valid(kn)) {
      st = MOE_ERR_INVALID_ARG;
      break;
    }
    if (dt == s->dtype && act == s->activation && v[2] == s->hidden && v[3] == s->inter && v[4] == s->num_experts &&
        v[5] == s->top_k && v[6] <= T && T <= v[7]) {
      *knobs = kn;
      *found = 1;
      break;
    }
  }
  fclose(f);
  if (st != MOE_OK) {
    moe_default_knobs(knobs);
    *found = 0;
  }
  return st;
}

}  // extern "C"
