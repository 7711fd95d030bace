// Routing, token permutation and activation / weight quantisation kernels.
#include "moe_stages.h"

namespace moe {

// ------------------------------------------------------------------ routing
// One wave per token.  Each lane holds experts lane, lane+64, ... (E <= 1024,
// up to 16 per lane).  k rounds of a wave-wide arg-max under the total order
// (logit descending, id ascending) pick the experts; slot j is the j-th pick.
// Weights: softmax over the k picked logits [vLLM PR 40082 report,
// "Implementation" item 1: routing inside the fused call].
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int* __restrict__ ids, float* __restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < T) route_token(logits, t, E, k, ids, wts, threadIdx.x & 63);
}

// Blocks 0 .. nsort-1: the stable counting sort (one block: permute_block;
// several, for large P: permute_chunk over chunks of `chunk` pairs); the
// other blocks: in-kernel quantisation of the bf16 hidden states.
constexpr int kPermThreads = 512;
// Pairs up to which one block sorts (a decode batch); above it the sort is
// split into chunks of at least kPermChunkMin pairs over at most
// kPermMaxSortBlocks blocks, each of which counts all P ids once.
constexpr int kPermOneBlockMax = 16384, kPermChunkMin = 4096, kPermMaxSortBlocks = 32;

template <int DT>
__global__ __launch_bounds__(kPermThreads) void permute_quant_kernel(const int* __restrict__ ids, int P, int E,
                                                                     int* __restrict__ offsets,
                                                                     int* __restrict__ sorted_pairs,
                                                                     int* __restrict__ pair_pos,
                                                                     const uint16_t* __restrict__ x, long long n_elem,
                                                                     uint8_t* __restrict__ xq_codes,
                                                                     uint8_t* __restrict__ xq_scales,
                                                                     uint16_t* __restrict__ xq_deq, int do_quant,
                                                                     int nsort, int chunk) {
  extern __shared__ int perm_lds[];  // sized by the launch for the sort blocks' path
  constexpr int NW = kPermThreads / 64;
  if ((int)blockIdx.x < nsort) {
    if (nsort == 1) {
      permute_block<NW>(ids, P, E, offsets, sorted_pairs, pair_pos, reinterpret_cast<int(*)[1024]>(perm_lds),
                        perm_lds + NW * 1024);
    } else {
      const int c0 = min(P, (int)blockIdx.x * chunk);
      permute_chunk<NW>(ids, P, E, c0, min(P, c0 + chunk), offsets, sorted_pairs, pair_pos, perm_lds);
    }
    return;
  }
  if (!do_quant) return;
  const long long gtid = (long long)(blockIdx.x - nsort) * kPermThreads + threadIdx.x;
  const long long gstride = (long long)(gridDim.x - nsort) * kPermThreads;
  quantize_x_blocks<DT>(x, n_elem, xq_codes, xq_scales, xq_deq, gtid, gstride);
}

// Small batches (T <= the sorting block's waves): block 0 routes the tokens
// (one wave each) and then sorts the pairs it wrote, so a decode step needs
// one launch for routing and permutation instead of two; the other blocks
// quantise x as in permute_quant_kernel.  Same routing and sort code, so the
// same bits as moe_route followed by moe_permute.
template <int DT>
__global__ __launch_bounds__(kPermThreads) void route_permute_quant_kernel(
    const float* __restrict__ logits, int T, int k, int E, int* ids, float* __restrict__ wts,
    int* __restrict__ offsets, int* __restrict__ sorted_pairs, int* __restrict__ pair_pos,
    const uint16_t* __restrict__ x, long long n_elem, uint8_t* __restrict__ xq_codes,
    uint8_t* __restrict__ xq_scales, uint16_t* __restrict__ xq_deq, int do_quant) {
  extern __shared__ int perm_lds[];
  constexpr int NW = kPermThreads / 64;
  if (blockIdx.x == 0) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int t = w; t < T; t += NW) route_token(logits, t, E, k, ids, wts, lane);
    __syncthreads();  // the block's id stores before its sort reads them
    permute_block<NW>(ids, T * k, E, offsets, sorted_pairs, pair_pos, reinterpret_cast<int(*)[1024]>(perm_lds),
                      perm_lds + NW * 1024);
    return;
  }
  if (!do_quant) return;
  const long long gtid = (long long)(blockIdx.x - 1) * kPermThreads + threadIdx.x;
  const long long gstride = (long long)(gridDim.x - 1) * kPermThreads;
  quantize_x_blocks<DT>(x, n_elem, xq_codes, xq_scales, xq_deq, gtid, gstride);
}

// ------------------------------------------------------------------ batched activation format
// Tokens arrive bucketed per expert, x [E, M, H] with counts[e] valid rows
// (clamped to [0, M]).  The grouped GEMMs then run with one "pair" per valid
// row: offsets = exclusive prefix of the clamped counts, rows[offsets[e] + r]
// = e M + r (the row of the batched buffer), so the gate/up GEMM reads
// activation row rows[i] and the down GEMM writes y row rows[i] in place.

// One block of 1024 threads: offsets[0..E] (E <= 1024).
__global__ __launch_bounds__(1024) void batched_offsets_kernel(const int* __restrict__ counts, int E, int M,
                                                               int* __restrict__ offsets) {
  __shared__ int sc[1024];
  const int t = threadIdx.x;
  const int c = t < E ? min(max(counts[t], 0), M) : 0;
  sc[t] = c;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // Hillis-Steele inclusive scan
    const int v = t >= d ? sc[t - d] : 0;
    __syncthreads();
    sc[t] += v;
    __syncthreads();
  }
  if (t < E) offsets[t] = sc[t] - c;
  if (t == E - 1) offsets[E] = sc[t];
}

// rows[] of every valid row, and (unless the activations are used in place)
// the quantisation of all E M rows of x.
template <int DT>
__global__ __launch_bounds__(kPermThreads) void batched_rows_quant_kernel(
    const int* __restrict__ counts, const int* __restrict__ offsets, int E, int M, int* __restrict__ rows,
    const uint16_t* __restrict__ x, long long n_elem, uint8_t* __restrict__ xq_codes, uint8_t* __restrict__ xq_scales,
    uint16_t* __restrict__ xq_deq, int do_quant) {
  const long long gtid = (long long)blockIdx.x * kPermThreads + threadIdx.x;
  const long long gstride = (long long)gridDim.x * kPermThreads;
  for (long long i = gtid; i < (long long)E * M; i += gstride) {
    const int e = (int)(i / M), r = (int)(i % M);
    if (r < min(max(counts[e], 0), M)) rows[offsets[e] + r] = (int)i;
  }
  if (do_quant) quantize_x_blocks<DT>(x, n_elem, xq_codes, xq_scales, xq_deq, gtid, gstride);
}

hipError_t launch_batched_prep(int dt, const int* counts, int E, int M, int H, int* offsets, int* rows,
                               const uint16_t* x, uint8_t* xq, hipStream_t s) {
  dt = act_dt(dt);
  const int R = E * M;
  hipLaunchKernelGGL(batched_offsets_kernel, dim3(1), dim3(1024), 0, s, counts, E, M, offsets);
  const long long n_elem = (long long)R * H;
  const int do_quant = dt != DT_BF16;
  uint8_t* xq_scales = do_quant ? xq + act_scale_offset(dt, R, H) : nullptr;
  uint16_t* xq_deq = do_quant ? reinterpret_cast<uint16_t*>(xq + act_dequant_offset(dt, R, H)) : nullptr;
  const long long work = do_quant ? n_elem / 4 : (long long)R;
  const int blocks = (int)min((work + kPermThreads - 1) / kPermThreads, (long long)4096);
  if (dt == DT_MXFP8)
    hipLaunchKernelGGL(batched_rows_quant_kernel<DT_MXFP8>, dim3(blocks), dim3(kPermThreads), 0, s, counts, offsets,
                       E, M, rows, x, n_elem, xq, xq_scales, xq_deq, do_quant);
  else if (dt == DT_NVFP4)
    hipLaunchKernelGGL(batched_rows_quant_kernel<DT_NVFP4>, dim3(blocks), dim3(kPermThreads), 0, s, counts, offsets,
                       E, M, rows, x, n_elem, xq, xq_scales, xq_deq, do_quant);
  else
    hipLaunchKernelGGL(batched_rows_quant_kernel<DT_BF16>, dim3(blocks), dim3(kPermThreads), 0, s, counts, offsets,
                       E, M, rows, x, n_elem, xq, xq_scales, xq_deq, 0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dense NVFP4 linear
// One "expert" holding all M rows: offsets {0, M}, rows[i] = i, and the
// NVFP4 quantisation of x [M, K] (per 16, global scale 1).
__global__ __launch_bounds__(kPermThreads) void dense_prep_kernel(int M, int* __restrict__ offsets,
                                                                  int* __restrict__ rows,
                                                                  const uint16_t* __restrict__ x, long long n_elem,
                                                                  uint8_t* __restrict__ xq_codes,
                                                                  uint8_t* __restrict__ xq_scales,
                                                                  uint16_t* __restrict__ xq_deq) {
  const long long gtid = (long long)blockIdx.x * kPermThreads + threadIdx.x;
  const long long gstride = (long long)gridDim.x * kPermThreads;
  if (gtid == 0) {
    offsets[0] = 0;
    offsets[1] = M;
  }
  for (long long i = gtid; i < M; i += gstride) rows[i] = (int)i;
  quantize_x_blocks<DT_NVFP4>(x, n_elem, xq_codes, xq_scales, xq_deq, gtid, gstride);
}

hipError_t launch_dense_prep(int M, int K, int* offsets, int* rows, const uint16_t* x, uint8_t* xq, hipStream_t s) {
  const long long n_elem = (long long)M * K;
  const int blocks = (int)min((n_elem / 4 + kPermThreads - 1) / kPermThreads, (long long)4096);
  hipLaunchKernelGGL(dense_prep_kernel, dim3(max(blocks, 1)), dim3(kPermThreads), 0, s, M, offsets, rows, x, n_elem,
                     xq, xq + act_scale_offset(DT_NVFP4, M, K),
                     reinterpret_cast<uint16_t*>(xq + act_dequant_offset(DT_NVFP4, M, K)));
  return hipGetLastError();
}

// ------------------------------------------------------------------ weight quantisation
// fp32 master weights -> canonical codes (the load-time preprocessing step).

__global__ void quant_w_bf16_kernel(const float* __restrict__ w, long long n, uint16_t* __restrict__ out) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    out[i] = f32_to_bf16(w[i]);
}

// MXFP8: 8 lanes x 4 elements per block of 32 along K.
__global__ void quant_w_mxfp8_kernel(const float* __restrict__ w, long long n, uint8_t* __restrict__ codes,
                                     uint8_t* __restrict__ scales) {
  const long long nthreads = n / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < ((nthreads + 63) / 64) * 64;
       i += (long long)gridDim.x * blockDim.x) {
    const bool ok = i < nthreads;
    float4 v = ok ? reinterpret_cast<const float4*>(w)[i] : make_float4(0, 0, 0, 0);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = wave_max_xor(amax, 1, 4);
    int s = mx_scale_exp(amax);
    const uint32_t out = e4m3x4_from_f32(ldexpf(v.x, -s), ldexpf(v.y, -s), ldexpf(v.z, -s), ldexpf(v.w, -s));
    if (ok) {
      reinterpret_cast<uint32_t*>(codes)[i] = out;
      if ((i & 7) == 0) scales[i >> 3] = (uint8_t)(s + 127);
    }
  }
}

// NVFP4 pass 1: per-matrix amax as fp32 bits (non-negative floats order like
// their bit patterns), atomically max-ed into amax_bits[m] (zeroed first).
__global__ void amax_per_matrix_kernel(const float* __restrict__ w, long long per_matrix, int count,
                                       unsigned int* __restrict__ amax_bits) {
  const int m = blockIdx.y;
  const float* src = w + (long long)m * per_matrix;
  float a = 0.f;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < per_matrix;
       i += (long long)gridDim.x * blockDim.x)
    a = fmaxf(a, fabsf(src[i]));
  a = wave_max_xor(a, 1, 32);
  if ((threadIdx.x & 63) == 0) atomicMax(&amax_bits[m], __float_as_uint(a));
}

// NVFP4 pass 2: 4 lanes x 4 elements per block of 16; alpha = amax / 2688.
__global__ void quant_w_nvfp4_kernel(const float* __restrict__ w, long long per_matrix, int count,
                                     const unsigned int* __restrict__ amax_bits, uint8_t* __restrict__ codes,
                                     uint8_t* __restrict__ scales) {
  const long long nthreads = per_matrix * count / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < ((nthreads + 63) / 64) * 64;
       i += (long long)gridDim.x * blockDim.x) {
    const bool ok = i < nthreads;
    const int m = ok ? (int)((i * 4) / per_matrix) : 0;
    const float amax_e = __uint_as_float(amax_bits[m]);
    const float alpha = amax_e > 0.f ? amax_e / 2688.0f : 1.0f;
    float4 v = ok ? reinterpret_cast<const float4*>(w)[i] : make_float4(0, 0, 0, 0);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = wave_max_xor(amax, 1, 2);
    const float t = amax / 6.0f;
    const float u = t / alpha;
    const uint32_t sc_code = e4m3_from_f32(u);
    const float d = e4m3_to_f32(sc_code) * alpha;
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t c = d > 0.f ? e2m1_from_f32(vv[j] / d, 1.0f) : ((__float_as_uint(vv[j]) >> 28) & 8u);
      out |= c << (4 * j);
    }
    if (ok) {
      reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)out;
      if ((i & 3) == 0) scales[i >> 2] = (uint8_t)sc_code;
    }
  }
}

__global__ void alpha_finalize_kernel(unsigned int* __restrict__ amax_bits_then_alpha, int count) {
  int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < count) {
    float a = __uint_as_float(amax_bits_then_alpha[m]);
    float alpha = a > 0.f ? a / 2688.0f : 1.0f;
    reinterpret_cast<float*>(amax_bits_then_alpha)[m] = alpha;
  }
}

__global__ void fill_u32_kernel(unsigned int* __restrict__ p, long long n, unsigned int v) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

// NVFP4 global-scale fold: one e4m3 block scale per thread (grid-stride).
__global__ void fold_scale_kernel(const uint8_t* __restrict__ in, const float* __restrict__ alpha, long long n,
                                  long long per_matrix, uint8_t* __restrict__ out) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    out[i] = (uint8_t)e4m3_from_f32(e4m3_to_f32(in[i]) * alpha[i / per_matrix]);
}

hipError_t launch_fold_global_scale(int count, long long scales_per_matrix, const uint8_t* scales_in,
                                    const float* alpha_in, uint8_t* scales_out, float* alpha_out, hipStream_t s) {
  const long long n = (long long)count * scales_per_matrix;
  const int threads = 256, blocks = (int)min((n + threads - 1) / threads, (long long)65536);
  hipLaunchKernelGGL(fold_scale_kernel, dim3(blocks), dim3(threads), 0, s, scales_in, alpha_in, n, scales_per_matrix,
                     scales_out);
  // a second launch, so that alpha_out may alias alpha_in
  hipLaunchKernelGGL(fill_u32_kernel, dim3((count + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<unsigned int*>(alpha_out), (long long)count, 0x3F800000u);
  return hipGetLastError();
}


// ------------------------------------------------------------------ launchers

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* wts, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

int route_permute_max_tokens() { return kPermThreads / 64; }

hipError_t launch_route_permute(int dt, const float* logits, int T, int k, int E, int H, int* ids, float* wts,
                                int* offsets, int* sorted_pairs, int* pair_pos, const uint16_t* x, uint8_t* xq,
                                hipStream_t s) {
  if (T > route_permute_max_tokens()) return hipErrorInvalidValue;
  dt = act_dt(dt);
  const long long n_elem = (long long)T * H;
  const int do_quant = !(dt == DT_BF16 && (const void*)xq == (const void*)x);
  uint8_t* xq_scales = xq + act_scale_offset(dt, T, H);
  uint16_t* xq_deq = reinterpret_cast<uint16_t*>(xq + act_dequant_offset(dt, T, H));
  const long long work = dt == DT_BF16 ? n_elem / 8 : n_elem / 4;
  const int qblocks = do_quant ? (int)min((work + kPermThreads - 1) / kPermThreads, (long long)4096) : 0;
  const size_t lds = sizeof(int) * permute_lds_ints<kPermThreads / 64>();
#define MOE_RP(D)                                                                                              \
  hipLaunchKernelGGL(route_permute_quant_kernel<D>, dim3(1 + qblocks), dim3(kPermThreads), lds, s, logits, T, k, \
                     E, ids, wts, offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant)
  if (dt == DT_BF16) MOE_RP(DT_BF16);
  else if (dt == DT_MXFP8) MOE_RP(DT_MXFP8);
  else MOE_RP(DT_NVFP4);
#undef MOE_RP
  return hipGetLastError();
}

hipError_t launch_permute(int dt, const int* ids, int T, int k, int E, int H, int* offsets, int* sorted_pairs,
                          int* pair_pos, const uint16_t* x, uint8_t* xq, hipStream_t s) {
  dt = act_dt(dt);  // only the activation format matters here
  const int P = T * k;
  const long long n_elem = (long long)T * H;
  const int do_quant = !(dt == DT_BF16 && (const void*)xq == (const void*)x);
  uint8_t* xq_scales = xq + act_scale_offset(dt, T, H);
  uint16_t* xq_deq = reinterpret_cast<uint16_t*>(xq + act_dequant_offset(dt, T, H));
  long long work = dt == DT_BF16 ? n_elem / 8 : n_elem / 4;
  int qblocks = do_quant ? (int)min((work + kPermThreads - 1) / kPermThreads, (long long)4096) : 0;
  // sort blocks: one up to kPermOneBlockMax pairs, else chunks (multiples of
  // 64 waves' steps) over at most kPermMaxSortBlocks blocks, none empty
  int nsort = 1, chunk = P;
  if (P > kPermOneBlockMax) {
    const int per = kPermThreads;  // chunk granularity: one 64-pair step per wave
    const int want = (int)min((long long)kPermMaxSortBlocks, ((long long)P + kPermChunkMin - 1) / kPermChunkMin);
    chunk = (int)((((long long)P + want - 1) / want + per - 1) / per * per);
    nsort = (P + chunk - 1) / chunk;
  }
  const size_t lds = sizeof(int) * (nsort == 1 ? permute_lds_ints<kPermThreads / 64>()
                                               : permute_chunk_lds_ints<kPermThreads / 64>(E));
  switch (dt) {
    case DT_BF16:
      hipLaunchKernelGGL(permute_quant_kernel<DT_BF16>, dim3(nsort + qblocks), dim3(kPermThreads), lds, s, ids, P,
                         E, offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant, nsort,
                         chunk);
      break;
    case DT_MXFP8:
      hipLaunchKernelGGL(permute_quant_kernel<DT_MXFP8>, dim3(nsort + qblocks), dim3(kPermThreads), lds, s, ids, P,
                         E, offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant, nsort,
                         chunk);
      break;
    default:
      hipLaunchKernelGGL(permute_quant_kernel<DT_NVFP4>, dim3(nsort + qblocks), dim3(kPermThreads), lds, s, ids, P,
                         E, offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant, nsort,
                         chunk);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_weights(int dt, int count, int rows, int K, const float* w, void* codes, void* scales,
                                   float* alpha, hipStream_t s) {
  dt = weight_dt(dt);
  const long long n = (long long)count * rows * K;
  const int threads = 256;
  if (dt == DT_BF16) {
    int blocks = (int)min((n + threads - 1) / threads, (long long)65536);
    hipLaunchKernelGGL(quant_w_bf16_kernel, dim3(blocks), dim3(threads), 0, s, w, n, (uint16_t*)codes);
  } else if (dt == DT_MXFP8) {
    int blocks = (int)min((n / 4 + threads - 1) / threads, (long long)65536);
    hipLaunchKernelGGL(quant_w_mxfp8_kernel, dim3(blocks), dim3(threads), 0, s, w, n, (uint8_t*)codes,
                       (uint8_t*)scales);
  } else {
    unsigned int* bits = reinterpret_cast<unsigned int*>(alpha);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((count + 255) / 256), dim3(256), 0, s, bits, (long long)count, 0u);
    const long long per = (long long)rows * K;
    int bx = (int)min((per + threads - 1) / threads, (long long)1024);
    hipLaunchKernelGGL(amax_per_matrix_kernel, dim3(bx, count), dim3(threads), 0, s, w, per, count, bits);
    int blocks = (int)min((n / 4 + threads - 1) / threads, (long long)65536);
    hipLaunchKernelGGL(quant_w_nvfp4_kernel, dim3(blocks), dim3(threads), 0, s, w, per, count,
                       (const unsigned int*)bits, (uint8_t*)codes, (uint8_t*)scales);
    hipLaunchKernelGGL(alpha_finalize_kernel, dim3((count + 255) / 256), dim3(256), 0, s, bits, count);
  }
  return hipGetLastError();
}

}  // namespace moe
