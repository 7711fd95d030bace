// Routing, token permutation and activation / weight quantisation kernels.
#include "moe_kernels.h"

namespace moe {

// ------------------------------------------------------------------ routing
// One wave per token.  Each lane holds experts lane, lane+64, ... (E <= 1024,
// up to 16 per lane).  k rounds of a wave-wide arg-max under the total order
// (logit descending, id ascending) pick the experts; slot j is the j-th pick.
// Weights: softmax over the k picked logits [vLLM PR 40082 report,
// "Implementation" item 1: routing inside the fused call].
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int e = lane + 64 * i;
    float x = e < E ? row[e] : -INFINITY;
    v[i] = (x == x) ? x : -INFINITY;  // NaN never wins; results stay in range
    if (e >= E) taken |= 1u << i;
  }
  float my_val = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int id = lane + 64 * i;
      bool better = !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && id < bi));
      bv = better ? v[i] : bv;
      bi = better ? id : bi;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      float ov = __shfl_xor(bv, m, 64);
      int oi = __shfl_xor(bi, m, 64);
      bool better = ov > bv || (ov == bv && oi < bi);
      bv = better ? ov : bv;
      bi = better ? oi : bi;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  const float m0 = __shfl(my_val, 0, 64);
  float ex = lane < k ? expf(my_val - m0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = ex / sum;
  }
}

// ------------------------------------------------------------------ permutation
// Block 0: stable counting sort of the P = T*k pairs by expert.  Each of the 8
// waves owns a contiguous segment of pairs; pass 1 builds per-wave expert
// histograms in LDS, a scan turns them into per-(wave, expert) start
// positions, pass 2 walks each segment in order and ranks pairs of equal
// expert inside a 64-pair step with ballots on the id bits.
// Blocks 1..: in-kernel quantisation of the bf16 hidden states.
constexpr int kPermThreads = 512;
constexpr int kPermWaves = kPermThreads / 64;

__device__ void permute_block(const int* __restrict__ ids, int P, int E, int* __restrict__ offsets,
                              int* __restrict__ sorted_pairs, int* __restrict__ pair_pos) {
  __shared__ int hist[kPermWaves][1024];
  __shared__ int scan_tmp[kPermThreads];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kPermWaves * 1024; i += kPermThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int S = ((P + kPermWaves * 64 - 1) / (kPermWaves * 64)) * 64;  // segment, multiple of 64
  const int seg0 = min(P, w * S), seg1 = min(P, (w + 1) * S);
  // ids outside [0, E) are clamped: results are then unspecified but every access stays in bounds
  for (int p = seg0 + lane; p < seg1; p += 64) atomicAdd(&hist[w][min(max(ids[p], 0), E - 1)], 1);
  __syncthreads();
  // per-thread experts 2*tid, 2*tid+1: totals, block exclusive scan
  int e0 = 2 * tid, local = 0;
  int tot[2] = {0, 0};
  for (int j = 0; j < 2; ++j) {
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
  for (int j = 0; j < 2; ++j) {
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
  for (int p0 = seg0; p0 < seg1; p0 += 64) {
    const int p = p0 + lane;
    const bool valid = p < seg1;
    const int id = valid ? min(max(ids[p], 0), E - 1) : 0;
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
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
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
        uint32_t out = 0, d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c = e4m3_from_f32(ldexpf(v[j], -s));
          out |= c << (8 * j);
          d[j] = __float_as_uint(ldexpf(e4m3_to_f32(c), s)) >> 16;  // exact in bf16
        }
        if (ok) {
          reinterpret_cast<uint32_t*>(codes)[i] = out;
          if (sub == 0) scales[blk] = (uint8_t)(s + 127);
          reinterpret_cast<uint2*>(deq)[i] = make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
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

template <int DT>
__global__ __launch_bounds__(kPermThreads) void permute_quant_kernel(const int* __restrict__ ids, int P, int E,
                                                                     int* __restrict__ offsets,
                                                                     int* __restrict__ sorted_pairs,
                                                                     int* __restrict__ pair_pos,
                                                                     const uint16_t* __restrict__ x, long long n_elem,
                                                                     uint8_t* __restrict__ xq_codes,
                                                                     uint8_t* __restrict__ xq_scales,
                                                                     uint16_t* __restrict__ xq_deq, int do_quant) {
  if (blockIdx.x == 0) {
    permute_block(ids, P, E, offsets, sorted_pairs, pair_pos);
    return;
  }
  if (!do_quant) return;
  const long long gtid = (long long)(blockIdx.x - 1) * kPermThreads + threadIdx.x;
  const long long gstride = (long long)(gridDim.x - 1) * kPermThreads;
  quantize_x_blocks<DT>(x, n_elem, xq_codes, xq_scales, xq_deq, gtid, gstride);
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
    uint32_t out = e4m3_from_f32(ldexpf(v.x, -s)) | (e4m3_from_f32(ldexpf(v.y, -s)) << 8) |
                   (e4m3_from_f32(ldexpf(v.z, -s)) << 16) | (e4m3_from_f32(ldexpf(v.w, -s)) << 24);
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

// ------------------------------------------------------------------ launchers

hipError_t launch_route(const float* logits, int T, int E, int k, int* ids, float* wts, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, wts);
  return hipGetLastError();
}

hipError_t launch_permute(int dt, const int* ids, int T, int k, int E, int H, int* offsets, int* sorted_pairs,
                          int* pair_pos, const uint16_t* x, uint8_t* xq, hipStream_t s) {
  const int P = T * k;
  const long long n_elem = (long long)T * H;
  const int do_quant = !(dt == DT_BF16 && (const void*)xq == (const void*)x);
  uint8_t* xq_scales = xq + act_scale_offset(dt, T, H);
  uint16_t* xq_deq = reinterpret_cast<uint16_t*>(xq + act_dequant_offset(dt, T, H));
  long long work = dt == DT_BF16 ? n_elem / 8 : n_elem / 4;
  int qblocks = do_quant ? (int)min((work + kPermThreads - 1) / kPermThreads, (long long)4096) : 0;
  switch (dt) {
    case DT_BF16:
      hipLaunchKernelGGL(permute_quant_kernel<DT_BF16>, dim3(1 + qblocks), dim3(kPermThreads), 0, s, ids, P, E,
                         offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant);
      break;
    case DT_MXFP8:
      hipLaunchKernelGGL(permute_quant_kernel<DT_MXFP8>, dim3(1 + qblocks), dim3(kPermThreads), 0, s, ids, P, E,
                         offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant);
      break;
    default:
      hipLaunchKernelGGL(permute_quant_kernel<DT_NVFP4>, dim3(1 + qblocks), dim3(kPermThreads), 0, s, ids, P, E,
                         offsets, sorted_pairs, pair_pos, x, n_elem, xq, xq_scales, xq_deq, do_quant);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_weights(int dt, int count, int rows, int K, const float* w, void* codes, void* scales,
                                   float* alpha, hipStream_t s) {
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
