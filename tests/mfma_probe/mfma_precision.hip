// Test instrument: accumulation precision of the gfx950 matrix instructions
// on MX-scaled e4m3 operands (e4m3 codes with one e8m0 scale per 32 along K,
// the MXFP8 format of the layer).  Not part of the MoE library.
//
// For A [32 tiles, K] and B [32, K], wave t computes the 32 x 32 tile
// A[32 t .. 32 t + 32) B^T three ways:
//   chain: the block-scaled fp8 instruction (v_mfma_scale_f32_32x32x64_f8f6f4)
//          accumulating in its own C operand over the K / 64 steps;
//   fresh: the same instruction with a zero C operand at every step, the
//          step results summed in fp32 by vector adds;
//   bf16:  every e4m3 value times its scale converted to bf16 (exact: 4
//          significant bits, a power-of-two scale) and the bf16 instruction
//          (v_mfma_f32_32x32x16_bf16) accumulating over the K / 16 steps.
// Operand layouts (32 x 32 family): lane l holds row l % 32 of A (of B).
// fp8, a 64-long K step: bytes 0-15 of lane l are K offsets 16 (l / 32) +
// [0, 16), bytes 16-31 are 32 + 16 (l / 32) + [0, 16), and the scale operand
// of lane l applies to bytes 0-15 (l < 32) or 16-31 (l >= 32) of both lanes
// of its row -- K block l / 32 of the step (the grouping measured with one
// lane's scale changed at a time).  bf16, a 16-long K step: lane l holds K
// offsets 8 (l / 32) + [0, 8).  Result element i of lane l is
// D[(i % 4) + 8 (i / 4) + 4 (l / 32)][l % 32].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline bf16x8_t to_bf16(uint2 w, uint32_t e8m0) {
  const float sc = __uint_as_float(e8m0 << 23);  // 2^(e8m0 - 127) for e8m0 in [1, 254]
  bf16x2_t r[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, false),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, true),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, false),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, true)};
  bf16x8_t o;
  __builtin_memcpy(&o, r, 16);
  return o;
}

// the 32 fp8 bytes of half h of a 64-long K step starting at p
__device__ inline i32x8_t load_fp8_operand(const uint8_t* p, int h) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p + 16 * h);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 32 + 16 * h);
  i32x8_t v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

__global__ __launch_bounds__(64) void precision_kernel(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                                       const uint8_t* sb, int K, float* chain, float* fresh,
                                                       float* viabf16) {
  const int l = threadIdx.x, r = l & 31, h = l >> 5, t = blockIdx.x;
  const uint8_t* ar = a + (size_t)(32 * t + r) * K;
  const uint8_t* br = b + (size_t)r * K;
  const uint8_t* sar = sa + (size_t)(32 * t + r) * (K / 32);
  const uint8_t* sbr = sb + (size_t)r * (K / 32);
  const f32x16_t zero = {};
  f32x16_t c = {}, f = {}, q = {};
  for (int k0 = 0; k0 < K; k0 += 64) {
    const i32x8_t av = load_fp8_operand(ar + k0, h), bv = load_fp8_operand(br + k0, h);
    const int s_a = sar[k0 / 32 + h], s_b = sbr[k0 / 32 + h];
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, s_a, 0, s_b);
    const f32x16_t step = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, zero, 0, 0, 0, s_a, 0, s_b);
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] += step[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = k0 + 16 * j + 8 * h;
      const bf16x8_t a8 = to_bf16(*reinterpret_cast<const uint2*>(ar + kk), sar[kk / 32]);
      const bf16x8_t b8 = to_bf16(*reinterpret_cast<const uint2*>(br + kk), sbr[kk / 32]);
      q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, q, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const size_t o = ((size_t)32 * t + (i & 3) + 8 * (i >> 2) + 4 * h) * 32 + r;
    chain[o] = c[i];
    fresh[o] = f[i];
    viabf16[o] = q[i];
  }
}

}  // namespace

// a [32 tiles, K] and b [32, K] e4m3 codes, sa [32 tiles, K / 32] and
// sb [32, K / 32] e8m0 bytes in [1, 254] (device, row-major); chain, fresh,
// viabf16 [32 tiles, 32] fp32 (device).  K a positive multiple of 64.
// Returns 0, 1 for bad sizes, 2 for a launch error.
extern "C" __attribute__((visibility("default"))) int mfma_precision_probe(const void* a, const void* sa,
                                                                           const void* b, const void* sb,
                                                                           int tiles, int K, float* chain,
                                                                           float* fresh, float* viabf16,
                                                                           void* stream) {
  if (tiles <= 0 || K <= 0 || K % 64 != 0) return 1;
  hipLaunchKernelGGL(precision_kernel, dim3(tiles), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                     (const uint8_t*)sa, (const uint8_t*)b, (const uint8_t*)sb, K, chain, fresh, viabf16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
