// Achievable-peak probe for the benchmark's roofline context (not part of the
// MoE library): a stream of independent v_mfma_f32_32x32x16_bf16 from
// registers, no memory traffic in the loop.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters, float seed) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed * (float)(i - (int)threadIdx.x));
  }
  f32x16_t acc[8];
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Enqueue `blocks` blocks of 256 threads, each wave issuing iters x 8 MFMAs
// (32x32x16 bf16, 32768 flops each); `out` holds blocks * 256 floats.
extern "C" __attribute__((visibility("default"))) int moe_probe_mfma_bf16(float* out, int blocks, int iters,
                                                                           hipStream_t s) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
