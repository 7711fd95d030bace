// Device-side building blocks of the MI355X (gfx950) MoE library: element
// codecs (bit-exact, integer-only where rounding decides a code), wave-level
// reductions and the MFMA operand types.
//
// Formats: OCP e4m3fn (bias 7, max 448, no inf), OCP MX e2m1 and e8m0, bf16.
// Rounding: nearest, ties to even; encoders saturate to the largest finite
// magnitude and carry the sign bit over (a value that rounds to zero keeps
// its sign).  The pages name the formats and block sizes only (NVFP4 = e2m1 +
// e4m3 scale per 16, MXFP8 = e4m3 + e8m0 scale per 32) [MegaMoE drop
// workflow, §3, the per-block quantise helpers of kernel_helpers.py].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 round to nearest even (finite inputs; overflow rounds to
// inf), by the hardware convert (v_cvt_pk_bf16_f32).  It agrees bit for bit
// with the integer rounding (u + 0x7FFF + lsb) >> 16 on finite inputs:
// checked on MI355X over 4M random fp32 bit patterns (denormals and
// overflow included) and every tie of every bf16 value.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 b = (__bf16)f;
  uint16_t u;
  __builtin_memcpy(&u, &b, 2);
  return u;
}

// fp32 -> fp16 bits (round to nearest even; used only for values that are
// exactly representable, so no rounding happens)
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// ------------------------------------------------------------------ e4m3fn

// Round-to-nearest-even, saturating e4m3fn code of a finite fp32 value,
// computed on the integer bits so no floating-point rounding is involved.
__device__ __forceinline__ uint32_t e4m3_from_f32(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448: saturate
  int e = (int)(a >> 23);                      // biased fp32 exponent
  if (e < 121) {                               // |v| < 2^-6: e4m3 subnormal range, quantum 2^-9
    if (e == 0) return sign;                   // fp32 subnormal: far below 2^-10
    int sh = 141 - e;                          // |v| * 2^9 = m * 2^-sh, sh >= 21
    if (sh > 25) return sign;                  // < 2^-1 quanta: rounds to 0
    uint32_t m = (a & 0x7FFFFFu) | 0x800000u;
    uint32_t q = m >> sh, rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
    q += (rem > half) | ((rem == half) & (q & 1u));
    return sign | q;                           // q == 8 is the smallest normal, code 0x08
  }
  uint32_t m = a & 0x7FFFFFu;
  uint32_t q = ((uint32_t)(e - 120) << 3) | (m >> 20);
  uint32_t rem = m & 0xFFFFFu;
  q += (rem > 0x80000u) | ((rem == 0x80000u) & (q & 1u));  // never reaches 0x7F below 448
  return sign | q;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(__float_as_uint(mag) | s);
}

// e4m3 codes (bytes 0..3) of four finite fp32 values, by the hardware
// converter at scale 1 after a clamp to +-448: the same codes as
// e4m3_from_f32 (nearest, ties to even, saturating, sign kept).  Checked on
// MI355X over every bf16 value, every e4m3 rounding midpoint and its fp32
// neighbours and 2M random fp32 values (no mismatch); the bit-exact parity
// tests of the quantised activations and weights run through it.
__device__ __forceinline__ uint32_t e4m3x4_from_f32(float a, float b, float c, float d) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  auto sat = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
  v2s o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, sat(a), sat(b), 1.0f, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, sat(c), sat(d), 1.0f, true);
  return (uint32_t)(uint16_t)o[0] | ((uint32_t)(uint16_t)o[1] << 16);
}

// MX quantisation of four values of one block with scale exponent sx: the
// e4m3 codes of v * 2^-sx (returned, bytes 0..3) and the exact dequantised
// values code * 2^sx as 4 bf16 in `deq`.  sx = -127 (an all-zero or
// sub-2^-118 block, e8m0 byte 0) takes the integer path for the copy.
__device__ __forceinline__ uint32_t mx_encode4(float a, float b, float c, float d, int sx, uint2& deq) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t v = e4m3x4_from_f32(ldexpf(a, -sx), ldexpf(b, -sx), ldexpf(c, -sx), ldexpf(d, -sx));
  if (sx > -127) {
    const float sc = __uint_as_float((uint32_t)(sx + 127) << 23);  // 2^sx
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, sc, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, sc, true);
    __builtin_memcpy(&deq.x, &p0, 4);
    __builtin_memcpy(&deq.y, &p1, 4);
  } else {
    uint32_t dd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dd[j] = __float_as_uint(ldexpf(e4m3_to_f32((v >> (8 * j)) & 0xFFu), sx)) >> 16;
    deq = make_uint2(dd[0] | (dd[1] << 16), dd[2] | (dd[3] << 16));
  }
  return v;
}

// ------------------------------------------------------------------ e2m1

// e2m1 code of v relative to a positive scale sc: nearest of
// {0,.5,1,1.5,2,3,4,6} * sc, ties to the even code, saturating.  The
// midpoints times sc are exact in fp32 for the scales used here (an e4m3
// value, or 1), so the comparisons decide the code exactly.
__device__ __forceinline__ uint32_t e2m1_from_f32(float v, float sc) {
  float a = fabsf(v);
  uint32_t idx = 0;
  idx += (a > 0.25f * sc);
  idx += (a >= 0.75f * sc);   // tie 0.75: between codes 1 and 2 -> 2 (even)
  idx += (a > 1.25f * sc);    // tie 1.25: codes 2/3 -> 2
  idx += (a >= 1.75f * sc);   // tie 1.75: codes 3/4 -> 4
  idx += (a > 2.5f * sc);     // tie 2.5: codes 4/5 -> 4
  idx += (a >= 3.5f * sc);    // tie 3.5: codes 5/6 -> 6
  idx += (a > 5.0f * sc);     // tie 5: codes 6/7 -> 6
  return ((__float_as_uint(v) >> 28) & 8u) | idx;
}

// e2m1 code -> fp32 value (exact).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(mag | ((c & 8u) << 28));
}

// ------------------------------------------------------------------ MX scale

// floor(log2 a) - 8, clamped to [-127, 127], for a >= 0 (a = 0 -> -127).
// 8 is the exponent of e4m3's largest power of two (448 = 1.75 * 2^8).
__device__ __forceinline__ int mx_scale_exp(float amax) {
  uint32_t a = __float_as_uint(amax) & 0x7FFFFFFFu;
  int fl;
  if (a == 0) return -127;
  if (a >= 0x00800000u) fl = (int)(a >> 23) - 127;
  else fl = (31 - (int)__clz(a)) - 149;  // subnormal: value = a * 2^-149
  int s = fl - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_max_xor(float v, int mask_lo, int mask_hi) {
  for (int m = mask_lo; m <= mask_hi; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

}  // namespace moe
