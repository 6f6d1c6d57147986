// fp8 e4m3 and e8m0 helpers of the activation quantisation, shared by the
// quantisation kernels, the GEMM epilogues and the router's fused
// quantisation at decode (every producer of a quantised activation rounds
// the same way).
#pragma once

#include "common.h"

namespace moe {

// e4m3 (OCP) of v, v already within [-448, 448]; round to nearest even
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
  return (uint32_t)hi;
}
__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Power-of-two scale >= v (v > 0) as its e8m0 code; 127 (2^0) for v == 0.
__device__ __forceinline__ uint32_t e8m0_at_least(float v) {
  if (!(v > 0.f)) return 127u;
  const uint32_t u = __float_as_uint(v);
  uint32_t e = (u >> 23) & 0xFFu;
  if (e == 0u) return 1u;                 // below the normal range: smallest code used
  if ((u & 0x7FFFFFu) != 0u) e += 1u;     // not a power of two: round up
  return e > 254u ? 254u : e;
}
__device__ __forceinline__ float e8m0_value(uint32_t code) { return __uint_as_float(code << 23); }
__device__ __forceinline__ float e8m0_inv(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// Scale of one activation group from its amax: FP8 (128 values) an fp32
// scale amax / 448 (1 for an all-zero group), MX (32 values) the e8m0 code
// of pow2_at_least(amax / 448), both quotients in fp32.  A value then
// becomes v / scale in fp32, clamped to +-448 and rounded to e4m3 (ties to
// even).  FP8 divides (correctly rounded): multiplying by an fp32 1 / scale
// instead moves values that sit exactly on an e4m3 rounding tie (frequent
// for bf16 inputs) to one side of it.  MX multiplies by e8m0_inv(code), an
// exact power of two, which is the same value.
__device__ __forceinline__ float fp8_group_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }
// MX code without the division: for amax = 1.m x 2^(E-127) with E in
// [10, 254], the fp32 quotient amax / 448 (448 = 1.75 x 2^8) rounds to at
// most 2^e exactly when amax <= 448 x 2^e (the rounding boundary above
// 448 x 2^e lies below the next fp32 value), so the code is E - 8, plus one
// when m > 1.75 (mantissa field above 0x600000).  Other exponents (tiny or
// non-finite amax) take the quotient.
__device__ __forceinline__ uint32_t mx_group_code(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const uint32_t E = (u >> 23) & 0xFFu;
  if (E >= 10u && E <= 254u) return E - 8u + (((u & 0x7FFFFFu) > 0x600000u) ? 1u : 0u);
  return e8m0_at_least(amax / 448.f);
}
__device__ __forceinline__ float fp8_scaled(float v, float scale) { return clamp448(v / scale); }

}  // namespace moe
