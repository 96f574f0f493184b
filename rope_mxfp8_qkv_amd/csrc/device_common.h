// Device-side helpers of the gfx950 kernels: bf16 and E4M3 conversions written from the
// formats' bit layouts.  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkvmx {

// bf16 bits -> fp32 (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (low half = a), round to nearest, ties to even: one
// V_CVT_PK_BF16_F32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// fp32 -> FP8 E4M3 ("fn": max 448, no infinities), round to nearest even, saturating at +-448.
// The sign bit is kept, so negative values that round to zero give 0x80.
//  - |v| < 2^-6 lies on the subnormal grid of step 2^-9: code = rint(|v| * 2^9) (0..8; 8 is the
//    smallest normal, 0x08, so the carry into the exponent field is automatic).
//  - otherwise round the fp32 mantissa to 3 bits (RNE on the bit pattern) and rebias the
//    exponent from 127 to 7; a mantissa carry moves into the exponent field by itself.
// Both candidates are computed and one is selected, so the conversion is branch-free.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t sub = (uint32_t)rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t nrm = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return (a < 0.015625f ? sub : nrm) | sign;
}

// Four E4M3 codes (round to nearest even, saturating at +-448, sign kept) packed little-endian
// (byte i = code of the i-th argument), by the hardware's packing conversion after a clamp to
// [-448, 448] (the conversion itself does not saturate).  Equal to f32_to_e4m3 on every finite
// fp32 input: qkvmx_e4m3_convert_check compares the two on all 2^32 bit patterns.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return (uint32_t)w;
}

}  // namespace qkvmx
