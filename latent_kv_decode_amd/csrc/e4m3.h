// e4m3.h -- OCP 8-bit float E4M3 codes on gfx950: decoding to bfloat16 and
// rounding float32 values to codes.
//
// Every E4M3 value (normal or subnormal) is exact in bf16, so the scaled
// packed conversion with scale 1 (two codes to two bf16 per instruction; OCP
// E4M3 on gfx950: bias 7, no infinities, S.1111.111 NaN) gives the values
// exactly.
#pragma once

#include <hip/hip_runtime.h>

namespace lkv {

typedef unsigned e4m3_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned e4m3_u32x4;

// Four codes (one 32-bit word, code 0 in the low byte) to four bf16 values in
// two words (value 0 in the low half of word 0).
__device__ __forceinline__ e4m3_u32x2 e4m3x4_to_bf16x4(unsigned word) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
  const b2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
  return e4m3_u32x2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
}

// Eight codes to eight bf16 values (16 bytes).
__device__ __forceinline__ e4m3_u32x4 e4m3x8_to_bf16x8_bits(unsigned w0, unsigned w1) {
  const e4m3_u32x2 a = e4m3x4_to_bf16x4(w0), b = e4m3x4_to_bf16x4(w1);
  return e4m3_u32x4{a[0], a[1], b[0], b[1]};
}

// Nearest OCP E4M3 code of a float32 value (ties to the even code;
// magnitudes past 448, infinities included, saturate to 448; NaN gives the
// NaN code S.1111.111 with the value's sign bit).  Normal results: the
// mantissa rounded to 3 bits by integer rounding of the float32 bits (a carry
// moves the exponent); below 2^-6: the nearest multiple of 2^-9, whose code is
// that multiple (8 lands on 2^-6, code 8).
__device__ __forceinline__ unsigned e4m3_encode(float x) {
  const unsigned sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);  // NaN -> 448 here; replaced below
  const unsigned b = __float_as_uint(a);
  // normal: bits rounded at mantissa bit 20; the biased exponent 120 + e
  // and the 3 mantissa bits then read as code ((e + 7) << 3 | m)
  const unsigned normal = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 960u;
  const unsigned sub = static_cast<unsigned>(rintf(a * 512.f));
  const unsigned code = (a < 0x1p-6f ? sub : normal) | sign;
  return __builtin_isnan(x) ? (0x7Fu | sign) : code;
}

}  // namespace lkv
