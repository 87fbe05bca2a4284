// e4m3.h -- OCP 8-bit float E4M3 codes to bfloat16 on gfx950.
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

}  // namespace lkv
