// mxfp4 (E2M1 elements, E8M0 group scale) -> bf16, exact (gfx950). Shared
// by the paged gather and the sparse attention that reads the same cache.
//
// An E2M1 magnitude is 0.5, or (1 + m/2) * 2^(e-1), so times 2^(b-127) it is
// a bf16 with biased exponent e-1+b (b-1 for code 1) and one mantissa bit;
// the only non-normal outcomes are the two subnormal exponents (b <= 1) and
// overflow to inf (exponent >= 255). No rounding ever happens. Scale bytes
// 2..252 use gfx950's scaled fp4->bf16 convert; the rest build the bit
// pattern with integer ops. E8M0 0xFF means 0 here (the cache's rule).
#pragma once

#include "xk_internal.h"

namespace xk {

__device__ __forceinline__ uint32_t e2m1_e8m0_to_bf16(uint32_t code, uint32_t scale) {
  const uint32_t sign = (code & 8u) << 12;
  const uint32_t mag = code & 7u;
  if (mag == 0u || scale == 0xFFu) return sign;  // +-0 * s, or x * 0
  const bool normal_code = mag >= 2u;            // codes 2..7: e >= 1
  const int biased = normal_code ? int(mag >> 1) - 1 + int(scale) : int(scale) - 1;
  const uint32_t mant = normal_code ? (mag & 1u) : 0u;
  if (biased >= 255) return sign | 0x7F80u;                       // overflow -> inf
  if (biased >= 1) return sign | (uint32_t(biased) << 7) | (mant << 6);
  // biased in {-1, 0}: subnormal, value (2 + mant) * 2^(biased-128) = field * 2^-133
  return sign | ((2u + mant) << (biased + 5));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Eight E2M1 elements (one dword, element 2i in the low nibble of byte i)
// times one E8M0 scale byte -> eight bf16 (element 2i in the low half of
// dword i). For scale bytes 2..252 every product is a normal bf16 and exact,
// so the hardware scaled convert (2 elements per instruction, exact in that
// range) is used; extreme bytes take the integer construction above.
__device__ __forceinline__ u32x4 decode8(uint32_t nib, uint32_t sc) {
  u32x4 v;
  if (sc >= 2u && sc <= 252u) {
    const float scale = __uint_as_float(sc << 23);  // 2^(sc-127), a normal float
    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, scale, 0));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, scale, 1));
    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, scale, 2));
    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, scale, 3));
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (nib >> (8 * b)) & 0xFFu;
      v[b] = e2m1_e8m0_to_bf16(byte & 0xFu, sc) | (e2m1_e8m0_to_bf16(byte >> 4, sc) << 16);
    }
  }
  return v;
}

}  // namespace xk
