// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Round an fp32 value to bf16 (nearest, ties to even). Inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Eight 4-bit codes u (packed so that code 2p sits in bits [4p, 4p+4) and
// code 2p+1 in bits [16+4p, 16+4p+4)) become eight bf16 values 128 + u:
// OR-ing a code into the mantissa of bf16 128.0 (0x4300, ulp 1) is exact.
// Since q = u - 8, each value equals q + 136; the 136 * sum(x) excess is
// removed by the caller. The mask and the exponent bits are held in
// registers (gfx9 VOP3 encodings take no literal), so each output dword is
// one v_and_or_b32: the empty asm statements only hide the constants' values
// from the optimiser (which would otherwise fold them back into literals);
// they emit no instruction, so every register write stays visible to the
// compiler's hazard checks (an instruction written in inline asm is not).
__device__ __forceinline__ bf16x8_t dequant_u4_plus128(uint32_t w) {
  uint32_t m = 0xf000fu, c = 0x43004300u;
  asm("" : "+s"(m));
  asm("" : "+v"(c));
  const uint32_t p0 = (w & m) | c;
  const uint32_t p1 = ((w >> 4) & m) | c;
  const uint32_t p2 = ((w >> 8) & m) | c;
  const uint32_t p3 = ((w >> 12) & m) | c;
  return __builtin_bit_cast(bf16x8_t, make_uint4(p0, p1, p2, p3));
}

// Eight FP4 e2m1 codes (byte b holds codes 2b, 2b+1, low nibble first)
// become eight bf16 values code * 2^e, where e is the exponent field of
// `scale` (gfx950's conversion uses only the scale's exponent bits; an E8M0
// byte shifted into them gives exactly 2^(byte - 127), byte 0 included).
// Exact whenever the product is a bf16 value.
__device__ __forceinline__ bf16x8_t dequant_fp4(uint32_t w, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// D(16x16, fp32) = A(16x32) * B(32x16) + C on the bf16 matrix cores.
// Lane l supplies A row (l % 16) and B column (l % 16), each with the 8
// consecutive K values 8*(l/16) .. 8*(l/16)+7; it receives D rows
// 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace moe
