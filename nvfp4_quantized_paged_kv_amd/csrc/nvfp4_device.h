// Device-side format helpers for the gfx950 kernels.
//
// E4M3 here is OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
// subnormals m * 2^-9, largest finite 448, no infinities (grer.cn blog "NVFP4
// KV cache and the memory wall", section 2: the per-16 block scale is FP8
// E4M3).  E2M1 is 1 sign, 2 exponent, 1 mantissa bit (cloud.tencent.com.cn
// "NVFP4: breaking the memory wall of GPU inference", E2M1 encoding section).
//
// Every file that includes this is compiled with -ffp-contract=off: the exact
// rounding decisions below rely on products being rounded where written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Nearest E4M3 byte to r >= 0 (r finite or +inf): ties to the even mantissa,
// saturating at 448 (0x7E), values at or below 2^-10 round to 0.
// Scaling by powers of two and rint (round-half-even) are exact in float64.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(double r) {
  if (!(r < 448.0)) return 0x7Eu;
  if (r < 0x1p-6) return (uint32_t)__builtin_rint(r * 512.0);  // subnormal grid m * 2^-9; m == 8 is 2^-6
  int e;
  (void)__builtin_frexp(r, &e);                                    // r = f * 2^e, f in [0.5, 1)
  const int E = e - 1;                                             // floor(log2 r), -6..8
  const uint32_t m = (uint32_t)__builtin_rint(__builtin_ldexp(r, 3 - E));  // 8..16
  return (uint32_t)((E + 7) << 3) + m - 8u;                        // m == 16 carries into the exponent
}

// Exact float value of an E4M3 byte without its sign bit (b < 0x80; 0x7F
// reads as 480): the f16 bit pattern b << 7 holds the value times 2^-8,
// subnormals included (see below).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b << 7)) * 256.0f;
}

// Two E4M3 bytes (each < 0x80) to packed f16 holding value * 2^-8: the f16 bit
// pattern byte << 7 puts the E4M3 exponent field on the f16 exponent field
// (bias 15 vs 7) and its mantissa on the top mantissa bits; E4M3 subnormals
// land on f16 subnormals with the same factor.
__device__ __forceinline__ half2_t e4m3_pair_to_f16_scaled(uint32_t b0, uint32_t b1) {
  return __builtin_bit_cast(half2_t, (b0 << 7) | (b1 << 23));
}

// FP4 (E2M1) byte `sel` of `w` -> two f16 values (low nibble -> element 0),
// each multiplied by 2^8 (the hardware applies the power-of-two part of the
// f32 scale operand; the product is exact: |e2m1| * 256 <= 1536).
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_f16_x256(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, SEL);
}

// The same without the factor: the two E2M1 values exactly.
template <int SEL>
__device__ __forceinline__ half2_t fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

}  // namespace nvfp4kv
