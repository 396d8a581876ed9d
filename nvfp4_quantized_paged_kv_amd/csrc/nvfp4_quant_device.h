// NVFP4 quantization of one 16-value block for the gfx950 kernels: the exact
// rounding used by quantize-on-append (quant_append.hip) and by the decode
// step that appends its new tokens itself (decode_attn.hip), so both write
// the same bytes.  grer.cn blog "NVFP4 KV cache and the memory wall",
// section 2: 16 consecutive values share an E4M3 scale, the tensor an FP32
// scale, and a block's amax maps to the E2M1 maximum 6.
//
// Scale: bs = E4M3 nearest to amax/(6g), from a float64 quotient within
// about 2^-104 of the exact one (no such error can cross or land on an E4M3
// midpoint, and an exact midpoint comes out exactly).
// Codes, fast path: v_cvt_scalef32_pk_fp4_f32 (nearest E2M1, ties to even,
// saturating at 6) of |x| times c_lo and times c_hi, two float32 bounds of
// 1/(bs*g) (the float32 reciprocal scaled by 1 -/+ 2^-20); equal codes are
// the exact code, and an exact tie always makes them differ.  Codes, exact
// path (a block where any pair differs, or a zero scale): the magnitude is the
// number of float32 thresholds u_k the value exceeds, where u_k = RN(mid_k*bs*g)
// corrected by the sign of the exact FMA residual (ties count for odd k).
// Every file that includes this is compiled with -ffp-contract=off.
#pragma once

#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {

__device__ __forceinline__ float threshold_f32(float a, float g, bool odd) {
  const float hi = a * g;                      // rounded product (no contraction)
  const float lo = __builtin_fmaf(a, g, -hi);  // exact residual a*g - hi
  const float pred = __int_as_float(__float_as_int(hi) - 1);
  const bool down = odd ? (lo <= 0.0f) : (lo < 0.0f);
  return down ? pred : hi;
}

template <typename InT>
__device__ __forceinline__ void load_block(const InT* src, float (&x)[16]);

template <>
__device__ __forceinline__ void load_block<uint16_t>(const uint16_t* src, float (&x)[16]) {
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load_block<float>(const float* src, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

// Lane exchange within 32 lanes: the value of lane l ^ X (ds_swizzle, bitmask mode).
template <int X>
__device__ __forceinline__ double swz_xor(double v) {
  const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), (X << 10) | 0x1F);
  const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), (X << 10) | 0x1F);
  return __hiloint2double(hi, lo);
}

// One fast Walsh-Hadamard stage across lanes: this lane holds the elements
// whose index has bit `mine` (0 or 1) set at this stage, its partner lane l ^ X
// the others: (a, c) -> (a + c, a - c).
template <int X>
__device__ __forceinline__ void wht_cross(double* d, int n, bool mine) {
  for (int i = 0; i < n; ++i) {
    const double o = swz_xor<X>(d[i]);
    d[i] = mine ? o - d[i] : d[i] + o;
  }
}

// Fast Walsh-Hadamard stages over the N values one lane holds (index bits below log2 N).
template <int N>
__device__ __forceinline__ void wht_local(double (&d)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & h) == 0) {
        const double a = d[i], c = d[i + h];
        d[i] = a + c;
        d[i + h] = a - c;
      }
}

// Hadamard rotation of K before quantization (cloud.tencent.com.cn "NVFP4:
// breaking the memory wall of GPU inference", quantization tricks: an
// orthogonal transform spreads outliers over the vector): k' = H k * 2^-4 with
// H the 128-point Sylvester matrix, H[i][j] = (-1)^popcount(i & j).  A row is
// NB blocks of N values, block b in the lanes l ^ (4 * b) of one 32-lane
// group; the transform runs in float64 (every sum of 128 values with a
// 24-bit significand spanning at most 22 binades -- 38 for bf16 -- is exact)
// and is rounded to float32 once.
template <int N, int NB>
__device__ __forceinline__ void hadamard_rotate_k(float (&x)[N], int b) {
  double d[N];
#pragma unroll
  for (int i = 0; i < N; ++i) d[i] = (double)x[i];
  wht_local<N>(d);
  wht_cross<4>(d, N, (b & 1) != 0);
  wht_cross<8>(d, N, (b & 2) != 0);
  if (NB == 8) wht_cross<16>(d, N, (b & 4) != 0);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = (float)(d[i] * 0.0625);
}

// E4M3 scale byte of a block whose largest magnitude is amax: the E4M3 value
// nearest to amax/(6g).  r6 = 1/(6g) rounded to float64 (computed once per
// call by the caller).
__device__ __forceinline__ uint32_t block_scale_byte(float amax, float g, double r6) {
  // amax/(6g) without a division: q0 = amax*r6 is within 2^-52 (relative) of
  // the quotient, and one correction with the exact residual amax - q0*6g
  // (one fma; 6g is exact in float64) brings it within about 2^-104.  An
  // exact quotient that is an E4M3 midpoint (5 significant bits) then comes
  // out exactly, and any other quotient lies at least 2^-31 (relative) from
  // every midpoint (amax has 24 significant bits, 6*g*midpoint at most 31),
  // so the E4M3 rounding below sees the same side as for the exact quotient.
  const double a = (double)amax, g6 = 6.0 * (double)g;
  const double q0 = a * r6;
  return e4m3_encode_rne_sat(__builtin_fma(__builtin_fma(-q0, g6, a), r6, q0));
}

// Value k (lane-varying) of the 8 values x[8i .. 8i+7]: a select tree over the
// bits of k.  The values pass through an empty asm first, so the selects act
// on registers: selects between elements of x would otherwise be folded into
// an indexed load, which moves the whole array out of registers (into LDS or
// scratch memory) in every kernel that quantizes blocks.
template <int N>
__device__ __forceinline__ float pick8(const float (&x)[N], int i, int k) {
  float v0 = x[8 * i], v1 = x[8 * i + 1], v2 = x[8 * i + 2], v3 = x[8 * i + 3];
  float v4 = x[8 * i + 4], v5 = x[8 * i + 5], v6 = x[8 * i + 6], v7 = x[8 * i + 7];
  asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3), "+v"(v4), "+v"(v5), "+v"(v6), "+v"(v7));
  const float a0 = (k & 1) ? v1 : v0, a1 = (k & 1) ? v3 : v2, a2 = (k & 1) ? v5 : v4, a3 = (k & 1) ? v7 : v6;
  const float b0 = (k & 2) ? a1 : a0, b1 = (k & 2) ? a3 : a2;
  return (k & 4) ? b1 : b0;
}

// 4 * the midpoint between E2M1 magnitudes m and m + 1 (m = 0..6): 1, 3, 5, 7, 10, 14, 20.
__device__ __forceinline__ uint32_t e2m1_mid_x4(uint32_t m) {
  return __builtin_amdgcn_perm(0x00140E0Au, 0x07050301u, 0x0C0C0C00u | m);
}

// E2M1 codes of N values (N a multiple of 8) of a block with scale bs = E4M3
// value of its scale byte: packed[i] holds values 8i .. 8i+7, low nibble =
// even value.  Each value's code is decided on its own, so a block may be
// split over lanes.  Fast path: the two bracketing conversions; where they
// agree the code is exact.  Where they differ (the value lies within about
// 2^-20 of a rounding midpoint: common when g comes from bf16 data), the
// lower code's magnitude m or m + 1 is right, and the exact threshold between
// them decides (ties to the even magnitude).  Zero and extreme scales take the
// threshold path for every value.
template <int N>
__device__ __forceinline__ void encode_codes(const float (&x)[N], float bs, float g, uint32_t (&packed)[N / 8]) {
#pragma unroll
  for (int i = 0; i < N / 8; ++i) packed[i] = 0u;
  // the fast path needs bs*g (rounded) to be a normal float32 whose reciprocal
  // is normal too
  const float bsg = bs * g;
  if (bsg >= 0x1p-125f && bsg <= 0x1p125f) {
    // r is within 1 ulp (2^-23) of 1/bsg and bsg within 2^-24 of bs*g, so the
    // margins of 2^-20 keep c_lo below and c_hi above 1/(bs*g) by more than
    // 0.74 * 2^-20 after rounding
    const float r = __builtin_amdgcn_rcpf(bsg);
    const float c_lo = r * (1.0f - 0x1p-20f), c_hi = r * (1.0f + 0x1p-20f);
    uint32_t hi[N / 8];
#pragma unroll
    for (int i = 0; i < N / 8; ++i) hi[i] = 0u;
#pragma unroll
    for (int q = 0; q < N / 2; ++q) {
      switch (q & 3) {  // the byte select of the conversion is an immediate
        case 0:
          packed[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed[q >> 2], x[2 * q] * c_lo, x[2 * q + 1] * c_lo, 1.0f, 0);
          hi[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[q >> 2], x[2 * q] * c_hi, x[2 * q + 1] * c_hi, 1.0f, 0);
          break;
        case 1:
          packed[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed[q >> 2], x[2 * q] * c_lo, x[2 * q + 1] * c_lo, 1.0f, 1);
          hi[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[q >> 2], x[2 * q] * c_hi, x[2 * q + 1] * c_hi, 1.0f, 1);
          break;
        case 2:
          packed[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed[q >> 2], x[2 * q] * c_lo, x[2 * q + 1] * c_lo, 1.0f, 2);
          hi[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[q >> 2], x[2 * q] * c_hi, x[2 * q + 1] * c_hi, 1.0f, 2);
          break;
        default:
          packed[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed[q >> 2], x[2 * q] * c_lo, x[2 * q + 1] * c_lo, 1.0f, 3);
          hi[q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[q >> 2], x[2 * q] * c_hi, x[2 * q + 1] * c_hi, 1.0f, 3);
          break;
      }
    }
    // c_hi / c_lo < 1 + 2^-19, so the two products straddle at most one
    // midpoint: where the codes differ, hi's magnitude is lo's plus one (same sign)
    const float bs4 = 0.25f * bs;
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const uint32_t d = packed[i] ^ hi[i];
      uint32_t m = (d | (d >> 1) | (d >> 2) | (d >> 3)) & 0x11111111u;  // bit 4j: value 8i + j differs
      while (m != 0u) {
        const int pos = __builtin_ctz(m);
        m &= m - 1u;
        const uint32_t mag = (packed[i] >> pos) & 7u;
        // 4*mid and bs/4 have at most 5 and 4 significant bits: the product is exact
        const float u = threshold_f32((float)e2m1_mid_x4(mag) * bs4, g, (mag & 1u) != 0u);
        if (fabsf(pick8<N>(x, i, pos >> 2)) > u) packed[i] += 1u << pos;
      }
    }
    return;
  }
  float u[7];
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
  for (int k = 0; k < 7; ++k) u[k] = bs == 0.0f ? __builtin_inff() : threshold_f32(mids[k] * bs, g, (k & 1) != 0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float ax = fabsf(x[k]);
    const bool c2 = ax > u[3];
    const bool c1 = ax > (c2 ? u[5] : u[1]);
    const float t0 = c2 ? (c1 ? u[6] : u[4]) : (c1 ? u[2] : u[0]);
    const bool c0 = ax > t0;
    const uint32_t mag = (c2 ? 4u : 0u) | (c1 ? 2u : 0u) | (c0 ? 1u : 0u);
    const uint32_t code = mag | ((__float_as_uint(x[k]) >> 28) & 8u);
    packed[k >> 3] |= code << (4 * (k & 7));
  }
}

// One quantized block: 16 E2M1 codes (low nibble = even value) and the E4M3 scale byte.
struct QuantBlock {
  uint32_t packed[2];
  uint32_t sb;
};

// r6 = 1/(6g) rounded to float64 (computed once per call by the caller).
__device__ __forceinline__ QuantBlock quantize_block16(const float (&x)[16], float g, double r6) {
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));
  QuantBlock q;
  q.sb = block_scale_byte(amax, g, r6);
  encode_codes<16>(x, e4m3_value(q.sb), g, q.packed);
  return q;
}

// Store block b (dims 16b .. 16b+15) of the token in `slot` (>= 0, inside the
// cache) and kv head h into the K planes: K tiles are token-major (row o: 64
// code bytes, 8 scale bytes).
__device__ __forceinline__ void store_k_block(uint8_t* codes, uint8_t* scales, int H, int32_t slot, int h, int b,
                                              const QuantBlock& q) {
  const int64_t page = (uint32_t)slot / kPageSize;
  const int o = (int)((uint32_t)slot % kPageSize);
  const int64_t tile = page * H + h;
  *reinterpret_cast<uint2*>(codes + tile * kTileCodeBytes + o * 64 + 8 * b) = make_uint2(q.packed[0], q.packed[1]);
  scales[tile * kTileScaleBytes + o * 8 + b] = (uint8_t)q.sb;
}

// V tiles: lane r = d/8 of token quad o/4 owns bytes (o/4)*256 + r*16 .. +15,
// two 8-byte halves for the slot pairs (o/4)*4 + {0,1} and + {2,3}; a half is
// an even-dimension word then an odd-dimension word, and byte c of a word
// holds dimension 8r + 2c (+1 in the odd word) of the pair's even slot in its
// low nibble and of the odd slot in its high nibble.  The decode's PV operand
// is then a plain conversion of those bytes.  Scale byte b*16 + o.
//
// Block b covers lanes 2b and 2b+1.  The words of lane 2b + k for a slot pair
// from the pair's packed code words k (even slot e, odd slot f):
__device__ __forceinline__ uint2 v_pair_words(uint32_t e, uint32_t f) {
  return make_uint2((e & 0x0F0F0F0Fu) | ((f << 4) & 0xF0F0F0F0u), ((e >> 4) & 0x0F0F0F0Fu) | (f & 0xF0F0F0F0u));
}

__device__ __forceinline__ uint8_t* v_half(uint8_t* codes, int H, int32_t slot, int h, int r) {
  const int64_t page = (uint32_t)slot / kPageSize;
  const int o = (int)((uint32_t)slot % kPageSize);
  return codes + (page * H + h) * kTileCodeBytes + (o >> 2) * 256 + r * 16 + ((o >> 1) & 1) * 8;
}

// Both slots of a pair are written in this call by two lanes: the lane of slot
// parity k writes lane 2b + k's half of the pair from its own packed word k
// and the partner's (`other` = the partner's packed word k), and the even
// slot's lane writes both scale bytes (`other_sb` = the partner's).
__device__ __forceinline__ void store_v_pair(uint8_t* codes, uint8_t* scales, int H, int32_t slot, int h, int b,
                                             const QuantBlock& q, uint32_t other, uint32_t other_sb) {
  const int k = slot & 1;
  const uint32_t mine = k ? q.packed[1] : q.packed[0];
  *reinterpret_cast<uint2*>(v_half(codes, H, slot, h, 2 * b + k)) = k ? v_pair_words(other, mine) : v_pair_words(mine, other);
  if (k == 0) {
    const int64_t page = (uint32_t)slot / kPageSize;
    const int o = (int)((uint32_t)slot % kPageSize);
    *reinterpret_cast<uint16_t*>(scales + (page * H + h) * kTileScaleBytes + b * 16 + o) =
        (uint16_t)(q.sb | (other_sb << 8));
  }
}

// A slot written without its pair partner: only this slot's nibbles change,
// by an atomic AND then OR on each of its two 8-byte halves (the partner's
// nibbles may be written by another lane of the same call).
__device__ __forceinline__ void store_v_alone(uint8_t* codes, uint8_t* scales, int H, int32_t slot, int h, int b,
                                              const QuantBlock& q) {
  const bool odd = slot & 1;
  const uint64_t keep = odd ? 0x0F0F0F0F0F0F0F0Full : 0xF0F0F0F0F0F0F0F0ull;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint2 w = odd ? v_pair_words(0u, q.packed[k]) : v_pair_words(q.packed[k], 0u);
    uint64_t* at = reinterpret_cast<uint64_t*>(v_half(codes, H, slot, h, 2 * b + k));
    __hip_atomic_fetch_and(at, keep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(at, (uint64_t)w.x | ((uint64_t)w.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int64_t page = (uint32_t)slot / kPageSize;
  const int o = (int)((uint32_t)slot % kPageSize);
  scales[(page * H + h) * kTileScaleBytes + b * 16 + o] = (uint8_t)q.sb;
}

// Lane exchange with lane l ^ 1 (ds_swizzle, bitmask mode); every lane of the
// 32-lane group must be active.
__device__ __forceinline__ uint32_t swz_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (1 << 10) | 0x1F);
}

}  // namespace nvfp4kv
