// MXFP4 quantize-on-append for gfx950: the 4-bit format NVFP4 is compared
// against (nmedialink.com "NVIDIA NVFP4: LLM memory doubled, inference 3x",
// accuracy section and Fig. 6; cloud.tencent.com.cn "NVFP4: breaking the
// memory wall of GPU inference", E2M1 encoding and two-level scaling section:
// one scale per 32 values).  The scale is the OCP MX v1.0 one: a power of two
// stored as an E8M0 byte, X = 2^(floor(log2 amax) - 2) (2 = exponent of the
// E2M1 maximum 6), clamped to 2^-127 .. 2^127; no tensor-wide scale.
//
// One thread owns one 32-value block of one (token, kv head): lane order,
// fastest first, is token within a group of 4, block, group of 4 within 16
// consecutive tokens, kv head, group of 16 tokens, so one wave writes a whole
// (page, kv head) tile when the tokens fill a page.
//
// Exactness: for a finite float amax with exponent field E, floor(log2 amax)
// is E - 127 (E >= 1), so the scale byte is max(E - 2, 0).  |x| * 2^(127 -
// byte) is then exact (a power of two, result below 8), and the E2M1 code is
// found by comparisons against the exact midpoints, ties to the even code.
#include <type_traits>

#include "nvfp4_quant_device.h"

namespace nvfp4kv {
namespace {

template <typename InT>
__device__ __forceinline__ void load_block32(const InT* src, float (&x)[32]);

template <>
__device__ __forceinline__ void load_block32<uint16_t>(const uint16_t* src, float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 a = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ __forceinline__ void load_block32<float>(const float* src, float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

// E2M1 magnitude code of y >= 0 (y exact): nearest of 0, .5, 1, 1.5, 2, 3, 4, 6,
// ties to the even code, everything from 5 up saturating at 6.  A tie between
// codes k and k+1 goes up when k is odd, hence >= at the midpoints 0.75, 1.75
// and 3.5 and > at 0.25, 1.25, 2.5 and 5.
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
  const bool c2 = y >= 1.75f;
  const bool c1 = c2 ? y >= 3.5f : y >= 0.75f;
  const float t0 = c2 ? (c1 ? 5.0f : 2.5f) : (c1 ? 1.25f : 0.25f);
  const bool c0 = y > t0;
  return (c2 ? 4u : 0u) | (c1 ? 2u : 0u) | (c0 ? 1u : 0u);
}

struct MxTensor {
  const void* x;
  uint8_t* codes;
  uint8_t* scales;
};

// kRotK: K rows are Hadamard-rotated before quantization (the 4 blocks of a
// row sit in lanes l, l^4, l^8, l^12; lanes without a token hold token 0 and
// take part in the exchanges, then skip the store).
template <typename InT, bool kRotK>
__global__ __launch_bounds__(256) void mx_append_kernel(MxTensor k, MxTensor v, const int32_t* slots,
                                                        int64_t token_stride, int32_t num_tokens, int32_t H,
                                                        int32_t num_pages, int64_t n_threads) {
  const MxTensor& T = blockIdx.y ? v : k;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_threads) return;  // n_threads is a multiple of 64: whole waves leave together
  const int tq = (int)(i & 3), b = (int)((i >> 2) & 3), tg = (int)((i >> 4) & 3);
  const uint32_t gh = (uint32_t)(i >> 6);  // group of 16 tokens * H + kv head (< 2^31, checked by the host)
  const int h = (int)(gh % (uint32_t)H);
  const int64_t t = 16 * (int64_t)(gh / (uint32_t)H) + 4 * tg + tq;
  const int32_t slot = t < num_tokens ? slots[t] : -1;
  const bool store = slot >= 0 && (int64_t)slot < (int64_t)num_pages * kPageSize;

  float x[32];
  load_block32<InT>(reinterpret_cast<const InT*>(T.x) + (store ? t : 0) * token_stride + (int64_t)h * kHeadDim + 32 * b,
                    x);
  if (kRotK && blockIdx.y == 0) hadamard_rotate_k<32, 4>(x, b);
  if (!store) return;
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
  const int E = (int)(__float_as_uint(amax) >> 23);  // exponent field (amax >= 0, finite)
  const uint32_t sb = (uint32_t)max(E - 2, 0);
  const float inv = __uint_as_float((254u - sb) << 23);  // 2^(127 - sb), a normal float for sb <= 252
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t code = e2m1_mag(fabsf(x[j]) * inv) | ((__float_as_uint(x[j]) >> 28) & 8u);
    packed[j >> 3] |= code << (4 * (j & 7));
  }

  const int64_t page = (uint32_t)slot / kPageSize;
  const int o = (int)((uint32_t)slot % kPageSize);
  const int64_t tile = page * H + h;
  if (blockIdx.y == 0) {  // K: token-major rows, scale byte o*4 + b
    *reinterpret_cast<uint4*>(T.codes + tile * kTileCodeBytes + o * 64 + 16 * b) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    T.scales[tile * kMxTileScaleBytes + o * 4 + b] = (uint8_t)sb;
  } else {  // V: 8-dim words of 4 tokens interleaved, scale byte b*16 + o
    uint8_t* base = T.codes + tile * kTileCodeBytes + (o >> 2) * 256 + (o & 3) * 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<uint32_t*>(base + (4 * b + w) * 16) = packed[w];
    T.scales[tile * kMxTileScaleBytes + b * 16 + o] = (uint8_t)sb;
  }
}

}  // namespace

hipError_t launch_mx_append(const MxAppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream) {
  const int64_t n_threads = (int64_t)((p.num_tokens + 15) / 16) * 16 * p.H * 4;  // tokens rounded up to groups of 16
  if (n_threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_threads + 255) / 256), 2, 1);
  const MxTensor k{p.x[0], p.codes[0], p.scales[0]}, v{p.x[1], p.codes[1], p.scales[1]};
  auto go = [&](auto rot) {
    constexpr bool R = decltype(rot)::value;
    if (dtype == NVFP4_DTYPE_BF16)
      hipLaunchKernelGGL((mx_append_kernel<uint16_t, R>), grid, dim3(256), 0, stream, k, v, p.slots, p.token_stride,
                         p.num_tokens, p.H, p.num_pages, n_threads);
    else
      hipLaunchKernelGGL((mx_append_kernel<float, R>), grid, dim3(256), 0, stream, k, v, p.slots, p.token_stride,
                         p.num_tokens, p.H, p.num_pages, n_threads);
  };
  if (p.rot_k) go(std::true_type{}); else go(std::false_type{});
  return hipGetLastError();
}

}  // namespace nvfp4kv
