// NVFP4 quantize-on-append for gfx950.
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 2 (two-level
// scaling: 16 consecutive values share an E4M3 scale, the tensor shares an FP32
// scale, each block's amax maps to the E2M1 maximum 6) and section 3 (new K/V
// are quantized to NVFP4 when written to the cache); nmedialink.com "NVIDIA
// NVFP4: LLM memory doubled, inference 3x", Fig. 3 (quantize before append).
//
// One thread owns one 16-value block of one (token, kv head): it reads the 16
// inputs (32 B bf16 / 64 B f32), so the block's amax needs no cross-lane work,
// and writes 8 code bytes plus 1 scale byte.  Lane order, fastest first: token
// within a group of 4, block, group of 4 within 16 consecutive tokens, kv head,
// group of 16 tokens.  Sixteen consecutive tokens usually fill one page, so a
// 256-lane workgroup writes whole (page, kv head) tiles of two heads: its K and
// V code runs and its 128-B scale rows are complete lines written by one CU.
//
// Exact rounding.  bs = E4M3 nearest to amax/(6g): the float64 quotient of the
// float32 amax and the exact float64 6g is correctly rounded, and no float64
// rounding can cross or land on an E4M3 midpoint (a midpoint times 6g has at
// most 31 significant bits, amax 24), so rounding that quotient is exact.
// Codes: the E2M1 magnitude of x is the number of midpoints T_k = mid_k*bs*g
// (mid = 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) that |x| passes, where passing
// an exact tie counts only when it rounds to the even code (k odd).  Each T_k
// is turned into a float32 threshold u_k with "|x| passes T_k <=> |x| > u_k"
// exactly: a_k = mid_k*bs is exact in float32 (7 significant bits),
// hi = RN(a_k*g) and lo = fma(a_k, g, -hi) is the exact residual, so
//   k even: u_k = lo < 0  ? pred(hi) : hi      (|x| > T_k)
//   k odd : u_k = lo <= 0 ? pred(hi) : hi      (|x| >= T_k)
// (global scales are restricted to [2^-100, 2^100], which keeps a_k*g in the
// float32 normal range).  The magnitude then follows from three comparisons
// (binary search over the 7 thresholds).
//
// Fast path.  The hardware conversion v_cvt_scalef32_pk_fp4_f32 rounds a
// float32 to the nearest E2M1 code, ties to the even code, saturating at 6.
// With c_lo < 1/(bs*g) < c_hi (float64 reciprocal scaled by 1 -/+ 2^-21, then
// rounded to float32), the float32 products satisfy |x|*c_lo < |x|/(bs*g) <
// |x|*c_hi even after their own rounding.  The code is a nondecreasing step
// function of the magnitude, so if both products give the same code, that is
// the code of the exact |x|/(bs*g).  An exact tie lies strictly between the
// two products and makes their codes differ.  A block where any of the 16
// pairs differ takes the threshold path above instead (rare: a value within
// about 2^-21 of a rounding boundary).
#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

__device__ __forceinline__ float threshold_f32(float a, float g, bool odd) {
  const float hi = a * g;                      // rounded product (no contraction in this file)
  const float lo = __builtin_fmaf(a, g, -hi);  // exact residual a*g - hi
  const float pred = __int_as_float(__float_as_int(hi) - 1);
  const bool down = odd ? (lo <= 0.0f) : (lo < 0.0f);
  return down ? pred : hi;
}

// Values 2Q and 2Q+1, times c_lo and times c_hi, to E2M1 codes in byte Q%4 of
// word Q/4 of lo and hi (low nibble = value 2Q).
template <int Q>
__device__ __forceinline__ void cvt_pair(uint32_t (&lo)[2], uint32_t (&hi)[2], const float (&x)[16], float c_lo,
                                         float c_hi) {
  lo[Q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo[Q >> 2], x[2 * Q] * c_lo, x[2 * Q + 1] * c_lo, 1.0f, Q & 3);
  hi[Q >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi[Q >> 2], x[2 * Q] * c_hi, x[2 * Q + 1] * c_hi, 1.0f, Q & 3);
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

// Quantize one 16-value block x and store its codes and scale byte at `slot`.
__device__ __forceinline__ void quantize_store(const float (&x)[16], const AppendTensor& T, const AppendParams& p,
                                               int which, int32_t slot, int h, int b) {
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(x[k]));

  const float g = T.g;
  const uint32_t sb = e4m3_encode_rne_sat((double)amax / (6.0 * (double)g));
  const float bs = e4m3_value(sb);

  uint32_t packed[2] = {0u, 0u};
  bool exact_path = bs == 0.0f;  // zero scale: every code is its sign (threshold path, thresholds +inf)
  if (!exact_path) {
    const double rcp = 1.0 / ((double)bs * (double)g);  // bs*g exact in float64
    const float c_lo = (float)(rcp * (1.0 - 0x1p-21)), c_hi = (float)(rcp * (1.0 + 0x1p-21));
    uint32_t hi[2] = {0u, 0u};
    cvt_pair<0>(packed, hi, x, c_lo, c_hi);
    cvt_pair<1>(packed, hi, x, c_lo, c_hi);
    cvt_pair<2>(packed, hi, x, c_lo, c_hi);
    cvt_pair<3>(packed, hi, x, c_lo, c_hi);
    cvt_pair<4>(packed, hi, x, c_lo, c_hi);
    cvt_pair<5>(packed, hi, x, c_lo, c_hi);
    cvt_pair<6>(packed, hi, x, c_lo, c_hi);
    cvt_pair<7>(packed, hi, x, c_lo, c_hi);
    exact_path = (packed[0] != hi[0]) | (packed[1] != hi[1]);
  }
  if (exact_path) {
    float u[7];
    const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
#pragma unroll
    for (int k = 0; k < 7; ++k) u[k] = bs == 0.0f ? __builtin_inff() : threshold_f32(mids[k] * bs, g, (k & 1) != 0);
    packed[0] = packed[1] = 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
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

  const int64_t page = (uint32_t)slot / kPageSize;  // slot >= 0 here
  const int o = (int)((uint32_t)slot % kPageSize);
  const int64_t tile = page * p.H + h;
  if (which == 0) {
    *reinterpret_cast<uint2*>(T.codes + tile * kTileCodeBytes + o * 64 + 8 * b) = make_uint2(packed[0], packed[1]);
    T.scales[tile * kTileScaleBytes + o * 8 + b] = (uint8_t)sb;
  } else {
    uint8_t* base = T.codes + tile * kTileCodeBytes + (o >> 2) * 256 + (o & 3) * 4;
    *reinterpret_cast<uint32_t*>(base + (2 * b) * 16) = packed[0];
    *reinterpret_cast<uint32_t*>(base + (2 * b + 1) * 16) = packed[1];
    T.scales[tile * kTileScaleBytes + b * 16 + o] = (uint8_t)sb;
  }
}

// Block index i of the flattened work -> (token t, kv head h, block b); t < 0 if past the end.
__device__ __forceinline__ void block_coords(int64_t i, const AppendParams& p, int64_t& t, int& h, int& b) {
  const int tq = (int)(i & 3), tg = (int)((i >> 5) & 3);
  b = (int)((i >> 2) & 7);
  const uint32_t gh = (uint32_t)(i >> 7);  // group of 16 tokens * H + kv head (< 2^31, checked by the host)
  h = (int)(gh % (uint32_t)p.H);
  t = 16 * (int64_t)(gh / (uint32_t)p.H) + 4 * tg + tq;
  if (t >= p.num_tokens) t = -1;
}

// Each thread takes R blocks, n_threads apart in the flattened order (so every
// pass keeps the page-tile lane pattern); all of their loads are issued before
// any of them is quantized.  R = 2 for bulk appends (more bytes in flight per
// wave), R = 1 for small ones, where the per-thread chain is the latency.
template <typename InT, int R>
__global__ __launch_bounds__(256) void quantize_append_kernel(AppendParams p, int64_t n_threads) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const AppendTensor& T = p.t[which];
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i0 >= n_threads) return;
  float x[R][16];
  int32_t slot[R];
  int h[R], b[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    int64_t t;
    block_coords(i0 + k * n_threads, p, t, h[k], b[k]);
    slot[k] = t >= 0 ? p.slots[t] : -1;
    if (slot[k] < 0 || (int64_t)slot[k] >= (int64_t)p.num_pages * kPageSize) {
      slot[k] = -1;
      t = 0;  // load token 0 (in range) and skip the store
    }
    load_block<InT>(reinterpret_cast<const InT*>(T.x) + t * p.token_stride + (int64_t)h[k] * kHeadDim + 16 * b[k], x[k]);
  }
#pragma unroll
  for (int k = 0; k < R; ++k)
    if (slot[k] >= 0) quantize_store(x[k], T, p, which, slot[k], h[k], b[k]);
}

// blocks (16 values of one token and head) from which an append counts as bulk
constexpr int64_t kAppendBulkBlocks = 1 << 18;

}  // namespace

hipError_t launch_quantize_append(const AppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream) {
  const int64_t n_blocks = (int64_t)((p.num_tokens + 15) / 16) * 16 * p.H * 8;  // tokens rounded up to groups of 16
  if (n_blocks == 0) return hipSuccess;
  // threads per pass, a multiple of 128 (one 16-token group of one head) so
  // every pass starts on a group boundary
  const bool bulk = n_blocks >= kAppendBulkBlocks;
  const int r = bulk ? 2 : 1;
  const int64_t n_threads = (n_blocks / 128 + r - 1) / r * 128;
  const dim3 grid((unsigned)((n_threads + 255) / 256), 2, 1);
  const bool bf16 = dtype == NVFP4_DTYPE_BF16;
  if (bf16 && bulk)
    hipLaunchKernelGGL((quantize_append_kernel<uint16_t, 2>), grid, dim3(256), 0, stream, p, n_threads);
  else if (bf16)
    hipLaunchKernelGGL((quantize_append_kernel<uint16_t, 1>), grid, dim3(256), 0, stream, p, n_threads);
  else if (bulk)
    hipLaunchKernelGGL((quantize_append_kernel<float, 2>), grid, dim3(256), 0, stream, p, n_threads);
  else
    hipLaunchKernelGGL((quantize_append_kernel<float, 1>), grid, dim3(256), 0, stream, p, n_threads);
  return hipGetLastError();
}

}  // namespace nvfp4kv
