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
// The block quantizer (exact E4M3 scale, E2M1 codes by the hardware
// conversion with an exact threshold fallback) is in nvfp4_quant_device.h,
// shared with the decode step that appends its own new tokens.
#include <type_traits>

#include "nvfp4_quant_device.h"

namespace nvfp4kv {
namespace {

// Quantize one 16-value block x and store its codes and scale byte at `slot`.
__device__ __forceinline__ void quantize_store(const float (&x)[16], const AppendTensor& T, const AppendParams& p,
                                               int which, int32_t slot, int h, int b) {
  store_block(T.codes, T.scales, p.H, which != 0, slot, h, b, quantize_block16(x, T.g));
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
// kRotK: K rows are Hadamard-rotated before quantization (the 8 blocks of a
// row sit in lanes l, l^4, .., l^28, so every lane of a 32-lane group takes
// part in the exchanges; idle lanes hold token 0 and skip the store).
template <typename InT, int R, bool kRotK>
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
  if (kRotK && which == 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) hadamard_rotate_k<16, 8>(x[k], b[k]);
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
  auto go = [&](auto rot) {
    constexpr bool K = decltype(rot)::value;
    if (bf16 && bulk)
      hipLaunchKernelGGL((quantize_append_kernel<uint16_t, 2, K>), grid, dim3(256), 0, stream, p, n_threads);
    else if (bf16)
      hipLaunchKernelGGL((quantize_append_kernel<uint16_t, 1, K>), grid, dim3(256), 0, stream, p, n_threads);
    else if (bulk)
      hipLaunchKernelGGL((quantize_append_kernel<float, 2, K>), grid, dim3(256), 0, stream, p, n_threads);
    else
      hipLaunchKernelGGL((quantize_append_kernel<float, 1, K>), grid, dim3(256), 0, stream, p, n_threads);
  };
  if (p.rot_k) go(std::true_type{}); else go(std::false_type{});
  return hipGetLastError();
}

}  // namespace nvfp4kv
