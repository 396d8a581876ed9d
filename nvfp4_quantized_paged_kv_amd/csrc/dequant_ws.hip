// NVFP4 pages -> FP8 E4M3 workspace, for the extend / chunked-prefill path on
// gfx950.
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, second data
// flow: the cached prefix of an extend request is dequantized into one FP8
// workspace pair that every layer overwrites (not one per layer);
// nmedialink.com "NVIDIA NVFP4: LLM memory doubled, inference 3x", Fig. 3:
// NVFP4 values are dequantized to FP8 before the attention that reads them.
//
// One thread owns one 16-value block of one (token, kv head) of one tensor.
// All 16 values share the block scale, so the block has only 8 possible output
// magnitudes: the thread computes those 8 E4M3 bytes exactly, then maps each
// code nibble through them with byte permutes (v_perm_b32) and writes 16 bytes.
//
// Exactness.  y = e2m1 * bs * g / s_ws.  The numerator is exact in float64
// (at most 30 significant bits) and a float64 quotient is correctly rounded;
// an E4M3 midpoint times s_ws has at most 29 significant bits, so no float64
// rounding crosses or lands on a midpoint and rounding the quotient gives the
// E4M3 value nearest the exact y.  Only magnitudes 0.5 and 1.5 need a
// division: the others are those two times 2, 4 or 8, and scaling a float64
// by a power of two is exact.
#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

// 8 code nibbles (one dword, low nibble first) -> 8 E4M3 bytes via the
// magnitude table (lut_lo = bytes for magnitudes 0..3, lut_hi = 4..7).
__device__ __forceinline__ uint2 map_nibbles(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  const uint32_t ev = __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  const uint32_t od = __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  // interleave: out bytes = ev0 od0 ev1 od1 | ev2 od2 ev3 od3  (perm: 0..3 = second operand, 4..7 = first)
  const uint32_t lo = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(od, ev, 0x07030602u);
  return make_uint2(lo, hi);
}

__global__ __launch_bounds__(256) void dequant_ws_kernel(DequantWsParams p) {
  const int which = blockIdx.z;  // 0 = K, 1 = V
  const int seq = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = (int)(i & 7);
  const int64_t row = i >> 3;
  const int h = (int)(row % p.H);
  const int64_t t = row / p.H;
  const int prefix = min(p.prefix_lens[seq], p.max_prefix_len);
  if (t >= prefix) return;
  const int64_t out_row = (int64_t)p.ws_offsets[seq] + t;
  if (out_row < 0 || out_row >= p.ws_capacity) return;
  const int page = p.block_table[(int64_t)seq * p.bt_stride + t / kPageSize];
  if ((unsigned)page >= (unsigned)p.num_pages) return;
  const int o = (int)(t % kPageSize);
  const int64_t tile = (int64_t)page * p.H + h;

  uint32_t w0, w1, sb;
  if (which == 0) {
    const uint2 c = *reinterpret_cast<const uint2*>(p.codes[0] + tile * kTileCodeBytes + o * 64 + 8 * b);
    w0 = c.x;
    w1 = c.y;
    sb = p.scales[0][tile * kTileScaleBytes + o * 8 + b];
  } else {
    const uint8_t* base = p.codes[1] + tile * kTileCodeBytes + (o >> 2) * 256 + (o & 3) * 4;
    w0 = *reinterpret_cast<const uint32_t*>(base + (2 * b) * 16);
    w1 = *reinterpret_cast<const uint32_t*>(base + (2 * b + 1) * 16);
    sb = p.scales[1][tile * kTileScaleBytes + b * 16 + o];
  }

  // E4M3 bytes of |e2m1_m| * bs * g / s_ws for the 8 magnitude codes.
  const double num = (double)e4m3_value(sb) * (double)p.g[which];  // exact: 4 + 24 bits
  const double ws = (double)p.ws_scale[which];
  const double y05 = (num * 0.5) / ws;
  const double y15 = (num * 1.5) / ws;
  const uint32_t m1 = e4m3_encode_rne_sat(y05);
  const uint32_t m2 = e4m3_encode_rne_sat(y05 * 2.0);
  const uint32_t m3 = e4m3_encode_rne_sat(y15);
  const uint32_t m4 = e4m3_encode_rne_sat(y05 * 4.0);
  const uint32_t m5 = e4m3_encode_rne_sat(y15 * 2.0);
  const uint32_t m6 = e4m3_encode_rne_sat(y05 * 8.0);
  const uint32_t m7 = e4m3_encode_rne_sat(y15 * 4.0);
  const uint32_t lut_lo = (m1 << 8) | (m2 << 16) | (m3 << 24);
  const uint32_t lut_hi = m4 | (m5 << 8) | (m6 << 16) | (m7 << 24);

  const uint2 a = map_nibbles(w0, lut_lo, lut_hi);
  const uint2 c = map_nibbles(w1, lut_lo, lut_hi);
  *reinterpret_cast<uint4*>(p.ws[which] + (out_row * p.H + h) * kHeadDim + 16 * b) = make_uint4(a.x, a.y, c.x, c.y);
}

}  // namespace

hipError_t launch_dequant_ws(const DequantWsParams& p, hipStream_t stream) {
  const int64_t per_seq = (int64_t)p.max_prefix_len * p.H * 8;
  if (per_seq == 0 || p.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)((per_seq + 255) / 256), (unsigned)p.num_seqs, 2);
  hipLaunchKernelGGL(dequant_ws_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
