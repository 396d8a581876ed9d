// NVFP4 pages -> FP8 E4M3 workspace, for the extend / chunked-prefill path on
// gfx950.
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, second data
// flow: the cached prefix of an extend request is dequantized into one FP8
// workspace pair that every layer overwrites (not one per layer);
// nmedialink.com "NVIDIA NVFP4: LLM memory doubled, inference 3x", Fig. 3:
// NVFP4 values are dequantized to FP8 before the attention that reads them.
//
// Work: a workgroup (4 waves) takes 64 consecutive (page, kv head) tiles of one
// sequence and one tensor; a wave moves a whole tile per step with 16-byte
// loads (1 KB of codes, 64 lanes) and writes 128-byte workspace rows.
// All values of a block share its scale byte, so every output byte is one of
// 8 magnitudes (times the code's sign) fixed by that byte: the workgroup first
// builds the 256-entry table scale byte -> 8 E4M3 bytes in LDS (one entry per
// thread), then each code nibble is mapped through its block's entry with
// byte permutes (v_perm_b32).
//
// Exactness of the table.  y = e2m1 * bs * g / s_ws.  The numerator is exact in
// float64 (at most 30 significant bits) and a float64 quotient is correctly
// rounded; an E4M3 midpoint times s_ws has at most 29 significant bits, so no
// float64 rounding crosses or lands on a midpoint and rounding the quotient
// gives the E4M3 value nearest the exact y.  Only magnitudes 0.5 and 1.5 need a
// division: the others are those two times 2, 4 or 8, and scaling a float64 by
// a power of two is exact.
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

constexpr int kWsWaves = 4;
constexpr int kWsTilesPerWave = 16;
constexpr int kWsTilesPerGroup = kWsWaves * kWsTilesPerWave;

__global__ __launch_bounds__(kWsWaves * 64) void dequant_ws_kernel(DequantWsParams p) {
  __shared__ uint2 s_lut[256];  // scale byte -> E4M3 bytes for magnitude codes 0..3 (x) and 4..7 (y)
  const int which = blockIdx.z;  // 0 = K, 1 = V
  const int seq = blockIdx.y;
  const int prefix = min(p.prefix_lens[seq], p.max_prefix_len);
  const int64_t tiles = (int64_t)((prefix + kPageSize - 1) / kPageSize) * p.H;
  const int64_t tile0 = (int64_t)blockIdx.x * kWsTilesPerGroup;
  if (tile0 >= tiles) return;

  {  // this thread's table entry: E4M3 bytes of |e2m1_m| * bs * g / s_ws, m = 0..7
    const double num = (double)e4m3_value(threadIdx.x & 0x7Fu) * (double)p.g[which];  // exact: 4 + 24 bits; sign bit ignored
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
    s_lut[threadIdx.x] = make_uint2((m1 << 8) | (m2 << 16) | (m3 << 24), m4 | (m5 << 8) | (m6 << 16) | (m7 << 24));
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t out0 = p.ws_offsets[seq];
  const uint8_t* codes = p.codes[which];
  const uint8_t* scales = p.scales[which];
  uint8_t* ws = p.ws[which];
  struct Tile {
    uint4 c;
    uint32_t sc;
    int pg, h;
    bool ok;
  };
  auto fetch = [&](int i) {
    Tile t;
    const int64_t tile = tile0 + (int64_t)i * kWsWaves + wave;  // consecutive tiles: heads of one page
    t.ok = tile < tiles;
    const int64_t tl = t.ok ? tile : 0;
    t.pg = (int)(tl / p.H);
    t.h = (int)(tl % p.H);
    const int page = p.block_table[(int64_t)seq * p.bt_stride + t.pg];
    t.ok = t.ok && (unsigned)page < (unsigned)p.num_pages;
    const int64_t tb = t.ok ? (int64_t)page * p.H + t.h : 0;
    t.c = *reinterpret_cast<const uint4*>(codes + tb * kTileCodeBytes + lane * 16);
    t.sc = which == 0 ? (uint32_t)*reinterpret_cast<const uint16_t*>(scales + tb * kTileScaleBytes + (lane >> 2) * 8 +
                                                                      2 * (lane & 3))
                      : *reinterpret_cast<const uint32_t*>(scales + tb * kTileScaleBytes + (lane & 15) / 2 * 16 +
                                                           4 * (lane >> 4));
    return t;
  };
  auto put = [&](const Tile& t) {
    if (!t.ok) return;
    if (which == 0) {
      // K tile, token-major: lane = (token o, dims 32q .. 32q+31), blocks 2q and 2q+1
      const int o = lane >> 2, q = lane & 3;
      const int64_t row = out0 + (int64_t)t.pg * kPageSize + o;
      if (t.pg * kPageSize + o < prefix && row >= 0 && row < p.ws_capacity) {
        const uint2 l0 = s_lut[t.sc & 0xFFu], l1 = s_lut[t.sc >> 8];
        const uint2 a = map_nibbles(t.c.x, l0.x, l0.y), b = map_nibbles(t.c.y, l0.x, l0.y);
        const uint2 d = map_nibbles(t.c.z, l1.x, l1.y), e = map_nibbles(t.c.w, l1.x, l1.y);
        uint4* dst = reinterpret_cast<uint4*>(ws + (row * p.H + t.h) * kHeadDim + 32 * q);
        dst[0] = make_uint4(a.x, a.y, b.x, b.y);
        dst[1] = make_uint4(d.x, d.y, e.x, e.y);
      }
    } else {
      // V tile: lane = (tokens 4*(lane/16) .. +3, dims 8*(lane%16) .. +7) as even- and
      // odd-dimension words of the token pairs (0, 1) and (2, 3) (a byte holds one
      // dimension of both tokens); regrouped here into one code dword per token
      const int o0 = 4 * (lane >> 4), d0 = 8 * (lane & 15);
      const uint32_t cw[4] = {(t.c.x & 0x0F0F0F0Fu) | ((t.c.y << 4) & 0xF0F0F0F0u),
                              ((t.c.x >> 4) & 0x0F0F0F0Fu) | (t.c.y & 0xF0F0F0F0u),
                              (t.c.z & 0x0F0F0F0Fu) | ((t.c.w << 4) & 0xF0F0F0F0u),
                              ((t.c.z >> 4) & 0x0F0F0F0Fu) | (t.c.w & 0xF0F0F0F0u)};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t row = out0 + (int64_t)t.pg * kPageSize + o0 + k;
        if (t.pg * kPageSize + o0 + k < prefix && row >= 0 && row < p.ws_capacity) {
          const uint2 l = s_lut[(t.sc >> (8 * k)) & 0xFFu];
          *reinterpret_cast<uint2*>(ws + (row * p.H + t.h) * kHeadDim + d0) = map_nibbles(cw[k], l.x, l.y);
        }
      }
    }
  };
  // two register sets of four tiles, each consumed in place: the next set's
  // loads are issued before the current set is written (fetch past the last
  // tile reads tile 0 and put skips it)
  Tile a0 = fetch(0), a1 = fetch(1), a2 = fetch(2), a3 = fetch(3);
  for (int i = 0; i < kWsTilesPerWave; i += 8) {
    if (tile0 + (int64_t)i * kWsWaves + wave >= tiles) break;
    const Tile b0 = fetch(i + 4), b1 = fetch(i + 5), b2 = fetch(i + 6), b3 = fetch(i + 7);
    put(a0);
    put(a1);
    put(a2);
    put(a3);
    if (tile0 + (int64_t)(i + 4) * kWsWaves + wave >= tiles) break;
    if (i + 8 < kWsTilesPerWave) {
      a0 = fetch(i + 8);
      a1 = fetch(i + 9);
      a2 = fetch(i + 10);
      a3 = fetch(i + 11);
    }
    put(b0);
    put(b1);
    put(b2);
    put(b3);
  }
}

}  // namespace

hipError_t launch_dequant_ws(const DequantWsParams& p, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.max_prefix_len + kPageSize - 1) / kPageSize) * p.H;
  if (tiles == 0 || p.num_seqs == 0) return hipSuccess;
  const dim3 grid((unsigned)((tiles + kWsTilesPerGroup - 1) / kWsTilesPerGroup), (unsigned)p.num_seqs, 2);
  hipLaunchKernelGGL(dequant_ws_kernel, grid, dim3(kWsWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
