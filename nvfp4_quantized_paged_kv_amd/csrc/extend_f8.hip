// Extend / prefill attention over the FP8 workspace in FP8 arithmetic, on
// gfx950's 32x32x64 FP8 MFMA.
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, first and
// second data flows: a chunked prefill / extend attends over its cached
// prefix from the FP8 workspace and over its own FP8 K/V.  The K and V bytes
// enter the MFMA as they are (no widening); so do Q and the softmax weights,
// each rounded to E4M3:
//   - Q row (query token, query head) times the base-2 logit scale c =
//     float32(sm_scale * k_ws_scale * log2 e), one float32 product per value:
//     codes E4M3(q c 2^-E), E the smallest integer with max|q c| <= 448 * 2^E
//     (an exact power-of-two scale; rounding to nearest, ties to even);
//   - logits x_t = 2^E sum_d Q8_d K8_td (fp32 accumulation in the MFMA);
//   - weights W8_t = E4M3(2^(x_t - m + 8)), m an integer >= every logit so
//     far (the ceiling of the running maximum: rescales are exact powers of
//     two), so every weight lies in (0, 256]; for |m| >= 2^27, where float32
//     cannot hold m - 8 exactly, 2^(x_t - m) instead;
//   - out = v_ws_scale * sum_t W8_t V8_t / sum_t W8_t, the row sum taken by
//     one more MFMA against E4M3 ones, so the output is a convex combination
//     of V rows with exactly the weights used.
// The per-element error of E4M3 (2^-4 relative) makes this a lower-precision
// contract than the f16 extend kernel's; the oracle states both.
//
// Work split as in the f16 kernel: one workgroup per (16 chunk tokens, kv
// head, sequence [, key share]); wave w owns query heads 2w, 2w+1 x 16 tokens
// = the 32 rows of a 32x32 MFMA block.  64-key K / V tiles are staged in LDS
// (double-buffered) by the first 256 threads.  Lane l (row r = l % 32, half
// hh = l / 32):
//   S^T block (32 keys x 32 rows) = K tile rows . Q^T: A = K (key r, dims
//   64c + 32hh .. +31), B = Q (row r, same dims); the result gives lane l the
//   scores of row r for keys 32kb + 8(i/4) + 4hh + i%4, i < 16, kb < 2.
//   PV: A = W8 of those 32 keys (row r; byte 16kb + i <-> that key), B = V^T
//   row (dim 32db + r) at the same 32 keys, which the loader writes to V^T
//   byte 32hh + 16kb + 4(i/4) + i%4.  The result gives lane l dim 32db + r of
//   rows 8(i/4) + 4hh + i%4.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kF8Tok = 16;                            // chunk tokens per workgroup
constexpr int kF8Keys = 64;                           // keys per LDS tile
constexpr int kF8KStride = 144;                       // LDS bytes per K row: 128 + 16 pad (b128 reads conflict-free)
constexpr int kF8VStride = 72;                        // LDS bytes per V^T row: 64 keys + 8 pad
constexpr int kF8KTile = kF8Keys * kF8KStride;
constexpr int kF8VTile = kHeadDim * kF8VStride;
constexpr int kF8BufferFlags = 0x00020000;            // gfx9 buffer resource word 3 for raw dword access
constexpr float kF8Headroom = 8.0f;                   // weights are E4M3 of 2^(x - m + 8) <= 256
constexpr int kF8One = 0x38383838;                    // four E4M3 ones

__device__ __forceinline__ v16f_t mfma_f8(v8i_t a, v8i_t b, v16f_t c) {
  // E4M3 x E4M3 (format codes 0, 0); unit E8M0 block scales (127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// max of x over lanes l and l ^ 32 (the two halves that hold one row's keys)
__device__ __forceinline__ float max_halves(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// four floats -> four E4M3 bytes (round to nearest, ties to even).  The
// first conversion writes the low half of a's register (its high half is
// replaced by the second), so no register has to be cleared first.
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ v8i_t lds_b256(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  return v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
__device__ __forceinline__ v8i_t lds_b256_8(const uint8_t* p) {  // 8-byte aligned rows
  const uint2 a = *reinterpret_cast<const uint2*>(p), b = *reinterpret_cast<const uint2*>(p + 8);
  const uint2 c = *reinterpret_cast<const uint2*>(p + 16), d = *reinterpret_cast<const uint2*>(p + 24);
  return v8i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, (int)d.x, (int)d.y};
}

template <bool QF32>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void extend_f8_kernel(ExtendParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kF8KTile];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kF8VTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, hh = lane >> 5;
  const int seq = blockIdx.z, h = blockIdx.y;
  // blockIdx.x = tile-from-the-end * splits + split: the tiles with the most keys start first
  const int S = p.splits;
  const int split = (int)(blockIdx.x % (uint32_t)S);
  const int tile = (int)(gridDim.x / (uint32_t)S) - 1 - (int)(blockIdx.x / (uint32_t)S);
  const int G = p.G, H = p.H;

  // ---- the sequence (device data is clamped, never trusted)
  const int nq = p.num_q_tokens;
  const int q0 = min(max(__builtin_amdgcn_readfirstlane(p.q_offsets[seq]), 0), nq);
  const int q1 = min(max(__builtin_amdgcn_readfirstlane(p.q_offsets[seq + 1]), q0), nq);
  const int C = min(q1 - q0, p.max_chunk);
  const int t0 = tile * kF8Tok;
  if (t0 >= C) return;
  const int ntok = min(kF8Tok, C - t0);
  const int P = min(max(__builtin_amdgcn_readfirstlane(p.prefix_lens[seq]), 0), p.ws_capacity);
  const int64_t woff = __builtin_amdgcn_readfirstlane(p.ws_offsets[seq]);
  const int n_keys = P + t0 + ntok;  // keys the tile's last token sees
  const int n_all = P + t0 + 1;      // keys every token of the tile sees
  const int n_kt = (n_keys + kF8Keys - 1) / kF8Keys;
  // this workgroup's key tiles [kt0, kt1): an equal share (possibly empty)
  const int kt0 = (int)((int64_t)split * n_kt / S), kt1 = (int)((int64_t)(split + 1) * n_kt / S);

  // ---- tile loads by threads tid < 256, through a per-tile descriptor over the
  // sequence's valid rows (rows past them, or past the workspace, read as 0).
  // K: key tid/4, 32 bytes at dims 32 * (tid % 4).
  // V: the 4 keys 32kb + 8g + 4hh' + (0..3) at dims 4vd .. 4vd+3, for kb = 0, 1
  // (two passes), g = (tid >> 3) & 3, hh' = tid >> 7, vd = (tid & 7) + 8 *
  // ((tid >> 5) & 3); a 4x4 byte transpose gives each of the 4 dims' rows the
  // 4 keys as one word at V^T byte 32hh' + 16kb + 4g.  In a 32-lane half of a
  // store the rows 4vd + e (stride 18 words) and the 4 g-words land on 32
  // distinct banks.
  const bool loader = tid < 256;
  const int row_bytes = H * kHeadDim;
  const int64_t valid_rows =
      (woff >= 0 && woff < p.ws_capacity) ? min((int64_t)n_keys, (int64_t)p.ws_capacity - woff) : 0;
  const int kk = tid >> 2, kc = tid & 3;
  const int vgq = (tid >> 3) & 3, vhh = (tid >> 7) & 1, vd = (tid & 7) + 8 * ((tid >> 5) & 3);
  const int ko = (kk * H + h) * kHeadDim + 32 * kc;
  int vo[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) vo[kb][j] = ((32 * kb + 8 * vgq + 4 * vhh + j) * H + h) * kHeadDim + 4 * vd;
  auto tile_rsrc = [&](const uint8_t* base, int kt) {
    const int64_t r0 = (int64_t)kt * kF8Keys;
    const int64_t rows = max((int64_t)0, min((int64_t)kF8Keys, valid_rows - r0));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + (woff + r0) * row_bytes, 0,
                                             (int)(rows * row_bytes), kF8BufferFlags);
  };
  uint4 kreg[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  uint32_t vreg[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  auto load_tile = [&](int kt) {
    if (!loader) return;
    const auto rk = tile_rsrc(p.ws_k, kt);
    const auto rv = tile_rsrc(p.ws_v, kt);
    kreg[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0));
    kreg[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16, 0, 0));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) vreg[kb][j] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo[kb][j], 0, 0);
  };
  auto store_tile = [&](int buf) {
    if (!loader) return;
    uint8_t* kp = &s_k[buf][kk * kF8KStride + 32 * kc];
    *reinterpret_cast<uint4*>(kp) = kreg[0];
    *reinterpret_cast<uint4*>(kp + 16) = kreg[1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t* w = vreg[kb];
      // 4x4 byte transpose: t[e] = dim 4vd + e of the 4 keys
      const uint32_t a_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
      const uint32_t a_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
      const uint32_t b_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
      const uint32_t b_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
      const uint32_t t[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u), __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                             __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u), __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
      uint8_t* vt = &s_v[buf][(4 * vd) * kF8VStride + 32 * vhh + 16 * kb + 4 * vgq];
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vt + e * kF8VStride) = t[e];
    }
  };
  if (kt0 < kt1) load_tile(kt0);

  // ---- Q of this lane's row: query head g, token tq; dims 64c + 32hh .. +31
  const bool active = 2 * wave < G;
  const int g = 2 * wave + (r >> 4), tq = r & 15;
  v8i_t qb[2];
  float tscale;
  {
    float qv[64];
#pragma unroll
    for (int k = 0; k < 64; ++k) qv[k] = 0.0f;
    if (active && g < G && tq < ntok) {
      const int64_t qoff = ((int64_t)(q0 + t0 + tq) * p.Hq + (int64_t)h * G + g) * kHeadDim + 32 * hh;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (QF32) {
          const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.q) + qoff + 64 * c);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint4 w = qp[k];
            qv[32 * c + 4 * k] = __uint_as_float(w.x);
            qv[32 * c + 4 * k + 1] = __uint_as_float(w.y);
            qv[32 * c + 4 * k + 2] = __uint_as_float(w.z);
            qv[32 * c + 4 * k + 3] = __uint_as_float(w.w);
          }
        } else {
          const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) + qoff + 64 * c);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint4 w = qp[k];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              qv[32 * c + 8 * k + 2 * j] = __uint_as_float(ww[j] << 16);
              qv[32 * c + 8 * k + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
            }
          }
        }
      }
    }
    // the logit scale goes on Q before the rounding (one float32 product per
    // value): the logits are then 2^E times the MFMA's sums, exactly
    float qmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      qv[k] *= p.qk_scale_log2;
      qmax = fmaxf(qmax, __builtin_fabsf(qv[k]));
    }
    qmax = max_halves(qmax);
    // E: the smallest integer with qmax <= 448 * 2^E (qmax = f 2^e, f in [0.5, 1); 448 = 0.875 * 2^9)
    int e = 0;
    const float f = __builtin_frexpf(qmax, &e);
    const int E = qmax > 0.0f ? (f <= 0.875f ? e - 9 : e - 8) : 0;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __builtin_ldexpf(qv[32 * c + 4 * w + j], -E);  // exact: |x| <= 448
        qb[c][w] = pack_e4m3(x[0], x[1], x[2], x[3]);
      }
    tscale = __builtin_ldexpf(1.0f, E);  // exact (a subnormal or 0 only for logits below 2^-117)
  }

  // running integer maximum (log2 domain) of this lane's row; -1e30 (an
  // integer-valued float): none yet, every weight relative to it is 0
  float m_run = -1.0e30f;
  v16f_t acc[4], lsum;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[d][i] = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) lsum[i] = 0.0f;
  v8i_t ones = {kF8One, kF8One, kF8One, kF8One, kF8One, kF8One, kF8One, kF8One};
  asm volatile("" : "+v"(ones));  // kept in registers, not rebuilt every tile
  const int lim = P + t0 + tq;  // last key of this lane's row

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    store_tile(buf);
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);  // in flight while this tile is computed
    if (!active) continue;

    // ---- S^T = K . Q^T for the tile's two 32-key blocks
    v16f_t Sb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Sb[kb][i] = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        Sb[kb] = mfma_f8(lds_b256(&s_k[buf][(32 * kb + r) * kF8KStride + 64 * c + 32 * hh]), qb[c], Sb[kb]);
    }
    // explicit wait states between the MFMA results and their first VALU reads
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(Sb[0]), "+v"(Sb[1]));

    // ---- causal mask: only tiles reaching past the keys every token sees
    const int kbase = kt * kF8Keys;
    if (kbase + kF8Keys > n_all) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kbase + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3) > lim) Sb[kb][i] = -__builtin_inff();
    }

    // ---- the row maximum moves (to the next integer at or above it) only
    // when a score passes the current one
    float lm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) lm = fmaxf(lm, Sb[kb][i]);
    const float pm = max_halves(lm) * tscale;  // exact
    if (__any(pm > m_run)) {
      const float m_new = fmaxf(m_run, __builtin_ceilf(pm));
      const float f = __builtin_amdgcn_exp2f(m_run - m_new);  // a power of two (or 0), exact
      // the accumulators hold rows 8(i/4) + 4hh + i%4: their factors come from those rows' lanes
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float fi = __shfl(f, 8 * (i >> 2) + 4 * hh + (i & 3));
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d][i] *= fi;
        lsum[i] *= fi;
      }
      m_run = m_new;
    }
    // m - 8 is exact below 2^27 (the float32 spacing there is at most 8);
    // above it m - 8 could round down by 16, so the headroom is dropped there
    const float msub = __builtin_fabsf(m_run) < 134217728.0f ? m_run - kF8Headroom : m_run;

    // ---- weights: E4M3 of 2^(x - m + 8), x = score * 2^E exact, one rounding in
    // the fused multiply-add (x <= m, so the argument is at most 8)
    v8i_t w8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sb[kb][4 * w + j], tscale, -msub));
        w8[4 * kb + w] = pack_e4m3(x[0], x[1], x[2], x[3]);
      }

    // ---- O += W8 . V and the row sums
#pragma unroll
    for (int db = 0; db < 4; ++db)
      acc[db] = mfma_f8(w8, lds_b256_8(&s_v[buf][(32 * db + r) * kF8VStride + 32 * hh]), acc[db]);
    lsum = mfma_f8(w8, ones, lsum);
  }
  if (!active) return;
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(lsum));

  // ---- lane holds dim 32db + r of rows 8(i/4) + 4hh + i%4
  if (S > 1) {
    // a share of the keys: the unnormalised partial, its maximum and sum (merged by the extend merge kernel)
    auto part_row = [&](int row) {
      const int gg = 2 * wave + (row >> 4), tt = row & 15;
      return p.part + (((int64_t)split * nq + q0 + t0 + tt) * p.Hq + (int64_t)h * G + gg) * kExtPartStride;
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * hh + (i & 3);
      if (2 * wave + (row >> 4) >= G || (row & 15) >= ntok) continue;
      float* pp = part_row(row);
#pragma unroll
      for (int db = 0; db < 4; ++db) pp[32 * db + r] = acc[db][i];
      if (r == 0) pp[kHeadDim + 1] = lsum[i];
    }
    if (hh == 0 && g < G && tq < ntok) part_row(r)[kHeadDim] = m_run;
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i >> 2) + 4 * hh + (i & 3);
    const int gg = 2 * wave + (row >> 4), tt = row & 15;
    if (gg >= G || tt >= ntok) continue;
    float* op = p.out + ((int64_t)(q0 + t0 + tt) * p.Hq + (int64_t)h * G + gg) * kHeadDim + r;
    const float fs = lsum[i] > 0.0f ? p.v_scale / lsum[i] : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) op[32 * db] = acc[db][i] * fs;
  }
}

}  // namespace

ExtendGeometry extend_f8_geometry(int32_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                  int32_t max_chunk, int32_t max_prefix) {
  ExtendGeometry geo{1, 0};
  if (num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_seqs <= 0 || max_chunk <= 0 || max_prefix < 0)
    return geo;
  // as for the f16 kernel: split a tile's keys only when the tiles fill at
  // most half a round of resident workgroups (2 waves per SIMD: two 4-wave
  // workgroups per CU, or one 8-wave one), filling one round with shares of
  // at least kExtMinShareKeys keys
  const int32_t G = num_q_heads / num_kv_heads;
  const int64_t round = 256 * (G > 8 ? 1 : 2);
  const int64_t tiles = (int64_t)((max_chunk + kF8Tok - 1) / kF8Tok) * num_kv_heads * num_seqs;
  const int64_t keys = (int64_t)max_prefix + max_chunk;
  int64_t s = round / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(keys / kExtMinShareKeys, 1));
  s = std::min<int64_t>(s, kExtMaxSplits);
  if (s <= 1) return geo;
  geo.splits = (int32_t)s;
  const size_t bytes = (size_t)s * (size_t)num_q_tokens * (size_t)num_q_heads * kExtPartStride * sizeof(float);
  geo.workspace_bytes = (bytes + 255) / 256 * 256;
  return geo;
}

hipError_t launch_extend_f8(const ExtendParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_chunk == 0 || p.num_q_tokens == 0) return hipSuccess;
  if (p.splits < 1 || p.splits > kExtMaxSplits) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((p.max_chunk + kF8Tok - 1) / kF8Tok * p.splits), (unsigned)p.H, (unsigned)p.num_seqs);
  const dim3 block(p.G <= 8 ? 256 : 512);  // at least 256 threads: the tile loaders
  if (q_dtype == NVFP4_DTYPE_F32)
    hipLaunchKernelGGL(extend_f8_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(extend_f8_kernel<false>, grid, block, 0, stream, p);
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_extend_merge(p, stream);
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
