// Split-K paged decode attention over an NVFP4 cache, dequantizing in
// registers, for gfx950 (CDNA4, wave64, MFMA).
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, third data
// flow: decode reads the whole cache for one short query, so its speed is set
// by the cache read; the 4-bit values are widened where they are loaded and the
// block scale is applied in registers, with no separate dequantization pass.
// Section 1 of the same blog: grouped-query heads share one KV head.
//
// Work decomposition.  A workgroup (kWaves waves) owns one (sequence, kv head,
// split of `pages_per_split` pages); wave w takes pages w, w+kWaves, ... of the
// split.  The page indices of a wave's pages sit one per lane (64 at a time)
// and are read with readlane, and the next page's K/V bytes are loaded before
// the current page is computed.  Per page (16 tokens):
//   QK^T  S[16 tok x 16 q] = K_page[16 x 128] . Q^T : 4 x mfma_f32_16x16x32_f16
//         (A = K: lane (tok = l%16, k-group l/16) loads 16 contiguous code bytes =
//          dims 32*(l/16)..+31 of its token; B = Q, the same dims, in registers)
//   online softmax in fp32 (exp2 domain), with a lazy max: the running max is
//         only raised when a page exceeds it by more than 2^8, so P <= 2^8;
//         row maxima across the 4 token groups use v_permlane16/32_swap
//   PV    O[16 q x 128] += P[16 x 16 tok] . V_page : 8 x mfma_f32_16x16x16_f16
//         (the QK^T output lane layout is exactly the PV A-operand layout; the V
//          tile layout gives lane l the 4 tokens 4*(l/16)..+3 of dims
//          8*(l%16)..+7 in 16 contiguous bytes; nibbles of two tokens are
//          re-paired with bit-field inserts so that one byte = one MFMA k-pair)
// Dequantization: v_cvt_scalef32_pk_f16_fp4 widens two E2M1 codes (times 2^8),
// and one v_pk_mul_f16 by (E4M3 scale * 2^-8, taken from the scale byte's bit
// pattern) gives e2m1 * bs exactly in f16 (at most 6 significant bits,
// magnitude in [2^-10, 2688]).  The FP32 global scales are applied to the
// logits (K) and to the final output (V).  Q is converted to f16 after an
// exact power-of-two prescale (float32 Q: as an f16 hi + lo pair).
// The waves of a workgroup merge their (max, sum, O) in LDS.  A sequence whose
// pages fit in one split is finished there (normalised output); otherwise the
// split writes a partial and a second kernel merges the splits.
#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

#ifndef NVFP4_DECODE_WAVES
#define NVFP4_DECODE_WAVES 16
#endif
#ifndef NVFP4_DECODE_TARGET_GROUPS
#define NVFP4_DECODE_TARGET_GROUPS 256
#endif
// One 16-wave workgroup fills a CU (4 waves per SIMD at <= 128 VGPRs), and
// about one workgroup per CU covers the call, so a batch with at least as many
// (sequence, kv head) units as CUs runs without splitting a sequence.
constexpr int kWaves = NVFP4_DECODE_WAVES;                     // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int64_t kTargetGroups = NVFP4_DECODE_TARGET_GROUPS;  // workgroups per call
constexpr int kMaxPagesPerWave = 128;                          // page indices a wave keeps in 2 lane registers
constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max must move

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

// Cross-lane max/sum over lanes l, l^16, l^32, l^48 (the 4 token groups of one
// query head) with the gfx950 row/half swaps: with both operands equal,
// permlane16_swap returns (row 2k, row 2k+1) values and permlane32_swap the
// (low half, high half) values.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <bool QF32>
__device__ __forceinline__ void load_q_lane(const void* q, int64_t row, int q4, bool real, float (&v)[32]) {
  if (!real) {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    return;
  }
  if (QF32) {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + row * kHeadDim + 32 * q4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 x = src[i];
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + row * kHeadDim + 32 * q4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
}

// The bytes one lane needs from one (page, kv head) tile, and the number of
// valid tokens in that page (0 for an out-of-range page index).
struct PageRegs {
  uint4 kw;      // K codes: token r, dims 32*q4 .. 32*q4+31
  uint32_t ksw;  // K scales: token r, blocks 2*q4, 2*q4+1
  uint4 vw;      // V codes: tokens 4*q4 .. 4*q4+3, dims 8*r .. 8*r+7
  uint32_t vsw;  // V scales: block r/2, tokens 4*q4 .. 4*q4+3
  int valid;
};

// Raw buffer loads from a per-page descriptor: the page's base address lives
// in SGPRs and each lane's offset inside the tile never changes, so the page
// loop does no per-lane address arithmetic; reads past the descriptor's range
// return 0.
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer resource word 3 for raw dword access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int64_t offset, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + offset), 0, bytes, kBufferFlags);
}

struct LaneOffsets {
  int kc, ks, vc, vs;
};

__device__ __forceinline__ PageRegs load_page(const DecodeParams& p, int page, int pg, int seq_len, int h,
                                              const LaneOffsets& lo) {
  const bool ok = (unsigned)page < (unsigned)p.num_pages;
  const int64_t tile = (int64_t)(ok ? page : 0) * p.H + h;
  const auto kc = tile_rsrc(p.k_codes, tile * kTileCodeBytes, kTileCodeBytes);
  const auto ks = tile_rsrc(p.k_scales, tile * kTileScaleBytes, kTileScaleBytes);
  const auto vc = tile_rsrc(p.v_codes, tile * kTileCodeBytes, kTileCodeBytes);
  const auto vs = tile_rsrc(p.v_scales, tile * kTileScaleBytes, kTileScaleBytes);
  PageRegs d;
  d.kw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, lo.kc, 0, 0));
  d.ksw = __builtin_amdgcn_raw_buffer_load_b16(ks, lo.ks, 0, 0);
  d.vw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vc, lo.vc, 0, 0));
  d.vsw = __builtin_amdgcn_raw_buffer_load_b32(vs, lo.vs, 0, 0);
  d.valid = ok ? min(kPageSize, seq_len - pg * kPageSize) : 0;
  return d;
}

template <bool QF32>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: lets the page loop run on SGPRs
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q4 = lane >> 4;

  const int seq_len = min(p.seq_lens[b], p.max_seq_len);
  const int n_pages = (seq_len + kPageSize - 1) / kPageSize;
  const int p_begin = split * p.pages_per_split;
  if (p_begin >= n_pages) {  // uniform for the whole workgroup
    if (n_pages == 0 && split == 0)
      for (int e = threadIdx.x; e < p.G * kHeadDim; e += kThreads)
        p.out[((int64_t)b * p.Hq + (int64_t)h * p.G) * kHeadDim + e] = 0.0f;  // empty sequence
    return;
  }
  const int p_end = min(p_begin + p.pages_per_split, n_pages);
  const int n_split = (n_pages + p.pages_per_split - 1) / p.pages_per_split;

  // ---- Q as the B operand: lane (q head r of the group, dims 32*q4 .. 32*q4+31)
  float qv[32];
  load_q_lane<QF32>(p.q, (int64_t)b * p.Hq + (int64_t)h * p.G + r, q4, r < p.G, qv);
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qv[i]));
  qmax = max_over_groups(qmax);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
  int qe = 0;
  (void)__builtin_frexpf(qmax, &qe);                                          // qmax < 2^qe
  const float qscale = qmax > 0.0f ? __builtin_ldexpf(1.0f, 15 - qe) : 1.0f;  // exact power of two
  half8_t qa[4];
  half8_t ql[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qv[8 * c + j] * qscale;
      qa[c][j] = (_Float16)x;
      if (QF32) ql[c][j] = (_Float16)(x - (float)qa[c][j]);
    }
  const float tscale = p.qk_scale_log2 / qscale;

  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  float4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- this wave's pages: pg_j = p_begin + wave + kWaves*j, j < n_mine <= 128
  // (the host keeps pages_per_split <= 128*kWaves); their indices sit in two
  // lane registers (pages j and j + 64 in lane j).
  const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
  const int n_mine = p_end - p_begin > wave ? (p_end - p_begin - wave + kWaves - 1) / kWaves : 0;
  const int pidx0 = lane < n_mine ? bt_row[p_begin + wave + kWaves * lane] : 0;
  const int pidx1 = lane + 64 < n_mine ? bt_row[p_begin + wave + kWaves * (lane + 64)] : 0;
  auto process = [&](const PageRegs& cur) {
    const int valid = cur.valid;

    // ---- S^T = K . Q^T over the page; lane (q head r, tokens 4*q4 .. 4*q4+3)
    const half2_t ks0 = e4m3_pair_to_f16_scaled(cur.ksw & 0xFFu, cur.ksw & 0xFFu);
    const half2_t ks1 = e4m3_pair_to_f16_scaled(cur.ksw >> 8, cur.ksw >> 8);
    float4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t kwa[4] = {cur.kw.x, cur.kw.y, cur.kw.z, cur.kw.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const half2_t sc = c < 2 ? ks0 : ks1;
      const half2_t e0 = fp4x2_to_f16_x256<0>(kwa[c]) * sc;
      const half2_t e1 = fp4x2_to_f16_x256<1>(kwa[c]) * sc;
      const half2_t e2 = fp4x2_to_f16_x256<2>(kwa[c]) * sc;
      const half2_t e3 = fp4x2_to_f16_x256<3>(kwa[c]) * sc;
      const half8_t a = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qa[c], S, 0, 0, 0);
      if (QF32) S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[c], S, 0, 0, 0);
    }

    // ---- online softmax (log2 domain).  Raw v_exp_f32: weights below 2^-126
    // of the running max flush to 0, which the f16 weights could not hold anyway.
    float t[4];
    if (valid == kPageSize) {
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = S[i] * tscale;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = (4 * q4 + i < valid) ? S[i] * tscale : -__builtin_inff();
    }
    const float pm = max_over_groups(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
    if (__any(pm > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, pm);
      const float f = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float fj = __shfl(f, 4 * q4 + jj);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][jj] *= fj;
      }
      m_run = m_new;
    }
    // m_run is -inf only while every token seen so far was masked (t = -inf too)
    const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(t[i] - m_use);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const half4_t pa = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

    // ---- O += P . V over the page; lane (dims 8*r .. 8*r+7, tokens 4*q4 .. 4*q4+3)
    uint32_t vsw = cur.vsw;
    if (valid != kPageSize) {
      const int nv = min(max(valid - 4 * q4, 0), 4);
      vsw &= nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);  // zero the scales of tokens past the end
    }
    const half2_t vs01 = e4m3_pair_to_f16_scaled(vsw & 0xFFu, (vsw >> 8) & 0xFFu);
    const half2_t vs23 = e4m3_pair_to_f16_scaled((vsw >> 16) & 0xFFu, vsw >> 24);
    const uint32_t E01 = bfi(0x0F0F0F0Fu, cur.vw.x, cur.vw.y << 4), O01 = bfi(0x0F0F0F0Fu, cur.vw.x >> 4, cur.vw.y);
    const uint32_t E23 = bfi(0x0F0F0F0Fu, cur.vw.z, cur.vw.w << 4), O23 = bfi(0x0F0F0F0Fu, cur.vw.z >> 4, cur.vw.w);
#define NVFP4_PV_STEP(C)                                                                   \
  {                                                                                        \
    const half2_t a0 = fp4x2_to_f16_x256<C>(E01) * vs01;                                   \
    const half2_t a1 = fp4x2_to_f16_x256<C>(E23) * vs23;                                   \
    const half2_t b0 = fp4x2_to_f16_x256<C>(O01) * vs01;                                   \
    const half2_t b1 = fp4x2_to_f16_x256<C>(O23) * vs23;                                   \
    const half4_t ve = {a0[0], a0[1], a1[0], a1[1]};                                       \
    const half4_t vo = {b0[0], b0[1], b1[0], b1[1]};                                       \
    acc[2 * C] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, ve, acc[2 * C], 0, 0, 0);       \
    acc[2 * C + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vo, acc[2 * C + 1], 0, 0, 0); \
  }
    NVFP4_PV_STEP(0)
    NVFP4_PV_STEP(1)
    NVFP4_PV_STEP(2)
    NVFP4_PV_STEP(3)
#undef NVFP4_PV_STEP
  };
  const LaneOffsets lo{r * 64 + q4 * 16, r * 8 + q4 * 2, lane * 16, (r >> 1) * 16 + q4 * 4};
  auto load_mine = [&](int j) {
    const int jc = min(j, n_mine - 1);
    const int page = jc < 64 ? __builtin_amdgcn_readlane(pidx0, jc) : __builtin_amdgcn_readlane(pidx1, jc - 64);
    return load_page(p, page, p_begin + wave + kWaves * jc, seq_len, h, lo);
  };
  // Two register sets, unrolled by two: each set is loaded one page ahead of
  // its use and refilled right after, so no register copy waits on a load in
  // flight (loads past the last page re-read that page).
  if (n_mine > 0) {
    PageRegs A = load_mine(0);
    for (int j = 0; j < n_mine; j += 2) {
      const PageRegs B = load_mine(j + 1);
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before any work on the current page
      process(A);
      if (j + 1 >= n_mine) break;
      A = load_mine(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      process(B);
    }
  }

  // ---- per-wave totals: the sum over the 4 token groups
  l_run = sum_over_groups(l_run);

  // ---- merge the waves in LDS
  __shared__ float s_o[kWaves][kMaxGroup][kHeadDim];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];
  if (q4 == 0) {
    s_m[wave][r] = m_run;
    s_l[wave][r] = l_run;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int i = 0; i < 8; ++i) s_o[wave][4 * q4 + jj][8 * r + i] = acc[i][jj];
  __syncthreads();

  const int64_t pbase = (((int64_t)b * p.H + h) * p.num_splits + split) * p.G;
  for (int e = threadIdx.x; e < p.G * kHeadDim; e += kThreads) {
    const int g = e >> 7, d = e & 127;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][g];
      if (mw != -__builtin_inff()) {
        const float f = exp2f(mw - M);
        O += s_o[w][g][d] * f;
        L += s_l[w][g] * f;
      }
    }
    if (n_split == 1) {
      // the whole sequence was in this split: normalise and write the output
      p.out[((int64_t)b * p.Hq + (int64_t)h * p.G + g) * kHeadDim + d] = L > 0.0f ? O / L * p.v_global : 0.0f;
    } else {
      p.part_o[(pbase + g) * kHeadDim + d] = O;
      if (d == 0) {
        p.part_ml[(pbase + g) * 2] = M;
        p.part_ml[(pbase + g) * 2 + 1] = L;
      }
    }
  }
}

// Merge the splits of each (sequence, kv head) that has more than one split,
// and normalise; zero the output of empty sequences.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int seq_len = min(p.seq_lens[b], p.max_seq_len);
  const int n_pages = (seq_len + kPageSize - 1) / kPageSize;
  const int n_split = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  if (n_split == 1) return;  // finished by the split kernel
  const int64_t pbase = ((int64_t)b * p.H + h) * p.num_splits;
  for (int e = threadIdx.x; e < p.G * kHeadDim; e += 256) {
    const int g = e >> 7, d = e & 127;
    float res = 0.0f;
    if (n_split > 0) {
      float M = -__builtin_inff();
      for (int s = 0; s < n_split; ++s) M = fmaxf(M, p.part_ml[((pbase + s) * p.G + g) * 2]);
      float O = 0.0f, L = 0.0f;
      if (M != -__builtin_inff()) {
        for (int s = 0; s < n_split; ++s) {
          const int64_t at = (pbase + s) * p.G + g;
          const float ms = p.part_ml[at * 2];
          if (ms == -__builtin_inff()) continue;
          const float f = exp2f(ms - M);
          O += p.part_o[at * kHeadDim + d] * f;
          L += p.part_ml[at * 2 + 1] * f;
        }
      }
      res = L > 0.0f ? O / L * p.v_global : 0.0f;
    }
    p.out[((int64_t)b * p.Hq + (int64_t)h * p.G + g) * kHeadDim + d] = res;
  }
}

}  // namespace

DecodeGeometry decode_geometry(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len) {
  DecodeGeometry geo{0, 0, 0, false};
  if (batch <= 0 || max_seq_len <= 0 || num_kv_heads <= 0 || num_q_heads <= 0) return geo;
  const int64_t max_pages = ((int64_t)max_seq_len + kPageSize - 1) / kPageSize;
  // Spread the pages of the whole call over about kTargetGroups workgroups, in
  // multiples of kWaves pages so every wave of a split gets work.
  int64_t pps = ((int64_t)batch * num_kv_heads * max_pages + kTargetGroups - 1) / kTargetGroups;
  pps = (pps + kWaves - 1) / kWaves * kWaves;
  if (pps < kWaves) pps = kWaves;
  if (pps > kMaxPagesPerWave * kWaves) pps = kMaxPagesPerWave * kWaves;  // page indices held in lanes
  const int64_t max_pps = (max_pages + kWaves - 1) / kWaves * kWaves;
  if (pps > max_pps) pps = max_pps;
  geo.pages_per_split = (int32_t)pps;
  geo.num_splits = (int32_t)((max_pages + pps - 1) / pps);
  geo.needs_combine = geo.num_splits > 1;
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t units = geo.num_splits > 1 ? (int64_t)batch * num_kv_heads * geo.num_splits * G : 0;
  geo.workspace_bytes = (size_t)(units * (kHeadDim + 2) * sizeof(float));
  return geo;
}

hipError_t launch_decode(const DecodeParams& p, nvfp4_dtype_t q_dtype, bool needs_combine, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (p.num_splits > 0) {
    const dim3 grid((unsigned)p.num_splits, (unsigned)p.H, (unsigned)p.batch);
    if (q_dtype == NVFP4_DTYPE_F32)
      hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Sequences of length 0 get zeros from the combine kernel; it is also needed
  // when max_seq_len == 0 (no split launched at all).
  if (needs_combine || p.num_splits == 0) {
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(p.batch * p.H)), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace nvfp4kv
