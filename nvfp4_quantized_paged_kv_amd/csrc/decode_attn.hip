// Split-K paged decode attention over an NVFP4 cache, dequantizing in
// registers, for gfx950 (CDNA4, wave64, MFMA).
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, third data
// flow: decode reads the whole cache for one short query, so its speed is set
// by the cache read; the 4-bit values are widened where they are loaded and the
// block scale is applied in registers, with no separate dequantization pass.
// Section 1 of the same blog: grouped-query heads share one KV head.
//
// Work decomposition.  A workgroup (4 waves) owns one (sequence, kv head,
// split of `pages_per_split` pages); wave w takes pages w, w+4, ... of the
// split.  Each wave runs one page (16 tokens) per iteration:
//   QK^T  S[16 tok x 16 q] = K_page[16 x 128] . Q^T : 4 x mfma_f32_16x16x32_f16
//         (A = K: lane (tok = l%16, k-group l/16) loads 16 contiguous code bytes =
//          dims 32*(l/16)..+31 of its token; B = Q, the same dims, in registers)
//   online softmax in fp32 (exp2 domain), with a lazy max: the running max is
//         only raised when a page exceeds it by more than 2^8, so P <= 2^8
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
// The 4 waves of a workgroup merge their (max, sum, O) in LDS and write one
// partial per split; a second kernel merges the splits and normalises.
#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

constexpr int kWaves = 4;
constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max must move

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

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

template <bool QF32>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q4 = lane >> 4;

  const int seq_len = min(p.seq_lens[b], p.max_seq_len);
  const int n_pages = (seq_len + kPageSize - 1) / kPageSize;
  const int p_begin = split * p.pages_per_split;
  if (p_begin >= n_pages) return;  // uniform for the whole workgroup
  const int p_end = min(p_begin + p.pages_per_split, n_pages);

  // ---- Q as the B operand: lane (q head r of the group, dims 32*q4 .. 32*q4+31)
  float qv[32];
  load_q_lane<QF32>(p.q, (int64_t)b * p.Hq + (int64_t)h * p.G + r, q4, r < p.G, qv);
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qv[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
  int qe = 0;
  (void)__builtin_frexpf(qmax, &qe);                              // qmax < 2^qe
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

  const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
  for (int pg = p_begin + wave; pg < p_end; pg += kWaves) {
    const int page = bt_row[pg];
    const bool page_ok = (unsigned)page < (unsigned)p.num_pages;
    const int64_t tile = (int64_t)(page_ok ? page : 0) * p.H + h;
    const int valid = page_ok ? min(kPageSize, seq_len - pg * kPageSize) : 0;

    const uint4 kw = *reinterpret_cast<const uint4*>(p.k_codes + tile * kTileCodeBytes + r * 64 + q4 * 16);
    const uint32_t ksw = *reinterpret_cast<const uint16_t*>(p.k_scales + tile * kTileScaleBytes + r * 8 + q4 * 2);
    const uint4 vw = *reinterpret_cast<const uint4*>(p.v_codes + tile * kTileCodeBytes + lane * 16);
    uint32_t vsw = *reinterpret_cast<const uint32_t*>(p.v_scales + tile * kTileScaleBytes + (r >> 1) * 16 + q4 * 4);

    // ---- S^T = K . Q^T over the page; lane (q head r, tokens 4*q4 .. 4*q4+3)
    const half2_t ks0 = e4m3_pair_to_f16_scaled(ksw & 0xFFu, ksw & 0xFFu);
    const half2_t ks1 = e4m3_pair_to_f16_scaled(ksw >> 8, ksw >> 8);
    float4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
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

    // ---- online softmax (log2 domain)
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (4 * q4 + i < valid) ? S[i] * tscale : -__builtin_inff();
    float pm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
    pm = fmaxf(pm, __shfl_xor(pm, 16));
    pm = fmaxf(pm, __shfl_xor(pm, 32));
    if (__any(pm > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, pm);
      const float f = m_run == -__builtin_inff() ? 0.0f : exp2f(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float fj = __shfl(f, 4 * q4 + jj);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][jj] *= fj;
      }
      m_run = m_new;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = t[i] == -__builtin_inff() ? 0.0f : exp2f(t[i] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const half4_t pa = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

    // ---- O += P . V over the page; lane (dims 8*r .. 8*r+7, tokens 4*q4 .. 4*q4+3)
    {
      const int nv = min(max(valid - 4 * q4, 0), 4);
      vsw &= nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);  // zero the scales of tokens past the end
    }
    const half2_t vs01 = e4m3_pair_to_f16_scaled(vsw & 0xFFu, (vsw >> 8) & 0xFFu);
    const half2_t vs23 = e4m3_pair_to_f16_scaled((vsw >> 16) & 0xFFu, vsw >> 24);
    const uint32_t E01 = bfi(0x0F0F0F0Fu, vw.x, vw.y << 4), O01 = bfi(0x0F0F0F0Fu, vw.x >> 4, vw.y);
    const uint32_t E23 = bfi(0x0F0F0F0Fu, vw.z, vw.w << 4), O23 = bfi(0x0F0F0F0Fu, vw.z >> 4, vw.w);
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
  }

  // ---- per-wave totals: the sum over the 4 token groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the 4 waves in LDS, write one partial for this split
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
  for (int e = threadIdx.x; e < p.G * kHeadDim; e += 256) {
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
    p.part_o[(pbase + g) * kHeadDim + d] = O;
    if (d == 0) {
      p.part_ml[(pbase + g) * 2] = M;
      p.part_ml[(pbase + g) * 2 + 1] = L;
    }
  }
}

// Merge the splits of each (sequence, kv head) and normalise.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int seq_len = min(p.seq_lens[b], p.max_seq_len);
  const int n_pages = (seq_len + kPageSize - 1) / kPageSize;
  const int n_split = (n_pages + p.pages_per_split - 1) / p.pages_per_split;
  const int64_t pbase = ((int64_t)b * p.H + h) * p.num_splits;
  for (int e = threadIdx.x; e < p.G * kHeadDim; e += 256) {
    const int g = e >> 7, d = e & 127;
    float res = 0.0f;
    if (n_split > 0) {
      float M = -__builtin_inff();
      for (int s = 0; s < n_split; ++s) M = fmaxf(M, p.part_ml[((pbase + s) * p.G + g) * 2]);
      float O = 0.0f, L = 0.0f;
      for (int s = 0; s < n_split; ++s) {
        const int64_t at = (pbase + s) * p.G + g;
        const float f = exp2f(p.part_ml[at * 2] - M);
        O += p.part_o[at * kHeadDim + d] * f;
        L += p.part_ml[at * 2 + 1] * f;
      }
      res = O / L * p.v_global;
    }
    p.out[((int64_t)b * p.Hq + (int64_t)h * p.G + g) * kHeadDim + d] = res;
  }
}

}  // namespace

DecodeGeometry decode_geometry(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len) {
  DecodeGeometry geo{0, 0, 0};
  if (batch <= 0 || max_seq_len <= 0 || num_kv_heads <= 0 || num_q_heads <= 0) return geo;
  const int64_t max_pages = ((int64_t)max_seq_len + kPageSize - 1) / kPageSize;
  // About 1024 workgroups (4 per CU, 16 waves per CU) over the whole call, in
  // multiples of 4 pages so every wave of a split gets work.
  const int64_t target_groups = 1024;
  int64_t pps = ((int64_t)batch * num_kv_heads * max_pages + target_groups - 1) / target_groups;
  pps = (pps + 3) / 4 * 4;
  if (pps < 4) pps = 4;
  const int64_t max_pps = (max_pages + 3) / 4 * 4;
  if (pps > max_pps) pps = max_pps;
  geo.pages_per_split = (int32_t)pps;
  geo.num_splits = (int32_t)((max_pages + pps - 1) / pps);
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t units = (int64_t)batch * num_kv_heads * geo.num_splits * G;
  geo.workspace_bytes = (size_t)(units * (kHeadDim + 2) * sizeof(float));
  return geo;
}

hipError_t launch_decode(const DecodeParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  if (p.num_splits > 0) {
    const dim3 grid((unsigned)p.num_splits, (unsigned)p.H, (unsigned)p.batch);
    if (q_dtype == NVFP4_DTYPE_F32)
      hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(p.batch * p.H)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
