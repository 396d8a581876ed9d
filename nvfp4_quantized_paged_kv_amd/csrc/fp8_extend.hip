// FP8 rows of new tokens, and causal extend / prefill attention over FP8
// workspace rows, for gfx950 (CDNA4, wave64, MFMA).
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3: in chunked
// prefill / extend the cached prefix is dequantized from NVFP4 into one FP8
// workspace that every layer reuses (dequant_ws.hip), and the K/V of the
// tokens being processed take part in attention as FP8, as in the first
// prefill.  Here the chunk's K/V are stored as FP8 rows right after their
// prefix (fp8_rows_kernel), and the chunk's queries attend causally over
// [prefix | chunk] (extend_kernel).  The attention is compute-bound (about
// 512 flops per query row and key for 256 bytes per key), so QK^T and PV run
// on MFMA; the E4M3 bytes are widened exactly to f16 in registers.
//
// extend_kernel work split: one workgroup per (16 chunk tokens, kv head,
// sequence); its rows are the 16 tokens of each of the G query heads of the
// kv head.  Wave w owns heads 2w and 2w+1 (two 16-row blocks).  Keys stream
// through LDS in tiles of 32, widened to f16 while they are staged (once per
// workgroup): K rows (padded), V transposed to [dim][key] so that a lane's PV
// operand (4 + 4 keys of one dim) is two 64-bit reads.  Per tile and wave:
//   S^T[key][token] = K . Q^T : 2 key blocks x 4 mfma_f32_16x16x32_f16 per
//                     row block (lane: key 16kb + l%16, dims 32*(l/16)..+31;
//                     Q in the same permuted dim order, so no shuffles)
//   online softmax in fp32 (exp2 domain, lazy max as in the decode kernel)
//   O[token][dim]  += P . V : 8 dim blocks x 2 mfma_f32_16x16x32_f16 (P as
//                     an f16 hi + lo pair, one MFMA each; the
//                     weights stay where the S^T layout put them: the
//                     contraction index is mapped onto the 32 keys to match)
// The FP32 per-tensor workspace scales go on the logits (K) and on the output
// (V); Q is converted to f16 after an exact power-of-two prescale (float32 Q
// as an f16 hi + lo pair), as in the decode kernel.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_kv_internal.h"

namespace nvfp4kv {
namespace {

// ------------------------------------------------------------------ FP8 rows
// One thread per 16 consecutive values of one (token, kv head); blockIdx.y
// picks K or V.  Byte = sign(x) | E4M3 nearest to |x| / ws_scale.  An E4M3
// midpoint times the divisor has at most 29 significant bits, so a float32
// dividend that is not on it lies at least 2^-30 (relative) away.  The
// quotient is |x| * RN(1/ws_scale) (within 2^-52) plus one correction with
// the exact residual |x| - q0 * ws_scale (one fma), within about 2^-104 of
// the exact one: it rounds like the exact quotient, and an exact midpoint
// comes out exactly (ties to even).
template <typename InT>
__global__ __launch_bounds__(256) void fp8_rows_kernel(Fp8RowsParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int tensor = blockIdx.y;
  if (i >= (int64_t)p.num_tokens * p.H * 8) return;
  const int grp = (int)(i & 7);
  const int64_t th = i >> 3;
  const int h = (int)(th % p.H);
  const int64_t t = th / p.H;
  const int row = p.rows[t];  // checked at the store: the input loads do not wait for it
  const uint8_t* src = reinterpret_cast<const uint8_t*>(p.x[tensor]) +
                       (t * p.token_stride + (int64_t)h * kHeadDim + grp * 16) * (int64_t)sizeof(InT);
  float v[16];
  if (sizeof(InT) == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 w = reinterpret_cast<const uint4*>(src)[k];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = __uint_as_float(ww[j] << 16);
        v[8 * k + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 w = reinterpret_cast<const uint4*>(src)[k];
      v[4 * k] = __uint_as_float(w.x);
      v[4 * k + 1] = __uint_as_float(w.y);
      v[4 * k + 2] = __uint_as_float(w.z);
      v[4 * k + 3] = __uint_as_float(w.w);
    }
  }
  const double s = (double)p.ws_scale[tensor], r = p.ws_rcp[tensor];
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const double a = (double)__builtin_fabsf(v[k]);
    const double q0 = a * r;
    const uint32_t mag = e4m3_encode_rne_sat(__builtin_fma(__builtin_fma(-q0, s, a), r, q0));
    const uint32_t byte = mag | ((__float_as_uint(v[k]) >> 24) & 0x80u);
    w[k >> 2] |= byte << (8 * (k & 3));
  }
  if (row < 0 || row >= p.ws_capacity) return;
  *reinterpret_cast<uint4*>(p.ws[tensor] + ((int64_t)row * p.H + h) * kHeadDim + grp * 16) =
      uint4{w[0], w[1], w[2], w[3]};
}

// ------------------------------------------------------------ extend attention
constexpr int kExtTok = 16;                        // chunk tokens per workgroup
constexpr int kExtKeys = 32;                       // keys per LDS tile
constexpr int kKStride = 272;                      // LDS bytes per K row: 128 f16 + 16 pad
// LDS bytes per transposed V row: 32 f16 keys + 8 pad.  With 72 the 16 lanes
// of a PV-operand read (16 rows, 8 bytes each) cover the 32 banks once; 80
// left rows r and r + 8 on the same banks (measured: bank-conflict cycles
// 47% -> 33% of LDS-active cycles, about 3% off the kernel)
constexpr int kVStride = 72;
constexpr int kBufferFlags = 0x00020000;           // gfx9 buffer resource word 3 for raw dword access
constexpr int kKTileBytes = kExtKeys * kKStride;
constexpr int kVTileBytes = kHeadDim * kVStride;
constexpr float kExtLazyMax = 8.0f;                // log2 headroom before the running max moves

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over lanes l, l^16, l^32, l^48 (the 4 key groups of one query row)
__device__ __forceinline__ float vmax_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Two E4M3 bytes of word `w` (bytes 0-1, or 2-3 with HI) widened exactly to
// an f16 pair, returned as its 32-bit pattern (scale operand 1.0).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Three waves per SIMD for bf16 queries (at most 168 VGPRs; the P hi + lo
// pair would otherwise take the kernel just past that); the float32-query
// kernel holds a second Q pair and runs two waves per SIMD either way.
template <bool QF32>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(QF32 ? 2 : 3))) void extend_kernel(
    ExtendParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kKTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kVTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int er = lane & 15, eq = lane >> 4;
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
  const int t0 = tile * kExtTok;
  if (t0 >= C) return;
  const int ntok = min(kExtTok, C - t0);
  const int P = min(max(__builtin_amdgcn_readfirstlane(p.prefix_lens[seq]), 0), p.ws_capacity);
  const int64_t woff = __builtin_amdgcn_readfirstlane(p.ws_offsets[seq]);
  const int n_keys = P + t0 + ntok;  // keys the tile's last token sees
  const int n_all = P + t0 + 1;      // keys every token of the tile sees
  const int n_kt = (n_keys + kExtKeys - 1) / kExtKeys;
  // this workgroup's key tiles [kt0, kt1): an equal share of the tile's keys
  // (a share may be empty; it then stores an empty partial)
  const int kt0 = (int)((int64_t)split * n_kt / S), kt1 = (int)((int64_t)(split + 1) * n_kt / S);

  // ---- tile loads: thread tid < 256 moves 16 K bytes (key tid/8, dims 16*(tid%8)..+15)
  // and a 4x4 block of V (keys 4*vg..+3, dims 4*vd..+3, with tid bits 0-1 and 4 giving
  // vg and bits 2-3 and 5-7 giving vd: the 16 lanes of one transposed LDS store span 4
  // key groups x 4 dim groups, which the 72-byte rows put on distinct banks; a wave
  // instruction still loads the same 8 keys x 32 dims from memory).  Raw buffer
  // loads through a per-tile descriptor over the sequence's valid rows: rows past
  // them (or past the workspace) read as 0, and a thread's offsets never change.
  const bool loader = tid < 256;
  const int kk = tid >> 3, kc = tid & 7;
  const int vg = (tid & 3) | (((tid >> 4) & 1) << 2), vd = ((tid >> 2) & 3) | ((tid >> 5) << 2);
  const int row_bytes = H * kHeadDim;
  const int64_t valid_rows = (woff >= 0 && woff < p.ws_capacity) ? min((int64_t)n_keys, (int64_t)p.ws_capacity - woff) : 0;
  const int ko = (kk * H + h) * kHeadDim + 16 * kc;
  int vo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vo[j] = ((4 * vg + j) * H + h) * kHeadDim + 4 * vd;
  auto tile_rsrc = [&](const uint8_t* base, int kt) {
    const int64_t r0 = (int64_t)kt * kExtKeys;
    const int64_t rows = max((int64_t)0, min((int64_t)kExtKeys, valid_rows - r0));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + (woff + r0) * row_bytes, 0,
                                             (int)(rows * row_bytes), kBufferFlags);
  };
  uint4 kreg = {0u, 0u, 0u, 0u};
  uint32_t vreg[4] = {0u, 0u, 0u, 0u};
  auto load_tile = [&](int kt) {
    if (!loader) return;
    const auto rk = tile_rsrc(p.ws_k, kt);
    const auto rv = tile_rsrc(p.ws_v, kt);
    kreg = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) vreg[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo[j], 0, 0);
  };
  // The tile goes into LDS already widened to f16 (once per workgroup, not per wave).
  auto store_tile = [&](int buf) {
    if (!loader) return;
    uint8_t* kp = &s_k[buf][kk * kKStride + 32 * kc];
    *reinterpret_cast<uint4*>(kp) = uint4{fp8x2_to_f16x2<false>(kreg.x), fp8x2_to_f16x2<true>(kreg.x),
                                          fp8x2_to_f16x2<false>(kreg.y), fp8x2_to_f16x2<true>(kreg.y)};
    *reinterpret_cast<uint4*>(kp + 16) = uint4{fp8x2_to_f16x2<false>(kreg.z), fp8x2_to_f16x2<true>(kreg.z),
                                               fp8x2_to_f16x2<false>(kreg.w), fp8x2_to_f16x2<true>(kreg.w)};
    // 4x4 byte transpose: t[e] = dim 4*vd+e of keys 4*vg .. 4*vg+3
    const uint32_t a_lo = __builtin_amdgcn_perm(vreg[1], vreg[0], 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
    const uint32_t a_hi = __builtin_amdgcn_perm(vreg[1], vreg[0], 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
    const uint32_t b_lo = __builtin_amdgcn_perm(vreg[3], vreg[2], 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(vreg[3], vreg[2], 0x07030602u);
    const uint32_t t[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u), __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                           __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u), __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
    uint8_t* vt = &s_v[buf][(4 * vd) * kVStride + 8 * vg];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<uint2*>(vt + e * kVStride) = uint2{fp8x2_to_f16x2<false>(t[e]), fp8x2_to_f16x2<true>(t[e])};
  };
  if (kt0 < kt1) load_tile(kt0);

  // ---- this wave's two row blocks: query heads 2*wave and 2*wave+1, tokens t0 .. t0+15
  const bool active = 2 * wave < G;
  half8_t qa[2][4], ql[2][4];
  float tscale[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int g = 2 * wave + rb;
    float qv[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) qv[k] = 0.0f;
    if (active && g < G && er < ntok) {
      const int64_t qoff = ((int64_t)(q0 + t0 + er) * p.Hq + (int64_t)h * G + g) * kHeadDim + 32 * eq;
      if (QF32) {
        const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.q) + qoff);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint4 w = qp[k];
          qv[4 * k] = __uint_as_float(w.x);
          qv[4 * k + 1] = __uint_as_float(w.y);
          qv[4 * k + 2] = __uint_as_float(w.z);
          qv[4 * k + 3] = __uint_as_float(w.w);
        }
      } else {
        const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 w = qp[k];
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            qv[8 * k + 2 * j] = __uint_as_float(ww[j] << 16);
            qv[8 * k + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
          }
        }
      }
    }
    float qmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) qmax = fmaxf(qmax, __builtin_fabsf(qv[k]));
    qmax = wave_max(qmax);
    int qe = 0;
    (void)__builtin_frexpf(qmax, &qe);  // qmax < 2^qe
    // exact power of two carrying the sign of the logit scale, so that tscale >= 0
    const float qscale = __builtin_copysignf(qmax > 0.0f ? __builtin_ldexpf(1.0f, 15 - qe) : 1.0f, p.qk_scale_log2);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xq = qv[8 * c + j] * qscale;
        qa[rb][c][j] = (_Float16)xq;
        ql[rb][c][j] = QF32 ? (_Float16)(xq - (float)qa[rb][c][j]) : (_Float16)0.0f;
      }
    tscale[rb] = fmaxf(p.qk_scale_log2 / qscale, __FLT_MIN__);
  }

  float m_run[2] = {-__FLT_MAX__, -__FLT_MAX__};  // -FLT_MAX: no maximum yet
  float m_lim[2] = {-__FLT_MAX__, -__FLT_MAX__};
  float l_run[2] = {0.0f, 0.0f};
  float4_t acc[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[rb][d] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    store_tile(buf);
    __syncthreads();
    if (kt + 1 < kt1) load_tile(kt + 1);  // in flight while this tile is computed
    if (!active) continue;

    // ---- S^T = K . Q^T for the tile's two 16-key blocks
    float4_t S[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t* kp = &s_k[buf][(16 * kb + er) * kKStride + 64 * eq];  // f16 dims 32*eq .. +31
      S[kb][0] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      S[kb][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const half8_t a = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(kp + 16 * c));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          S[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qa[rb][c], S[kb][rb], 0, 0, 0);
          if (QF32) S[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[rb][c], S[kb][rb], 0, 0, 0);
        }
      }
    }
    // explicit wait states between the MFMA results and their first VALU
    // reads (20 cover MFMAs of up to 16 passes), as in the decode kernel
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[1][0]), "+v"(S[1][1]));

    // ---- causal mask: only tiles reaching past the keys every token sees
    const int kbase = kt * kExtKeys;
    if (kbase + kExtKeys > n_all) {
      const int lim = P + t0 + er;  // last key of this lane's token
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + 16 * kb + 4 * eq + i > lim) {
            S[kb][0][i] = -__builtin_inff();
            S[kb][1][i] = -__builtin_inff();
          }
    }

    // ---- online softmax per row block (exp2 domain, lazy max)
    half4_t pa[2][2], pl[2][2];  // P as an f16 hi + lo pair
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // the lane's own 8 scores decide whether any row's maximum passes its
      // lazy bound; only then is the maximum over the 4 key groups taken
      // (tscale >= 0 and rounding are monotone: the maximum of the scaled
      // scores is the scaled maximum)
      const float lm = vmax(vmax(vmax(S[0][rb][0], S[0][rb][1]), vmax(S[0][rb][2], S[0][rb][3])),
                            vmax(vmax(S[1][rb][0], S[1][rb][1]), vmax(S[1][rb][2], S[1][rb][3]))) *
                       tscale[rb];
      if (__any(lm > m_lim[rb])) {
        const float pm = vmax_over_groups(lm);
        const float m_new = fmaxf(m_run[rb], pm);
        const float f = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float fj = __shfl(f, 4 * eq + jj);
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[rb][d][jj] *= fj;
        }
        m_run[rb] = m_new;
        m_lim[rb] = m_new + kExtLazyMax;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)  // the rounded product, as in pm: t - m_run <= kExtLazyMax for any logit
          pr[i] = __builtin_amdgcn_exp2f(S[kb][rb][i] * tscale[rb] - m_run[rb]);
        l_run[rb] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        // hi = p rounded toward zero to f16 (11 significant bits for p >= 2^-14) by
        // the packed conversion; lo = p - hi (exact in float32) rounded to f16 by
        // the mixed-precision FMA, which reads hi from the packed register.  The
        // multiplier 1.0 is opaque to the compiler, which would otherwise fold the
        // FMA into a subtraction with separate conversions.
        float one = 1.0f;
        asm volatile("" : "+s"(one));
        const half2_t h01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pr[0], pr[1]));
        const half2_t h23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pr[2], pr[3]));
        pa[rb][kb] = half4_t{h01[0], h01[1], h23[0], h23[1]};
        pl[rb][kb] = half4_t{(_Float16)__builtin_fmaf(pr[0], one, -(float)h01[0]),
                             (_Float16)__builtin_fmaf(pr[1], one, -(float)h01[1]),
                             (_Float16)__builtin_fmaf(pr[2], one, -(float)h23[0]),
                             (_Float16)__builtin_fmaf(pr[3], one, -(float)h23[1])};
      }
    }

    // ---- O += P . V, one 16x16x32 MFMA per dim block: its contraction index
    // k = 8*eq + j stands for key 4*eq + j (j < 4) of key block 0 and key
    // 16 + 4*eq + j - 4 of key block 1, which is how the S^T layout left the
    // weights in this lane; V is read from the transposed tile in the same order.
    // P enters as an f16 hi + lo pair (about 22 bits), the lo part first: with P
    // in f16 alone (11 bits) a row whose output nearly cancels can miss 1e-3 of
    // its largest value.
    half8_t pw[2], pwl[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      pw[rb] = __builtin_shufflevector(pa[rb][0], pa[rb][1], 0, 1, 2, 3, 4, 5, 6, 7);
      pwl[rb] = __builtin_shufflevector(pl[rb][0], pl[rb][1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint8_t* vp = &s_v[buf][(16 * db + er) * kVStride + 8 * eq];
      const uint2 v0 = *reinterpret_cast<const uint2*>(vp);       // f16 keys 4*eq .. +3
      const uint2 v1 = *reinterpret_cast<const uint2*>(vp + 32);  // f16 keys 16 + 4*eq .. +3
      const half8_t b = __builtin_bit_cast(half8_t, uint4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pwl[rb], b, acc[rb][db], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw[rb], b, acc[rb][db], 0, 0, 0);
    }
  }
  if (!active) return;

  // ---- lane holds O[token 4*eq + i][dim 16*db + er]
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int g = 2 * wave + rb;
    const float l_tot = sum_over_groups(l_run[rb]);  // lane er: the row sum of token er
    if (g >= G) continue;
    if (S > 1) {
      // a share of the keys: the unnormalised partial, its maximum and sum (merged by extend_merge_kernel)
      auto part_row = [&](int row) {
        return p.part + (((int64_t)split * p.num_q_tokens + q0 + t0 + row) * p.Hq + (int64_t)h * G + g) * kExtPartStride;
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * eq + i;
        if (row >= ntok) continue;
        float* pp = part_row(row) + er;
#pragma unroll
        for (int db = 0; db < 8; ++db) pp[16 * db] = acc[rb][db][i];
      }
      if (eq == 0 && er < ntok) {
        float* pp = part_row(er);
        pp[kHeadDim] = m_run[rb];
        pp[kHeadDim + 1] = l_tot;
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * eq + i;
      const float L = __shfl(l_tot, row);
      if (row >= ntok) continue;
      float* op = p.out + ((int64_t)(q0 + t0 + row) * p.Hq + (int64_t)h * G + g) * kHeadDim + er;
      const float f = p.v_scale / L;
#pragma unroll
      for (int db = 0; db < 8; ++db) op[16 * db] = acc[rb][db][i] * f;
    }
  }
}

// The split extend's merge, one workgroup per (chunk token, query head):
//   out = v_scale * sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),  M = max_s m_s
// over the splits' partials (an empty share has m_s = -FLT_MAX, l_s = 0 and
// O_s = 0, so it weighs nothing).  Thread s < S first takes split s's
// maximum and sum; then 8 groups of 32 threads each sum every 8th split's
// O (4 dims a thread, independent loads in flight) and LDS adds the groups.
__global__ __launch_bounds__(256) void extend_merge_kernel(ExtendParams p) {
  __shared__ float s_f[kExtMaxSplits];
  __shared__ float s_wm[4], s_wl[4];
  __shared__ float4 s_o[8][32];
  const int seq = blockIdx.y;
  const int t = (int)(blockIdx.x / (uint32_t)p.Hq), qh = (int)(blockIdx.x % (uint32_t)p.Hq);
  const int nq = p.num_q_tokens;
  const int q0 = min(max(p.q_offsets[seq], 0), nq);
  const int q1 = min(max(p.q_offsets[seq + 1], q0), nq);
  if (t >= min(q1 - q0, p.max_chunk)) return;
  const int S = p.splits, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok = q0 + t;
  const int64_t split_stride = (int64_t)nq * p.Hq * kExtPartStride;
  const float* base = p.part + (tok * p.Hq + qh) * kExtPartStride;

  const float m = tid < S ? base[tid * split_stride + kHeadDim] : -__FLT_MAX__;
  const float l = tid < S ? base[tid * split_stride + kHeadDim + 1] : 0.0f;
  float wm = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
  if (lane == 0) s_wm[wave] = wm;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_wm[0], s_wm[1]), fmaxf(s_wm[2], s_wm[3]));
  const float f = tid < S ? exp2f(m - M) : 0.0f;
  s_f[tid] = f;
  float wl = l * f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wl += __shfl_xor(wl, o);
  if (lane == 0) s_wl[wave] = wl;
  __syncthreads();

  const int sg = tid >> 5, d = 4 * (tid & 31);
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = sg; s < S; s += 8) {
    const float fs = s_f[s];
    const float4 o = *reinterpret_cast<const float4*>(base + s * split_stride + d);
    O.x += o.x * fs;
    O.y += o.y * fs;
    O.z += o.z * fs;
    O.w += o.w * fs;
  }
  s_o[sg][tid & 31] = O;
  __syncthreads();
  if (tid < 32) {
    float4 a = s_o[0][tid];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      const float4 b = s_o[g][tid];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const float L = (s_wl[0] + s_wl[1]) + (s_wl[2] + s_wl[3]);
    const float r = L > 0.0f ? p.v_scale / L : 0.0f;
    *reinterpret_cast<float4*>(p.out + (tok * p.Hq + qh) * kHeadDim + d) = make_float4(a.x * r, a.y * r, a.z * r, a.w * r);
  }
}

}  // namespace

ExtendGeometry extend_geometry(nvfp4_dtype_t q_dtype, int32_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t max_chunk, int32_t max_prefix) {
  ExtendGeometry geo{1, 0};
  if (num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_seqs <= 0 || max_chunk <= 0 || max_prefix < 0)
    return geo;
  // split a tile's keys only when the tiles alone fill at most half a round
  // of resident workgroups: 4-wave workgroups (up to 8 query heads per kv
  // head) take 3 per CU with bf16 queries (161 VGPRs, 3 waves per SIMD) and
  // 2 with float32 ones (211 VGPRs), 8-wave workgroups 1.  The split then
  // fills one round without starting a second (whose stragglers would take
  // as long as the whole first round), each share at least kExtMinShareKeys keys.
  const int32_t G = num_q_heads / num_kv_heads;
  const int64_t round = 256 * (G > 8 ? 1 : q_dtype == NVFP4_DTYPE_F32 ? 2 : 3);
  const int64_t tiles = (int64_t)((max_chunk + kExtTok - 1) / kExtTok) * num_kv_heads * num_seqs;
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

hipError_t launch_fp8_rows(const Fp8RowsParams& p, nvfp4_dtype_t dtype, hipStream_t stream) {
  const int64_t n = (int64_t)p.num_tokens * p.H * 8;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256), 2);
  if (dtype == NVFP4_DTYPE_F32)
    hipLaunchKernelGGL(fp8_rows_kernel<float>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(fp8_rows_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_chunk == 0 || p.num_q_tokens == 0) return hipSuccess;
  if (p.splits < 1 || p.splits > kExtMaxSplits) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((p.max_chunk + kExtTok - 1) / kExtTok * p.splits), (unsigned)p.H, (unsigned)p.num_seqs);
  const dim3 block(p.G <= 8 ? 256 : 512);  // at least 256 threads: the tile loaders
  if (q_dtype == NVFP4_DTYPE_F32)
    hipLaunchKernelGGL(extend_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(extend_kernel<false>, grid, block, 0, stream, p);
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_extend_merge(p, stream);
  }
  return hipGetLastError();
}

hipError_t launch_extend_merge(const ExtendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(extend_merge_kernel, dim3((unsigned)p.max_chunk * (unsigned)p.Hq, (unsigned)p.num_seqs), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
