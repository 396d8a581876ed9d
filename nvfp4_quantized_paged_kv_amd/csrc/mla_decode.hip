// Sparse-MLA over an NVFP4 latent cache, for gfx950: quantize-append of latent
// rows and decode attention over each query token's listed cache slots.
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 6 (closing
// note): the serving engine's NVFP4 KV cache supports GQA and Sparse MLA
// models.  An MLA cache row is the token's latent vector shared by every query
// head: 512 latent values and 64 rotary-key values.  The decode scores a query
// head against all 576 values and sums the first 512 (the absorbed-projection
// form); "sparse" means each query token attends only to the cache slots of
// its top-k list.  The row is stored with the GQA cache's two-level rule
// (section 2 of the same blog): 36 blocks of 16 values, one E4M3 scale per
// block, one FP32 scale per layer.
//
// Row layout: codes [num_slots][288] (byte j = values 2j, 2j+1, low nibble
// first), scales [num_slots][36] (byte b = block b).  A row's 32-value chunk c
// is 16 code bytes at 16c and 2 scale bytes at 2c.
//
// Decode work: one workgroup per (query token, 16*WAVES query heads, share of
// the list); wave w owns 16 heads.  Per tile of 32 list entries the workgroup
// gathers the rows (one thread per (entry, 32-value chunk): 16-byte code load,
// 2-byte scale load), dequantizes them once into LDS as f16 (e2m1 * bs is
// exact in f16), double-buffered, and every wave computes from that copy:
//   S^T[2 x 16 entries x 16 heads] = K . Q^T : 2 x 18 mfma_f32_16x16x32_f16
//     (A = staged rows, lane (entry l%16, dims 32c + 8*(l/16) .. +7), one
//      16-byte LDS read; B = Q in registers, f16 after an exact power-of-two
//      prescale)
//   online softmax in fp32 (log2 domain, lazy running max, as the GQA decode)
//   O[16 heads x 512] += P . V : 2 x 32 mfma_f32_16x16x32_f16; the k = 32
//     operand holds 8 of the tile's entries per 16-lane group (4 of each
//     half), P enters as an f16 hi + lo pair, one MFMA each; the V operand
//     -- those entries at one dim -- comes from the same row-major copy with
//     two transposing LDS reads (ds_read_b64_tr_b16: within each 16-lane
//     group, lane p receives element p%4 of the 8-byte chunks that lanes
//     p/4 + 4k address, k = 0..3)
// The global scale enters the logits and the final output.  When few query
// tokens leave CUs idle, each list is split into shares over several
// workgroups; each share stores its (max, sum, O) in the workspace and a merge
// launch combines them (one thread per 4 output values).
#include "mla_internal.h"
#include "nvfp4_quant_device.h"

namespace nvfp4kv {
namespace {

constexpr int kTile = 32;                        // list entries per tile
constexpr int kChunks = kMlaDim / 32;            // 18 chunks of 32 values per row
constexpr int kStageJobs = kTile * kChunks;      // 576 (entry, chunk) jobs per tile
constexpr int kRow = kMlaDim + 8;                // f16 per staged row (292 dwords: conflict-free 16-byte reads)
constexpr float kLazyMax = 8.0f;                 // log2 headroom before the running max must move

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over lanes l, l^16, l^32, l^48 (the 4 entry groups of one head)
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

// ---------------------------------------------------------- quantize-append
// One thread per (token, 32-value chunk): two blocks through the exact block
// quantizer of the GQA cache; 16 code bytes and 2 scale bytes stored.
template <typename InT>
__global__ __launch_bounds__(256) void mla_append_kernel(MlaAppendParams p) {
  const int64_t job = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (job >= (int64_t)p.num_tokens * kChunks) return;
  const int t = (int)(job / kChunks), c = (int)(job - (int64_t)t * kChunks);
  const InT* src = reinterpret_cast<const InT*>(p.x) + (int64_t)t * p.token_stride + 32 * c;
  float x0[16], x1[16];
  load_block<InT>(src, x0);
  load_block<InT>(src + 16, x1);
  const int32_t slot = p.slots[t];
  const QuantBlock q0 = quantize_block16(x0, p.g, p.r6);
  const QuantBlock q1 = quantize_block16(x1, p.g, p.r6);
  if ((uint32_t)slot >= (uint32_t)p.num_slots) return;  // skipped slot
  *reinterpret_cast<uint4*>(p.codes + (int64_t)slot * kMlaRowCodeBytes + 16 * c) =
      make_uint4(q0.packed[0], q0.packed[1], q1.packed[0], q1.packed[1]);
  *reinterpret_cast<uint16_t*>(p.scales + (int64_t)slot * kMlaRowScaleBytes + 2 * c) =
      (uint16_t)(q0.sb | (q1.sb << 8));
}

// ------------------------------------------------------------------ decode
struct Stage {
  uint4 w;      // 16 code bytes of the chunk
  uint32_t s;   // its 2 scale bytes
  int ok;       // the entry is a slot inside the cache
};

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mla_decode_kernel(MlaDecodeParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int kHeads = 16 * WAVES;
  constexpr int kPer = (kStageJobs + NT - 1) / NT;  // staging jobs per thread
  // One-wave workgroups (16 heads) stage into a single buffer: two 37 KB
  // buffers let only 2 such workgroups (2 of the CU's 4 SIMDs) be resident,
  // one lets 4; the next tile's rows are then written after this tile's PV.
  constexpr int kBufs = WAVES == 1 ? 1 : 2;
  __shared__ __align__(16) _Float16 s_k[kBufs][kTile * kRow];
  __shared__ int s_valid[kBufs][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int sp = (int)(blockIdx.x % (uint32_t)p.splits);
  const int u = (int)(blockIdx.x / (uint32_t)p.splits);  // unit: (query token, head block)
  const int t = u / p.HB, hb = u - t * p.HB;
  const int e0 = sp * p.per_split, e1 = min(e0 + p.per_split, p.topk);
  const int n_tiles = e1 > e0 ? (e1 - e0 + kTile - 1) / kTile : 0;
  const int32_t* idx_row = p.indices + (int64_t)t * p.topk;
  const int head0 = hb * kHeads + 16 * wave;  // first head of this wave

  // ---- staging: job j = (entry j % 32 of the tile, chunk j / 32).  Every
  // load is unconditional, from a clamped address that always lies inside its
  // array, and validity is applied where the data is used: a load under a
  // divergent branch would be waited on where the branches join, which would
  // serialize the prefetch.
  auto in_list = [&](int k, int j) -> bool { return j < kStageJobs && e0 + kTile * k + (j & (kTile - 1)) < e1; };
  auto slot_of = [&](int k, int j) -> int {  // the list entry (clamped to the share's last entry)
    return idx_row[min(e0 + kTile * k + (j & (kTile - 1)), e1 - 1)];
  };
  auto load_stage = [&](int j, int slot, bool listed) -> Stage {
    Stage st;
    st.ok = listed && (unsigned)slot < (unsigned)p.num_slots;
    const int64_t row = st.ok ? slot : 0;
    const int c = min(j / kTile, kChunks - 1);
    st.w = *reinterpret_cast<const uint4*>(p.codes + row * kMlaRowCodeBytes + 16 * c);
    st.s = *reinterpret_cast<const uint16_t*>(p.scales + row * kMlaRowScaleBytes + 2 * c);
    return st;
  };
  auto write_stage = [&](int buf, int j, const Stage& st) {
    if (j >= kStageJobs) return;
    const int e = j & (kTile - 1), c = j / kTile;
    const uint32_t sw = st.ok ? st.s : 0u;  // an entry outside the cache stages as zeros
    const half2_t s0 = e4m3_pair_to_f16_scaled(sw & 0xFFu, sw & 0xFFu);
    const half2_t s1 = e4m3_pair_to_f16_scaled((sw >> 8) & 0xFFu, (sw >> 8) & 0xFFu);
    const uint32_t w[4] = {st.ok ? st.w.x : 0u, st.ok ? st.w.y : 0u, st.ok ? st.w.z : 0u, st.ok ? st.w.w : 0u};
    _Float16* dst = &s_k[buf][e * kRow + 32 * c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // 8 values per code word: dims 32c + 8q .. +7
      const half2_t sc = q < 2 ? s0 : s1;
      const half2_t a0 = fp4x2_to_f16_x256<0>(w[q]) * sc;
      const half2_t a1 = fp4x2_to_f16_x256<1>(w[q]) * sc;
      const half2_t a2 = fp4x2_to_f16_x256<2>(w[q]) * sc;
      const half2_t a3 = fp4x2_to_f16_x256<3>(w[q]) * sc;
      const half8_t v = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      *reinterpret_cast<half8_t*>(dst + 8 * q) = v;
    }
    if (c == 0) s_valid[buf][e] = st.ok;
  };

  // ---- Q of this wave's 16 heads as the B operand: lane (head r, dims 32c + 8*g4 .. +7)
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)t * p.Hq + head0 + r) * kMlaDim + 8 * g4;
  uint4 qraw[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) qraw[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c);

  // prologue: slots of tiles 0 and 1, the rows of tile 0 into buffer 0 (an
  // empty share loads nothing: its list is not read)
  int slot_b[kPer];
  Stage st[kPer];
  if (n_tiles > 0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s0 = slot_of(0, tid + k * NT);
      slot_b[k] = slot_of(1, tid + k * NT);
      st[k] = load_stage(tid + k * NT, s0, in_list(0, tid + k * NT));
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      slot_b[k] = -1;
      st[k] = Stage{make_uint4(0u, 0u, 0u, 0u), 0u, 0};
    }
  }

  // |q| maximum straight from the bf16 bits (the magnitude order of finite
  // values is the order of their bit patterns without the sign)
  uint32_t qbits = 0u;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t w[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) qbits = max(qbits, max((w[j] << 16) & 0x7FFF0000u, w[j] & 0x7FFF0000u));
  }
  float qmax = __uint_as_float(qbits);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));  // wave maximum
  int qe = 0;
  (void)__builtin_frexpf(qmax, &qe);  // qmax < 2^qe
  // exact power of two with the logit scale's sign, so that tscale >= 0
  const float qscale = __builtin_copysignf(qmax > 0.0f ? __builtin_ldexpf(1.0f, 15 - qe) : 1.0f, p.qk_scale_log2);
  half8_t qa[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t w[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qa[c][2 * j] = (_Float16)(__uint_as_float(w[j] << 16) * qscale);
      qa[c][2 * j + 1] = (_Float16)(__uint_as_float(w[j] & 0xFFFF0000u) * qscale);
    }
  }
  const float tscale = fmaxf(p.qk_scale_log2 / qscale, __FLT_MIN__);

#pragma unroll
  for (int k = 0; k < kPer; ++k) write_stage(0, tid + k * NT, st[k]);
  __syncthreads();

  float m_run = -__FLT_MAX__, m_lim = -__FLT_MAX__, l_run = 0.0f;
  float4_t acc[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) acc[m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kBufs == 1 ? 0 : (kt & 1);
    // the next tile's rows go out before this tile is computed, the tile
    // after's slots too -- unconditionally (past the share's end the clamped
    // loads read valid memory and stage as zeros): a branch here would make the
    // compiler wait for every load in flight where the paths join
#pragma unroll
    for (int k = 0; k < kPer; ++k) st[k] = load_stage(tid + k * NT, slot_b[k], in_list(kt + 1, tid + k * NT));
#pragma unroll
    for (int k = 0; k < kPer; ++k) slot_b[k] = slot_of(kt + 2, tid + k * NT);

    // ---- S^T = K . Q^T for entries 0..15 (S0) and 16..31 (S1); lane (entries 4*g4 .. +3 of each, head r)
    const _Float16* kb = &s_k[buf][0];
    float4_t S0 = {0.0f, 0.0f, 0.0f, 0.0f}, S1 = {0.0f, 0.0f, 0.0f, 0.0f};
    {
      const _Float16* a0p = kb + r * kRow + 8 * g4;
      const _Float16* a1p = a0p + 16 * kRow;
      half8_t a0 = *reinterpret_cast<const half8_t*>(a0p), a1 = *reinterpret_cast<const half8_t*>(a1p);
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        // the next chunk's operands are read before this chunk's products
        half8_t n0 = a0, n1 = a1;
        if (c + 1 < kChunks) {
          n0 = *reinterpret_cast<const half8_t*>(a0p + 32 * (c + 1));
          n1 = *reinterpret_cast<const half8_t*>(a1p + 32 * (c + 1));
        }
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qa[c], S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qa[c], S1, 0, 0, 0);
        a0 = n0;
        a1 = n1;
      }
    }
    // the MFMA results are read by VALU next: 20 wait states cover the
    // write-to-read latency of MFMAs up to 16 passes
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(S0), "+v"(S1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!s_valid[buf][4 * g4 + i]) S0[i] = -__builtin_inff();
      if (!s_valid[buf][16 + 4 * g4 + i]) S1[i] = -__builtin_inff();
    }

    // ---- online softmax (log2 domain; tscale >= 0)
    const float pm = vmax_over_groups(vmax(vmax(vmax(S0[0], S0[1]), vmax(S0[2], S0[3])),
                                           vmax(vmax(S1[0], S1[1]), vmax(S1[2], S1[3])))) * tscale;
    if (__any(pm > m_lim)) {  // -inf (all masked) never moves the max
      const float m_new = fmaxf(m_run, pm);
      const float f = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float fj = __shfl(f, 4 * g4 + jj);  // head 4*g4 + jj of the accumulator rows
#pragma unroll
        for (int m = 0; m < 32; ++m) acc[m][jj] *= fj;
      }
      m_run = m_new;
      m_lim = m_new + kLazyMax;
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(S0[i] * tscale - m_run);
      pr[4 + i] = __builtin_amdgcn_exp2f(S1[i] * tscale - m_run);
    }
    l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    // P as an f16 hi + lo pair (about 22 bits); k-slot 8*g4 + j is entry 4*g4 + j (j < 4) or 16 + 4*g4 + j - 4
    half8_t ph, pl;
    // hi by the packed round-toward-zero conversion, lo = p - hi by the
    // mixed-precision FMA reading hi from the packed register (1.0 kept opaque
    // so that the FMA is not folded into a subtraction with separate conversions)
    float one = 1.0f;
    asm volatile("" : "+s"(one));
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pr[j], pr[j + 1]));
      ph[j] = h[0];
      ph[j + 1] = h[1];
      pl[j] = (_Float16)__builtin_fmaf(pr[j], one, -(float)h[0]);
      pl[j + 1] = (_Float16)__builtin_fmaf(pr[j + 1], one, -(float)h[1]);
    }

    // ---- O += P . V; V operand of dims 16m .. 16m+15: lane (dim 16m + r, entries 4*g4 .. +3 and
    // 16 + 4*g4 .. +3) by two transposing reads: lane q of the group addresses row 4*g4 + q/4
    // (and 16 rows further), dims 16m + 4*(q%4) .. +3
    typedef __attribute__((address_space(3))) const _Float16 lds_h;
    lds_h* vb0 = (lds_h*)(kb + (4 * g4 + (r >> 2)) * kRow + 4 * (r & 3));
    lds_h* vb1 = vb0 + 16 * kRow;
    auto vread = [&](int m) -> half8_t {
      const short4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vb0 + 16 * m));
      const short4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vb1 + 16 * m));
      return __builtin_bit_cast(half8_t, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // The next tile's staging (dequant VALU work and its LDS stores into the
    // other buffer) is spread between the PV MFMAs, which run asynchronously:
    // job k after output tile (k + 1) * (32 / kPer) - 1.
    constexpr int kAhead = 4;  // V operands in flight
    half8_t vq[kAhead];
#pragma unroll
    for (int m = 0; m < kAhead; ++m) vq[m] = vread(m);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const half8_t bv = vq[m % kAhead];
      if (m + kAhead < 32) vq[m % kAhead] = vread(m + kAhead);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv, acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bv, acc[m], 0, 0, 0);
      constexpr int kEvery = 32 / kPer;  // 32 / kEvery >= kPer slots
      if (kBufs == 2 && m % kEvery == kEvery - 1 && m / kEvery < kPer) write_stage(buf ^ 1, tid + (m / kEvery) * NT, st[m / kEvery]);
    }
    __syncthreads();
    if constexpr (kBufs == 1) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) write_stage(0, tid + k * NT, st[k]);
      __syncthreads();
    }
  }

  // ---- per-head totals: l over the 4 entry groups; each accumulator row i is head 4*g4 + i
  l_run = sum_over_groups(l_run);
  float m_row[4], l_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_row[i] = __shfl(m_run, 4 * g4 + i);
    l_row[i] = __shfl(l_run, 4 * g4 + i);
  }
  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = l_row[i] > 0.0f ? p.v_scale / l_row[i] : 0.0f;
      float* o = p.out + ((int64_t)t * p.Hq + head0 + 4 * g4 + i) * kMlaLatent + r;
#pragma unroll
      for (int m = 0; m < 32; ++m) o[16 * m] = acc[m][i] * inv;
    }
    return;
  }
  // ---- one share of a split list: store its partial (O unnormalised, max, sum)
  float* ps = p.part + ((int64_t)u * p.splits + sp) * kHeads * kMlaPartStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* row = ps + (16 * wave + 4 * g4 + i) * kMlaPartStride;
#pragma unroll
    for (int m = 0; m < 32; ++m) row[16 * m + r] = acc[m][i];
    if (r == 0) {
      row[kMlaLatent] = m_row[i];
      row[kMlaLatent + 1] = l_row[i];
    }
  }
}

// Merge of the shares of split lists: one thread per 4 output values of one
// (query token, head): the shares' (max, sum) and their 4 values of O.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaDecodeParams p, int heads_per_unit) {
  const int64_t job = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (token, head, 4 dims)
  if (job >= (int64_t)p.T * p.Hq * (kMlaLatent / 4)) return;
  const int d4 = (int)(job % (kMlaLatent / 4));
  const int64_t th = job / (kMlaLatent / 4);
  const int t = (int)(th / p.Hq), hq = (int)(th % p.Hq);
  const int hb = hq / heads_per_unit, h = hq - hb * heads_per_unit;
  const float* pu = p.part + (((int64_t)t * p.HB + hb) * p.splits * heads_per_unit + h) * kMlaPartStride;
  const int64_t share = (int64_t)heads_per_unit * kMlaPartStride;  // floats between two shares' rows
  float M = -__builtin_inff();
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, pu[s * share + kMlaLatent]);
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float L = 0.0f;
  for (int s = 0; s < p.splits; ++s) {
    const float* row = pu + s * share;
    const float f = exp2f(row[kMlaLatent] - M);  // a share without entries has max -FLT_MAX and sum 0
    const float4 o = *reinterpret_cast<const float4*>(row + 4 * d4);
    O.x += o.x * f;
    O.y += o.y * f;
    O.z += o.z * f;
    O.w += o.w * f;
    L += row[kMlaLatent + 1] * f;
  }
  const float inv = L > 0.0f ? p.v_scale / L : 0.0f;
  *reinterpret_cast<float4*>(p.out + th * kMlaLatent + 4 * d4) = make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
}

}  // namespace

hipError_t launch_mla_append(const MlaAppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t jobs = (int64_t)p.num_tokens * kChunks;
  const dim3 grid((unsigned)((jobs + 255) / 256));
  if (dtype == NVFP4_DTYPE_F32) hipLaunchKernelGGL(mla_append_kernel<float>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(mla_append_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

MlaGeometry mla_geometry(int32_t T, int32_t Hq, int32_t topk) {
  MlaGeometry geo{0, 0, 0, 0, 0};
  if (T <= 0 || Hq <= 0 || Hq % 16 != 0 || topk < 0) return geo;
  const int32_t waves = Hq >= 64 ? 4 : Hq / 16;
  if (Hq % (16 * waves) != 0) return geo;  // above 64 heads: a multiple of 64
  geo.waves = waves;
  geo.HB = Hq / (16 * waves);
  const int64_t units = (int64_t)T * geo.HB;
  // shares per unit: a wave for every SIMD of the 256 CUs (the kernel runs one
  // wave per SIMD), at least 256 list entries per share
  const int64_t unit_waves = units * waves;
  int64_t splits = unit_waves >= 1024 ? 1 : (1024 + unit_waves - 1) / unit_waves;
  const int64_t max_splits = topk / 256 > 1 ? topk / 256 : 1;
  if (splits > max_splits) splits = max_splits;
  int64_t per = topk > 0 ? (topk + splits - 1) / splits : kTile;
  per = (per + kTile - 1) / kTile * kTile;
  splits = topk > 0 ? (topk + per - 1) / per : 1;
  geo.splits = (int32_t)splits;
  geo.per_split = (int32_t)per;
  geo.workspace_bytes = splits > 1 ? (size_t)(units * splits * 16 * geo.waves * kMlaPartStride) * sizeof(float) : 0;
  return geo;
}

hipError_t launch_mla_decode(const MlaDecodeParams& p, int32_t waves, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)p.T * p.HB * p.splits));
  switch (waves) {
    case 1: hipLaunchKernelGGL(mla_decode_kernel<1>, grid, dim3(64), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(mla_decode_kernel<2>, grid, dim3(128), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(mla_decode_kernel<3>, grid, dim3(192), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(mla_decode_kernel<4>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t jobs = (int64_t)p.T * p.Hq * (kMlaLatent / 4);
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((jobs + 255) / 256)), dim3(256), 0, stream, p, 16 * waves);
  return hipGetLastError();
}

}  // namespace nvfp4kv
