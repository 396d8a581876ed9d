// Split-K paged decode attention over an NVFP4 cache, dequantizing in
// registers, for gfx950 (CDNA4, wave64, MFMA).
//
// grer.cn blog "NVFP4 KV cache and the memory wall", section 3, third data
// flow: decode reads the whole cache for one short query, so its speed is set
// by the cache read; the 4-bit values are widened where they are loaded and the
// block scale is applied in registers, with no separate dequantization pass.
// Section 1 of the same blog: grouped-query heads share one KV head.
//
// Work decomposition (stream-K over pages).  The (sequence, kv head, page)
// work of the whole call is laid out unit after unit -- unit u = b*H + h, in
// sequence order -- and the launch's workgroups (about one per CU) take equal
// contiguous shares of it, computed on the device from seq_lens, so ragged
// batches stay balanced.  A share may end inside a unit and start the next.
// Within a share, the 16 waves of a workgroup take pages w, w+16, ... of each
// unit segment; a wave's page indices sit in its lanes (read with readlane)
// and the next page's K/V bytes are loaded (raw buffer loads from a per-page
// SGPR descriptor) before the current page is computed.  Per page (16 tokens):
//   QK^T  S[16 tok x 16 q] = K_page[16 x 128] . Q^T : 4 x mfma_f32_16x16x32_f16
//         (A = K: lane (tok = l%16, k-group l/16) loads 16 contiguous code bytes =
//          dims 32*(l/16)..+31 of its token; B = Q, the same dims, in registers)
//   online softmax in fp32 (exp2 domain), with a lazy max: the running max is
//         only raised when a page exceeds it by more than 2^8, so P <= 2^8;
//         row maxima across the 4 token groups use v_permlane16/32_swap
//   PV    O[16 q x 128] += P[16 x 16 tok] . V_page : 16 x mfma_f32_16x16x16f16
//         (the QK^T output lane layout is exactly the PV A-operand layout; P
//          enters as an f16 hi + lo pair, one MFMA each against the same V
//          operand; the V tile gives lane l the 4 tokens 4*(l/16)..+3 of dims
//          8*(l%16)..+7 in 16 contiguous bytes, each byte one dimension of two
//          neighbouring tokens, so one conversion yields one MFMA k-pair)
// Dequantization: v_cvt_scalef32_pk_f16_fp4 widens two E2M1 codes, and one
// v_pk_mul_f16 by the E4M3 scale pair gives e2m1 * bs exactly in f16 (at most
// 6 significant bits, magnitude in [2^-10, 2688]).  K: the codes times 2^8 and
// the scale byte's bit pattern << 7 as f16 (bs * 2^-8), one pair per block;
// V: two tokens' scale bytes widened by v_cvt_scalef32_pk_f16_fp8 (exact).
// The FP32 global scales are applied to the
// logits (K) and to the final output (V).  Q is converted to f16 after an
// exact power-of-two prescale (float32 Q: as an f16 hi + lo pair).
// MXFP4 planes (kMX; E8M0 scale per 32 values, the format the NVFP4 pages
// compare against): a lane's K bytes are one whole 32-value block, so
// v_cvt_scalef32_pk_bf16_fp4 takes the block's E8M0 byte as its scale operand
// and returns the exact value in bf16 (every E2M1 code times 2^-127 .. 2^125
// is a bf16 number; f16 has too few exponent bits).  V is converted per token
// with that token's scale and re-paired by token with v_perm_b32.  QK^T and PV
// run on the bf16 MFMAs; P enters as a bf16 hi + lo pair filling the k = 32
// operand of one 16x16x32 MFMA (the same issue cost as 16x16x16 on gfx950).
// The waves merge their (max, sum, O) in LDS.  A workgroup that covered a whole
// unit writes its normalised output; otherwise it stores an unnormalised
// partial and bumps the unit's arrival counter, and the workgroup that arrives
// last merges the unit's partials, writes the output and resets the counter
// (no second kernel; agent-scope stores and loads keep the partials coherent
// across the XCDs' separate L2 caches).
#include <type_traits>

#include "nvfp4_quant_device.h"

namespace nvfp4kv {
namespace {

#ifndef NVFP4_DECODE_GROUPS
#define NVFP4_DECODE_GROUPS 256
#endif
// One 16-wave workgroup fills a CU (4 waves per SIMD at <= 128 VGPRs); the
// launch has one workgroup per CU (fewer for tiny calls).
constexpr int kWaves = 16;                                  // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int64_t kMaxGroups = NVFP4_DECODE_GROUPS;         // workgroups per call
constexpr int kMaxPagesPerWave = 128;                       // page indices a wave keeps in 2 lane registers
constexpr int kChunkPages = kMaxPagesPerWave * kWaves;      // pages of one unit a workgroup loads indices for at once
constexpr int kPartStride = kHeadDim + 2;                   // floats per (partial slot, q head)
constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max must move

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// An E8M0 byte as the f32 scale operand of the scaled conversions: the
// conversion takes the operand's exponent field as the power of two, so the
// byte goes there (byte 0 means 2^-127; every byte and E2M1 code was checked
// exact against c * 2^(byte - 127) on gfx950).
__device__ __forceinline__ float e8m0_f32(uint32_t b) { return __uint_as_float(b << 23); }

// MXFP4 byte SEL of w (two E2M1 codes, low nibble first) times 2^(e - 127) as two bf16, in one word.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
// f32 pair -> bf16 pair (round to nearest even), and the bf16 values back as f32.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Cross-lane max/sum over lanes l, l^16, l^32, l^48 (the 4 token groups of one
// query head) with the gfx950 row/half swaps: with both operands equal,
// permlane16_swap returns (row 2k, row 2k+1) values and permlane32_swap the
// (low half, high half) values.
// IEEE maximum (v_maximum3_f32 on gfx950): NaN-propagating, so the compiler
// adds no quieting copies around it as it does for fmaxf; the operands here
// are finite scores or -inf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float vmax_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
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

// Q of one lane: dims 32*q4 .. 32*q4+31 of the query row that starts `row_off`
// elements after the sequence's first query element `seq_base`; row_off < 0
// reads as 0 (past the buffer range).  The raw words are loaded first and
// widened later, so other loads can be issued in between.
template <bool QF32>
struct QRaw {
  uint4 w[QF32 ? 8 : 4];
};

template <bool QF32>
__device__ __forceinline__ QRaw<QF32> load_q_raw(const void* q, int64_t seq_base, int seq_elems, int row_off, int q4) {
  constexpr int esz = QF32 ? 4 : 2;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(q) + seq_base * esz), 0, seq_elems * esz, 0x00020000);
  const int off = row_off >= 0 ? (row_off + 32 * q4) * esz : seq_elems * esz;
  QRaw<QF32> r;
#pragma unroll
  for (int i = 0; i < (QF32 ? 8 : 4); ++i)
    r.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0));
  return r;
}

template <bool QF32>
__device__ __forceinline__ void widen_q(const QRaw<QF32>& r, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < (QF32 ? 8 : 4); ++i) {
    const uint32_t w[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (QF32) {
        v[4 * i + j] = __uint_as_float(w[j]);
      } else {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
}

// Q for a cache of Hadamard-rotated K: q' = H q / 8 (H the 128-point Sylvester
// matrix, so q'.k' = q.k for k' = H k / 16).  The lane holds dims 32*q4 + j:
// fast Walsh-Hadamard stages over j in registers, then over q4 with the lanes
// l ^ 16 and l ^ 32 (fp32: Q feeds only the scores, not a rounding decision).
__device__ __forceinline__ void hadamard_rotate_q(float (&v)[32], int q4) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float o = __shfl_xor(v[i], 16);
    v[i] = (q4 & 1) ? o - v[i] : v[i] + o;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float o = __shfl_xor(v[i], 32);
    v[i] = ((q4 & 2) ? o - v[i] : v[i] + o) * 0.125f;
  }
}

// The bytes one lane needs from one (page, kv head) tile, and the number of
// valid tokens in that page (0 for an out-of-range page index).
struct PageRegs {
  uint4 kw;      // K codes: token r, dims 32*q4 .. 32*q4+31
  uint32_t ksw;  // K scales: token r, blocks 2*q4, 2*q4+1 (MXFP4: block q4)
  uint4 vw;      // V codes, dims 8*r .. 8*r+7: even and odd dims of tokens 4*q4 + {0,1}, then of + {2,3}
  uint32_t vsw;  // V scales: block r/2 (MXFP4: r/4), tokens 4*q4 .. 4*q4+3
};

// Raw buffer loads from a per-page descriptor: the page's base address lives
// in SGPRs and each lane's offset inside the tile never changes, so the page
// loop does no per-lane address arithmetic; reads past the descriptor's range
// return 0.
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer resource word 3 for raw dword access
// Cache policy of the page loads: every page is read once per call, so the
// loads are non-temporal (gfx950 buffer-load aux bit 1, nt): streaming reads
// that do not displace reused data measured clearly faster than default loads.
#ifndef NVFP4_PAGE_LOAD_AUX
#define NVFP4_PAGE_LOAD_AUX 2
#endif
constexpr int kPageAux = NVFP4_PAGE_LOAD_AUX;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int64_t offset, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + offset), 0, bytes, kBufferFlags);
}

struct LaneOffsets {
  int kc, ks, vc, vs;
};

// The four planes' descriptors.  kPlane: one descriptor per plane for the
// whole call and the tile's offset in an SGPR (planes below 4 GiB); otherwise
// a descriptor per tile.
struct PlaneRsrc {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;
};

template <bool kPlane, bool kMX>
__device__ __forceinline__ PlaneRsrc plane_rsrc(const DecodeParams& p) {
  constexpr int kScaleBytes = kMX ? kMxTileScaleBytes : kTileScaleBytes;
  PlaneRsrc r;
  if (kPlane) {
    const int64_t tiles = (int64_t)p.num_pages * p.H;
    r.kc = tile_rsrc(p.k_codes, 0, (int)(uint32_t)(tiles * kTileCodeBytes));
    r.ks = tile_rsrc(p.k_scales, 0, (int)(uint32_t)(tiles * kScaleBytes));
    r.vc = tile_rsrc(p.v_codes, 0, (int)(uint32_t)(tiles * kTileCodeBytes));
    r.vs = tile_rsrc(p.v_scales, 0, (int)(uint32_t)(tiles * kScaleBytes));
  }
  return r;
}

template <bool kPlane, bool kMX>
__device__ __forceinline__ PageRegs load_page(const DecodeParams& p, const PlaneRsrc& pr, int page, int h,
                                              const LaneOffsets& lo) {
  constexpr int kScaleBytes = kMX ? kMxTileScaleBytes : kTileScaleBytes;
  const bool ok = (unsigned)page < (unsigned)p.num_pages;
  PageRegs d;
  if (kPlane) {
    const uint32_t tile = (uint32_t)(ok ? page : 0) * (uint32_t)p.H + (uint32_t)h;
    const int so_c = (int)(tile * kTileCodeBytes), so_s = (int)(tile * kScaleBytes);
    d.kw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr.kc, lo.kc, so_c, kPageAux));
    d.ksw = kMX ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(pr.ks, lo.ks, so_s, kPageAux)
                : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(pr.ks, lo.ks, so_s, kPageAux);
    d.vw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pr.vc, lo.vc, so_c, kPageAux));
    d.vsw = __builtin_amdgcn_raw_buffer_load_b32(pr.vs, lo.vs, so_s, kPageAux);
  } else {
    const int64_t tile = (int64_t)(ok ? page : 0) * p.H + h;
    const auto kc = tile_rsrc(p.k_codes, tile * kTileCodeBytes, kTileCodeBytes);
    const auto ks = tile_rsrc(p.k_scales, tile * kScaleBytes, kScaleBytes);
    const auto vc = tile_rsrc(p.v_codes, tile * kTileCodeBytes, kTileCodeBytes);
    const auto vs = tile_rsrc(p.v_scales, tile * kScaleBytes, kScaleBytes);
    d.kw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, lo.kc, 0, kPageAux));
    d.ksw = kMX ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(ks, lo.ks, 0, kPageAux)
                : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ks, lo.ks, 0, kPageAux);
    d.vw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vc, lo.vc, 0, kPageAux));
    d.vsw = __builtin_amdgcn_raw_buffer_load_b32(vs, lo.vs, 0, kPageAux);
  }
  return d;
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for this wave's outstanding vector memory operations (vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// A value every lane of the wave holds (read from LDS): keep it in an SGPR.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Decode step with its own append: the step's NT new tokens of unit (b, h)
// sit at positions sl-NT .. sl-1.  The wave that owns the page holding some of
// them in this segment quantizes and stores them (the exact quantizer of
// quantize-on-append) before it loads any page, and waits for the stores; no
// other wave or workgroup reads that page, so nothing waits across waves.
// k_new / v_new are [B][NT][H][128] in the query's dtype.
template <bool QF32>
__device__ __forceinline__ void append_own_tokens(const DecodeParams& p, int b, int h, int NT, int sl, int seg_begin,
                                                  int seg_end, int wave, int lane) {
  if (sl <= 0) return;
  const int first = max(sl - NT, 0);  // first new position
  for (int pg = first / kPageSize; pg <= (sl - 1) / kPageSize; ++pg) {  // at most 2 pages (NT <= 16)
    if (pg < seg_begin || pg >= seg_end || (pg - seg_begin) % kWaves != wave) continue;  // not this wave's page
    const int page = __builtin_amdgcn_readfirstlane(p.block_table[(int64_t)b * p.bt_stride + pg]);
    if ((unsigned)page >= (unsigned)p.num_pages) continue;  // a bad page index is skipped, as in quantize-on-append
    const int t_lo = max(first, kPageSize * pg), t_hi = min(sl, kPageSize * pg + kPageSize);
    for (int j = lane; j < (t_hi - t_lo) * 16; j += 64) {  // (token, tensor, block) jobs
      const int pos = t_lo + (j >> 4), which = (j >> 3) & 1, blk = j & 7;
      const int64_t src = (((int64_t)b * NT + (pos - (sl - NT))) * p.H + h) * kHeadDim + 16 * blk;
      float x[16];
      if (QF32) load_block<float>(reinterpret_cast<const float*>(which ? p.v_new : p.k_new) + src, x);
      else load_block<uint16_t>(reinterpret_cast<const uint16_t*>(which ? p.v_new : p.k_new) + src, x);
      const float g = which ? p.v_global : p.k_global;
      const QuantBlock q = quantize_block16(x, g, 1.0 / (6.0 * (double)g));
      // V: a token's slot pair partner is either older (in the cache) or not
      // yet written, or another lane's job: each token sets its own nibbles
      if (which) store_v_alone(const_cast<uint8_t*>(p.v_codes), const_cast<uint8_t*>(p.v_scales), p.H,
                               page * kPageSize + pos % kPageSize, h, blk, q);
      else store_k_block(const_cast<uint8_t*>(p.k_codes), const_cast<uint8_t*>(p.k_scales), p.H,
                         page * kPageSize + pos % kPageSize, h, blk, q);
    }
  }
}

// kMulti: several query tokens per sequence (per-row causal limits); the
// one-token instance keeps the plain decode's code.  kAppend: the step's new
// tokens are appended by the kernel itself (append_own_tokens).  kMX: MXFP4
// planes (one-token decode only).  kRot: the cache holds Hadamard-rotated K,
// so Q is rotated the same way (one-token decode only); rotated Q is not exact
// in 16 bits, so it always takes the hi + lo split of float32 Q.
template <bool QF32, bool kPlane, bool kMulti, bool kAppend, bool kMX, bool kRot>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  constexpr bool kSplitQ = QF32 || kRot;
  __shared__ int s_pref[kMaxDecodeBatch + 1];  // exclusive prefix of pages per sequence
  __shared__ int s_wsum[kWaves];
  __shared__ int s_flag;
  __shared__ float s_o[kWaves][kMaxGroup][kHeadDim];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];

  const int wg = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets the page loop run on SGPRs
  const int lane = tid & 63;
  const int q4 = lane >> 4;
  const int B = p.batch, H = p.H, G = p.G;
  const int NT = kMulti ? p.T : 1, R = kMulti ? p.R : G;  // NT query tokens per sequence; R = G*NT query rows per unit
  // output row of query row r (token r / G, head r % G) of unit (b, h): out is [B][NT][Hq][128]
  auto out_row = [&](int b, int h, int r) -> int64_t {
    return kMulti ? ((int64_t)b * NT + r / G) * p.Hq + (int64_t)h * G + r % G : (int64_t)b * p.Hq + (int64_t)h * G + r;
  };
  const PlaneRsrc planes = plane_rsrc<kPlane, kMX>(p);

  // ---- pages of every sequence and their exclusive prefix sums (4 sequences per thread)
  int pg[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    const int len = b < B ? min(p.seq_lens[b], p.max_seq_len) : 0;
    pg[i] = len > 0 ? (len + kPageSize - 1) / kPageSize + kDecodeUnitCost : 0;  // slots of one unit
    local += pg[i];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int wave_off = 0, total_slots = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int v = uni(s_wsum[i]);
    wave_off += i < wave ? v : 0;
    total_slots += v;
  }
  {
    int excl = wave_off + incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * tid + i;
      if (b < B) s_pref[b] = excl;
      excl += pg[i];
    }
    if (tid == 0) s_pref[B] = total_slots;
  }
  __syncthreads();

  // ---- empty sequences: zero their outputs (spread over the workgroups)
  for (int b = wg; b < B; b += p.num_groups) {
    if (uni(s_pref[b + 1]) == uni(s_pref[b]))
      for (int e = tid; e < NT * p.Hq * kHeadDim; e += kThreads) p.out[(int64_t)b * NT * p.Hq * kHeadDim + e] = 0.0f;
  }

  // ---- this workgroup's share [x0, x1) of the flattened work.  Unit u = b*H+h
  // occupies kDecodeUnitCost + pages_b slots from S_u: the first slots stand
  // for the fixed cost of a unit segment (Q, pipeline fill, merges), page k is
  // slot S_u + kDecodeUnitCost + k, so shares balance cost, not just pages.
  // (The host keeps this index space below 2^30.)
  const uint32_t T = (uint32_t)(H * total_slots);
  if (T == 0) return;
  const uint32_t W = (T + p.num_groups - 1) / (uint32_t)p.num_groups;
  const uint32_t x0 = (uint32_t)wg * W;
  if (x0 >= T) return;
  const uint32_t x1 = min(x0 + W, T);

  // first sequence b with H*s_pref[b+1] > x0
  int lo_b = 0, hi_b = B - 1;
  while (lo_b < hi_b) {
    const int mid = (lo_b + hi_b) >> 1;
    if ((uint32_t)(H * uni(s_pref[mid + 1])) > x0) hi_b = mid; else lo_b = mid + 1;
  }
  int b = lo_b;
  int pref_b = uni(s_pref[b]);
  int slots_b = uni(s_pref[b + 1]) - pref_b;
  int h = (int)((x0 - (uint32_t)(H * pref_b)) / (uint32_t)slots_b);
  uint32_t x = x0;
  for (;; x = (uint32_t)(H * pref_b + h * slots_b) + slots_b) {  // x: first slot of the next unit
    if (x >= x1) break;
    if (x > x0) {  // move to the unit that starts at x
      if (++h == H) {
        h = 0;
        do {
          ++b;
          pref_b = uni(s_pref[b]);
          slots_b = uni(s_pref[b + 1]) - pref_b;
        } while (slots_b == 0);
      }
    }
    const int pages_b = slots_b - kDecodeUnitCost;
    const uint32_t S_u = (uint32_t)(H * pref_b + h * slots_b) + kDecodeUnitCost;  // slot of page 0
    const int seg_begin = x > S_u ? (int)(x - S_u) : 0;
    const int seg_end = x1 > S_u ? (int)min((uint32_t)pages_b, x1 - S_u) : 0;
    if (seg_end <= seg_begin) continue;  // the share holds only this unit's overhead slots

    // Lane indices pass through an empty asm at every segment, so addresses
    // derived from them are recomputed here instead of being hoisted out of
    // the segment loop and spilled across the page loop.
    int et = tid;
    asm volatile("" : "+v"(et));
    const int el = et & 63, er = et & 15, eq = (et >> 4) & 3;

    // The segment's independent loads go out together: Q, the first chunk's
    // page indices and the sequence length.
    // ---- Q as the B operand: lane (query row r = token i * G + head g of the group,
    // dims 32*q4 .. 32*q4+31); rows past R read as 0
    const int ti = kMulti ? er / G : 0, tg = kMulti ? er - (er / G) * G : er;
    const QRaw<QF32> q_raw = load_q_raw<QF32>(p.q, (int64_t)b * NT * p.Hq * kHeadDim, NT * p.Hq * kHeadDim,
                                              er < R ? (ti * p.Hq + h * G + tg) * kHeadDim : -1, eq);
    // this wave's pages of a chunk [c0, c1): pg_j = c0 + wave + kWaves*j, j < n_mine <= 128;
    // their indices sit in two lane registers (pages j and j + 64 in lane j), read
    // through a descriptor that ends at the chunk's end (entries past it read 0)
    const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
    int c0 = seg_begin;
    int c1 = min(c0 + kChunkPages, seg_end);
    int n_mine = c1 - c0 > wave ? (c1 - c0 - wave + kWaves - 1) / kWaves : 0;
    auto chunk_rsrc = [&](int c_end) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(bt_row), 0, 4 * c_end, kBufferFlags);
    };
    auto rs_bt = chunk_rsrc(c1);
    int pidx0 = __builtin_amdgcn_raw_buffer_load_b32(rs_bt, 4 * (c0 + wave + kWaves * el), 0, 0);
    int pidx1 = __builtin_amdgcn_raw_buffer_load_b32(rs_bt, 4 * (c0 + wave + kWaves * (el + 64)), 0, 0);
    const int len_v = __builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p.seq_lens), 0, 4 * B, kBufferFlags), 4 * b, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // all of them in flight before Q is used
    // Q, both page-index registers and the length complete (they were issued
    // together; the first page's loads need the indices anyway): the page loop
    // then reads page indices without waiting.  Otherwise the compiler cannot
    // tell at the loop head that the index loads are done and drains every
    // load in flight before each page's index read.
    wait_vmem();

    const LaneOffsets lo = kMX ? LaneOffsets{er * 64 + eq * 16, er * 4 + eq, el * 16, (er >> 2) * 16 + eq * 4}
                               : LaneOffsets{er * 64 + eq * 16, er * 8 + eq * 2, el * 16, (er >> 1) * 16 + eq * 4};
    auto page_of = [&](int j) {
      return j < 64 ? __builtin_amdgcn_readlane(pidx0, j) : __builtin_amdgcn_readlane(pidx1, j - 64);
    };
    // kAppend: a wave stores the new tokens of its pages, and its stores must
    // be complete before it loads one of those pages (pages >= new_pg).  The
    // append goes after the first page's loads unless that page is one of
    // them, and the wait is deferred to the first load of such a page.
    const int new_sl = kAppend ? min(uni(len_v), p.max_seq_len) : 0;
    const int new_pg = kAppend ? max(new_sl - NT, 0) / kPageSize : 0;
    bool stores_pending = false;
    auto load_mine = [&](int j) {
      const int jj = min(j, n_mine - 1);
      if (kAppend && stores_pending && c0 + wave + kWaves * jj >= new_pg) {
        wait_vmem();
        stores_pending = false;
      }
      return load_page<kPlane, kMX>(p, planes, page_of(jj), h, lo);
    };
    const bool append_first = kAppend && c0 + wave >= new_pg;
    if (append_first) {
      append_own_tokens<QF32>(p, b, h, NT, new_sl, seg_begin, seg_end, wave, el);
      stores_pending = true;
    }
    // the first page's loads go out before the Q conversion below
    PageRegs A;
    if (n_mine > 0) A = load_mine(0);
    __builtin_amdgcn_sched_barrier(0);
    if (kAppend && !append_first) {
      append_own_tokens<QF32>(p, b, h, NT, new_sl, seg_begin, seg_end, wave, el);
      stores_pending = true;
    }

    float qv[32];
    widen_q<QF32>(q_raw, qv);
    if constexpr (kRot) hadamard_rotate_q(qv, eq);
    float qmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qv[i]));
    qmax = max_over_groups(qmax);
#define NVFP4_SWZ(K) qmax = fmaxf(qmax, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(qmax), ((K) << 10) | 0x1F)));
    NVFP4_SWZ(1) NVFP4_SWZ(2) NVFP4_SWZ(4) NVFP4_SWZ(8)
#undef NVFP4_SWZ
    int qe = 0;
    (void)__builtin_frexpf(qmax, &qe);                                          // qmax < 2^qe
    // exact power of two, with the sign of the logit scale so that tscale >= 0
    // (then the page maximum can be taken on the raw scores)
    const float qscale = __builtin_copysignf(qmax > 0.0f ? __builtin_ldexpf(1.0f, 15 - qe) : 1.0f, p.qk_scale_log2);
    using QVec = std::conditional_t<kMX, bf16x8_t, half8_t>;
    using QElem = std::conditional_t<kMX, __bf16, _Float16>;
    QVec qa[4];
    QVec ql[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xq = qv[8 * c + j] * qscale;
        const QElem hq = (QElem)xq;
        qa[c][j] = hq;
        if (kSplitQ) ql[c][j] = (QElem)(xq - (float)hq);
      }
    // The lo half of split Q (float32 or rotated Q) waits in this wave's slot
    // of the merge buffer, free until the wave's own merge writes it after the
    // page loop (the end of every segment has a barrier): 16 fewer live
    // registers, which took the split instances from 19-23 spilled registers,
    // some reloaded in the page loop, to 7 (rotated decode 9-20% faster).
    uint8_t* ql_lds = reinterpret_cast<uint8_t*>(&s_o[wave][0][0]) + 16 * el;
    if constexpr (kSplitQ) {
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<QVec*>(ql_lds + 1024 * c) = ql[c];
    }
    // > 0: a zero logit scale becomes FLT_MIN (uniform weights to fp32
    // precision), so masked scores (-inf) always give weight exactly 0
    const float tscale = fmaxf(p.qk_scale_log2 / qscale, __FLT_MIN__);
    const int seq_len = min(uni(len_v), p.max_seq_len);

    // running max; -FLT_MAX stands for "none yet" (exp2 of anything minus it is 0)
    float m_run = -__FLT_MAX__;
    float m_lim = -__FLT_MAX__;  // m_run + kLazyMax: the max moves only above this
    float l_run = 0.0f;
    float4_t acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // rem: tokens of the sequence from this page's first slot on (0 for a page
    // index outside the cache); the page holds min(rem, 16) of them
    auto process = [&](const PageRegs& cur, int rem) {

      // ---- S^T = K . Q^T over the page; lane (q head r, tokens 4*q4 .. 4*q4+3)
      float4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint32_t kwa[4] = {cur.kw.x, cur.kw.y, cur.kw.z, cur.kw.w};
      if constexpr (kMX) {
        const float ksc = e8m0_f32(cur.ksw & 0xFFu);  // the lane's 32 dims are one block
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, make_uint4(fp4x2_to_bf16<0>(kwa[c], ksc), fp4x2_to_bf16<1>(kwa[c], ksc),
                                   fp4x2_to_bf16<2>(kwa[c], ksc), fp4x2_to_bf16<3>(kwa[c], ksc)));
          S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qa[c], S, 0, 0, 0);
          if (kSplitQ) S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *reinterpret_cast<const QVec*>(ql_lds + 1024 * c), S, 0, 0, 0);
        }
      } else {
        // the scale byte b as the f16 pair (b << 7, b << 7): one 24-bit multiply by 0x00800080 each
        const half2_t ks0 = __builtin_bit_cast(half2_t, (cur.ksw & 0xFFu) * 0x00800080u);
        const half2_t ks1 = __builtin_bit_cast(half2_t, ((cur.ksw >> 8) & 0xFFu) * 0x00800080u);
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const half2_t sc = c < 2 ? ks0 : ks1;
          const half2_t e0 = fp4x2_to_f16_x256<0>(kwa[c]) * sc;
          const half2_t e1 = fp4x2_to_f16_x256<1>(kwa[c]) * sc;
          const half2_t e2 = fp4x2_to_f16_x256<2>(kwa[c]) * sc;
          const half2_t e3 = fp4x2_to_f16_x256<3>(kwa[c]) * sc;
          const half8_t a = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qa[c], S, 0, 0, 0);
          if (kSplitQ) S = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, *reinterpret_cast<const QVec*>(ql_lds + 1024 * c), S, 0, 0, 0);
        }
      }
      // The MFMA result is read next, possibly across the partial-page branch;
      // the compiler's wait-state insertion missed that path (the first read
      // came a few cycles after the MFMA), so wait explicitly: 20 wait states
      // cover the write-to-VALU-read latency of MFMAs up to 16 passes.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(S));

      // ---- online softmax (log2 domain) on t = S * tscale (tscale >= 0, so the
      // maximum of t is the maximum of S times tscale).  Raw v_exp_f32: weights
      // below 2^-126 of the running max flush to 0, which f16 could not hold.
      if (rem - (NT - 1) < kPageSize) {  // tokens past the end of some query row (or a bad page index)
        // query token i of NT sits at position seq_len - NT + i: its row sees
        // NT-1-i fewer keys than the sequence holds
        const int r = threadIdx.x & 15;
        const int vlim = kMulti ? rem - (r < R ? NT - 1 - r / G : 0) : rem;  // keys of this page the lane's row sees
  #pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * q4 + i >= vlim) S[i] = -__builtin_inff();
      }
      // The lane's own 4 scores decide whether any head's maximum passes its
      // lazy bound; only then is the maximum over the 4 token groups taken
      // (tscale >= 0 and rounding are monotone, so the maximum of the scaled
      // scores is the scaled maximum; -inf: all masked).
      const float lm = vmax(vmax3(S[0], S[1], S[2]), S[3]) * tscale;
      if (__any(lm > m_lim)) {
        const float pm = vmax_over_groups(lm);
        const float m_new = fmaxf(m_run, pm);
        const float f = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= f;
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float fj = __shfl(f, 4 * q4 + jj);
  #pragma unroll
          for (int i = 0; i < 8; ++i) acc[i][jj] *= fj;
        }
        m_run = m_new;
        m_lim = m_new + kLazyMax;
      }
      float pr[4];
  #pragma unroll
      // the rounded product, as in the page maximum (not a fused multiply-add):
      // t - m_run <= kLazyMax then holds for every logit, however large
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(S[i] * tscale - m_run);
      l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      if constexpr (kMX) {
        // ---- O += P . V: A = (P hi | P lo) of tokens 4*q4 .. 4*q4+3, B = (V | V) of the same tokens
        const uint32_t h01 = bf16_pair(pr[0], pr[1]), h23 = bf16_pair(pr[2], pr[3]);
        const uint32_t l01 = bf16_pair(pr[0] - bf16_lo(h01), pr[1] - bf16_hi(h01));
        const uint32_t l23 = bf16_pair(pr[2] - bf16_lo(h23), pr[3] - bf16_hi(h23));
        const bf16x8_t pa8 = __builtin_bit_cast(bf16x8_t, make_uint4(h01, h23, l01, l23));
        // lane: token 4*q4 + i in word i (dims 8*r .. 8*r+7, block r/4); tokens past
        // the end get zero codes and scale 1, so stale bytes never reach the MFMA
        uint32_t vw[4] = {cur.vw.x, cur.vw.y, cur.vw.z, cur.vw.w};
        float vsc[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i) vsc[i] = e8m0_f32((cur.vsw >> (8 * i)) & 0xFFu);
        if (rem < kPageSize) {
          const int nv = min(max(rem - 4 * q4, 0), 4);
  #pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= nv) {
              vw[i] = 0u;
              vsc[i] = 1.0f;
            }
        }
  #define NVFP4_MX_PV_STEP(C)                                                                        \
    {                                                                                                \
      const uint32_t c0 = fp4x2_to_bf16<C>(vw[0], vsc[0]), c1 = fp4x2_to_bf16<C>(vw[1], vsc[1]);    \
      const uint32_t c2 = fp4x2_to_bf16<C>(vw[2], vsc[2]), c3 = fp4x2_to_bf16<C>(vw[3], vsc[3]);    \
      const uint32_t e01 = __builtin_amdgcn_perm(c1, c0, 0x05040100u);                               \
      const uint32_t o01 = __builtin_amdgcn_perm(c1, c0, 0x07060302u);                               \
      const uint32_t e23 = __builtin_amdgcn_perm(c3, c2, 0x05040100u);                               \
      const uint32_t o23 = __builtin_amdgcn_perm(c3, c2, 0x07060302u);                               \
      const bf16x8_t ve = __builtin_bit_cast(bf16x8_t, make_uint4(e01, e23, e01, e23));              \
      const bf16x8_t vo = __builtin_bit_cast(bf16x8_t, make_uint4(o01, o23, o01, o23));              \
      acc[2 * C] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa8, ve, acc[2 * C], 0, 0, 0);           \
      acc[2 * C + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa8, vo, acc[2 * C + 1], 0, 0, 0);   \
    }
        NVFP4_MX_PV_STEP(0)
        NVFP4_MX_PV_STEP(1)
        NVFP4_MX_PV_STEP(2)
        NVFP4_MX_PV_STEP(3)
  #undef NVFP4_MX_PV_STEP
        return;
      }
      // P as an f16 hi + lo pair (about 22 bits): with P alone in f16 (11
      // bits) a row whose output nearly cancels -- outliers of opposite sign
      // in a few tokens -- could miss 1e-3 relative to the row's largest value.
      // hi = p rounded toward zero to f16 (11 significant bits for p >= 2^-14),
      // lo = p - hi (exact in float32) rounded to f16, by the mixed-precision
      // FMA that reads hi from its packed register and writes f16 directly.
      // The multiplier 1.0 is opaque to the compiler, which would otherwise
      // fold the FMA into a subtraction with separate conversions.
      float one = 1.0f;
      asm volatile("" : "+s"(one));
      const half2_t h01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pr[0], pr[1]));
      const half2_t h23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pr[2], pr[3]));
      const half4_t ph = {h01[0], h01[1], h23[0], h23[1]};
      const half4_t pl = {(_Float16)__builtin_fmaf(pr[0], one, -(float)h01[0]),
                          (_Float16)__builtin_fmaf(pr[1], one, -(float)h01[1]),
                          (_Float16)__builtin_fmaf(pr[2], one, -(float)h23[0]),
                          (_Float16)__builtin_fmaf(pr[3], one, -(float)h23[1])};

      // ---- O += P . V over the page; lane (dims 8*r .. 8*r+7, tokens 4*q4 .. 4*q4+3).
      // 16x16x16 MFMAs, one for P hi and one for P lo against the same V
      // operand: no register copies of V (a 16x16x32 MFMA taking the pair
      // would need V twice in its operand).
      uint32_t vsw = cur.vsw;
      if (rem < kPageSize) {
        const int nv = min(max(rem - 4 * q4, 0), 4);
        vsw &= nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);  // zero the scales of tokens past the end
      }
      // scale bytes of tokens (0, 1) and (2, 3) -> exact f16 pairs
      const half2_t vs01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsw, 1.0f, false);
      const half2_t vs23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsw, 1.0f, true);
      // byte C of a word: dim 8r + 2C (E) or 8r + 2C + 1 (O) of two tokens
      const uint32_t E01 = cur.vw.x, O01 = cur.vw.y, E23 = cur.vw.z, O23 = cur.vw.w;
  #define NVFP4_PV_STEP(C)                                                                   \
    {                                                                                        \
      const half2_t a0 = fp4x2_to_f16<C>(E01) * vs01;                                        \
      const half2_t a1 = fp4x2_to_f16<C>(E23) * vs23;                                        \
      const half2_t b0 = fp4x2_to_f16<C>(O01) * vs01;                                        \
      const half2_t b1 = fp4x2_to_f16<C>(O23) * vs23;                                        \
      const half4_t ve = {a0[0], a0[1], a1[0], a1[1]};                                       \
      const half4_t vo = {b0[0], b0[1], b1[0], b1[1]};                                       \
      acc[2 * C] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, ve, acc[2 * C], 0, 0, 0);        \
      acc[2 * C + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vo, acc[2 * C + 1], 0, 0, 0); \
      acc[2 * C] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, ve, acc[2 * C], 0, 0, 0);        \
      acc[2 * C + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vo, acc[2 * C + 1], 0, 0, 0); \
    }
      NVFP4_PV_STEP(0)
      NVFP4_PV_STEP(1)
      NVFP4_PV_STEP(2)
      NVFP4_PV_STEP(3)
  #undef NVFP4_PV_STEP
    };

    while (true) {
      // tokens of the sequence from page j's first slot on, 0 for a page index
      // outside the cache (uniform)
      auto valid_of = [&](int j) {
        return (unsigned)page_of(j) < (unsigned)p.num_pages ? seq_len - (c0 + wave + kWaves * j) * kPageSize : 0;
      };
      // Two register sets, unrolled by two: each set is loaded one page ahead of
      // its use and refilled right after, so no register copy waits on a load in
      // flight (loads past the last page re-read that page).
      if (n_mine > 0) {
        for (int j = 0; j < n_mine; j += 2) {
          const PageRegs Bp = load_mine(j + 1);
          __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before any work on the current page
          process(A, valid_of(j));
          if (j + 1 >= n_mine) break;
          A = load_mine(j + 2);
          __builtin_amdgcn_sched_barrier(0);
          process(Bp, valid_of(j + 1));
        }
      }
      // next chunk of the segment (only units of more than kChunkPages pages)
      c0 = c1;
      if (c0 >= seg_end) break;
      c1 = min(c0 + kChunkPages, seg_end);
      n_mine = c1 - c0 > wave ? (c1 - c0 - wave + kWaves - 1) / kWaves : 0;
      rs_bt = chunk_rsrc(c1);
      pidx0 = __builtin_amdgcn_raw_buffer_load_b32(rs_bt, 4 * (c0 + wave + kWaves * el), 0, 0);
      pidx1 = __builtin_amdgcn_raw_buffer_load_b32(rs_bt, 4 * (c0 + wave + kWaves * (el + 64)), 0, 0);
      wait_vmem();  // both index registers complete before the page loop (see the segment's first chunk)
      if (n_mine > 0) A = load_mine(0);
    }

    // ---- per-wave totals: the sum over the 4 token groups
    l_run = sum_over_groups(l_run);

    // ---- merge the waves in LDS
    int mt = tid;
    asm volatile("" : "+v"(mt));
    const int mr = mt & 15, mq = (mt >> 4) & 3;
    if (mq == 0) {
      s_m[wave][mr] = m_run;
      s_l[wave][mr] = l_run;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 8; ++i) s_o[wave][4 * mq + jj][8 * mr + i] = acc[i][jj];
    __syncthreads();

    const int u = b * H + h;
    const bool whole = seg_begin == 0 && seg_end == pages_b;
    const int64_t slot = (int64_t)u + wg;
    for (int e = mt; e < R * kHeadDim; e += kThreads) {
      const int g = e >> 7, d = e & 127;  // g: query row of the unit
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
      float O = 0.0f, L = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {  // a wave without tokens has m = -FLT_MAX, O = L = 0
        const float f = exp2f(s_m[w][g] - M);
        O += s_o[w][g][d] * f;
        L += s_l[w][g] * f;
      }
      if (whole) {
        p.out[out_row(b, h, g) * kHeadDim + d] = L > 0.0f ? O / L * p.v_global : 0.0f;
      } else {
        float* ps = p.part + (slot * R + g) * kPartStride;
        store_coherent(ps + d, O);
        if (d == 0) {
          store_coherent(ps + kHeadDim, M);
          store_coherent(ps + kHeadDim + 1, L);
        }
      }
    }
    if (!whole) {
      // the unit's partials live in slots u + w' for the workgroups w' that share it
      const int w_first = (int)(S_u / W), w_last = (int)((S_u + pages_b - 1) / W);
      wait_vmem();  // this wave's partial stores are complete before the arrival is counted
      __syncthreads();
      if (tid == 0) {
        // release: the workgroup's partial stores (ordered before this by the
        // barrier) are visible at agent scope before the count moves; acquire:
        // the last arriver's loads below see every other workgroup's partials
        const int old = __hip_atomic_fetch_add(p.counters + u, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = old == w_last - w_first;
      }
      __syncthreads();
      if (uni(s_flag)) {  // every other share of this unit is stored: merge them all
        for (int e = mt; e < R * kHeadDim; e += kThreads) {
          const int g = e >> 7, d = e & 127;
          float M = -__builtin_inff();
          for (int w2 = w_first; w2 <= w_last; ++w2)
            M = fmaxf(M, load_coherent(p.part + (((int64_t)u + w2) * R + g) * kPartStride + kHeadDim));
          float O = 0.0f, L = 0.0f;
          for (int w2 = w_first; w2 <= w_last; ++w2) {
            const float* ps = p.part + (((int64_t)u + w2) * R + g) * kPartStride;
            const float f = exp2f(load_coherent(ps + kHeadDim) - M);
            O += load_coherent(ps + d) * f;
            L += load_coherent(ps + kHeadDim + 1) * f;
          }
          p.out[out_row(b, h, g) * kHeadDim + d] = L > 0.0f ? O / L * p.v_global : 0.0f;
        }
        if (tid == 0) __hip_atomic_store(p.counters + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // LDS is reused by the next segment

  }
}

}  // namespace

DecodeGeometry decode_geometry(int32_t batch, int32_t rows_per_unit, int32_t num_kv_heads, int32_t max_seq_len) {
  DecodeGeometry geo{0, 0, 0};
  if (batch <= 0 || num_kv_heads <= 0 || rows_per_unit <= 0) return geo;
  const int64_t max_pages = ((int64_t)max(max_seq_len, 0) + kPageSize - 1) / kPageSize;
  // about one CU per 64 pages of the largest possible call, at most one workgroup per CU
  int64_t groups = ((int64_t)batch * num_kv_heads * max_pages + 63) / 64;
  groups = groups < 1 ? 1 : (groups > kMaxGroups ? kMaxGroups : groups);
  geo.num_groups = (int32_t)groups;
  const int64_t units = (int64_t)batch * num_kv_heads;
  geo.counters_bytes = (size_t)((units * 4 + 255) / 256 * 256);
  geo.workspace_bytes = geo.counters_bytes + (size_t)((units + groups) * rows_per_unit * kPartStride * sizeof(float));
  return geo;
}

hipError_t launch_decode(const DecodeParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)p.num_groups);
  // one descriptor per plane when every tile offset fits the 32-bit buffer offset
  const bool plane = (int64_t)p.num_pages * p.H * kTileCodeBytes <= (int64_t)UINT32_MAX;
  const bool f32 = q_dtype == NVFP4_DTYPE_F32;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, p); };
  auto pick = [&](auto multi, auto append, auto mx, auto rot) {
    constexpr bool M = decltype(multi)::value, A = decltype(append)::value, X = decltype(mx)::value,
                   Q = decltype(rot)::value;
    if (f32 && plane) go(decode_kernel<true, true, M, A, X, Q>);
    else if (f32) go(decode_kernel<true, false, M, A, X, Q>);
    else if (plane) go(decode_kernel<false, true, M, A, X, Q>);
    else go(decode_kernel<false, false, M, A, X, Q>);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  const bool append = p.k_new != nullptr;
  if ((p.mx || p.rot_q) && (p.T != 1 || append)) return hipErrorInvalidValue;  // one-token decode only (host-checked)
  if (p.mx) {
    if (p.rot_q) pick(F_{}, F_{}, T_{}, T_{}); else pick(F_{}, F_{}, T_{}, F_{});
  } else if (p.rot_q) {
    pick(F_{}, F_{}, F_{}, T_{});
  } else if (p.T > 1) {
    if (append) pick(T_{}, T_{}, F_{}, F_{}); else pick(T_{}, F_{}, F_{}, F_{});
  } else {
    if (append) pick(F_{}, T_{}, F_{}, F_{}); else pick(F_{}, F_{}, F_{}, F_{});
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
