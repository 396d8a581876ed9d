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
// and writes 8 code bytes plus 1 scale byte (K), or with the neighbouring lane
// 16 code bytes and 2 scale bytes of two slots that share V bytes.  Lane order,
// fastest first: token within a group of 4, block, group of 4 within 16
// consecutive tokens, kv head, group of 16 tokens.  Sixteen consecutive tokens usually fill one page, so a
// 256-lane workgroup writes whole (page, kv head) tiles of two heads: its K and
// V code runs and its 128-B scale rows are complete lines written by one CU.
// A thread's input load never waits for its slot: the slot is checked at the
// store.  Plain appends take one job per thread and run at the rate of the
// memory system.  Bulk appends of Hadamard-rotated K, whose arithmetic is the
// limit, run on a grid the device holds at once, each thread walking jobs a
// grid-wide stride apart and loading the next pair's inputs before it
// quantizes the current pair.  A decode step that appends with this kernel
// passes no slot array: each new token's slot comes from the block table at
// the position the step gives it (step_slot).
//
// The block quantizer (exact E4M3 scale, E2M1 codes by the hardware
// conversion with an exact threshold fallback) is in nvfp4_quant_device.h,
// shared with the decode step that appends its own new tokens.
#include <algorithm>
#include <type_traits>

#include "nvfp4_quant_device.h"

namespace nvfp4kv {
namespace {

// Block index i of the flattened work -> (token t, kv head h, block b); t < 0 if past the end.
__device__ __forceinline__ void block_coords(int64_t i, const AppendParams& p, int64_t& t, int& h, int& b) {
  const int tq = (int)(i & 3), tg = (int)((i >> 5) & 3);
  b = (int)((i >> 2) & 7);
  // group of 16 tokens * H + kv head (< 2^31, checked by the host); the 64
  // jobs of a wave share it (jobs come in aligned runs of 128), so the
  // division below runs on the scalar unit
  const uint32_t gh = __builtin_amdgcn_readfirstlane((uint32_t)(i >> 7));
  h = (int)(gh % (uint32_t)p.H);
  t = 16 * (int64_t)(gh / (uint32_t)p.H) + 4 * tg + tq;
  if (t >= p.num_tokens) t = -1;
}

// The raw input words of one block (16 values): 32 B of bf16 or 64 B of f32.
template <typename InT>
struct RawBlock {
  uint4 w[sizeof(InT) == 2 ? 2 : 4];
};

template <typename InT>
__device__ __forceinline__ RawBlock<InT> load_raw(const InT* src) {
  RawBlock<InT> r;
#pragma unroll
  for (int i = 0; i < (sizeof(InT) == 2 ? 2 : 4); ++i) r.w[i] = reinterpret_cast<const uint4*>(src)[i];
  return r;
}

template <typename InT>
__device__ __forceinline__ void widen(const RawBlock<InT>& r, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < (sizeof(InT) == 2 ? 2 : 4); ++i) {
    const uint32_t w[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sizeof(InT) == 2) {
        x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        x[4 * i + j] = __uint_as_float(w[j]);
      }
    }
  }
}

// One job: its block coordinates, slot (stored only if live and inside the
// cache) and raw inputs.
template <typename InT>
struct Job {
  RawBlock<InT> raw;
  RawBlock<InT> side_raw;  // V jobs at a wave edge: the other-side token's block (see finish_job)
  int64_t t;
  int32_t slot;
  int32_t side_slot;       // that token's slot, -1 if there is none
  bool live;
  int h, b;
};

// Slot of new token t of a decode step (AppendParams, slots == nullptr), -1 to skip.
__device__ __forceinline__ int32_t step_slot(const AppendParams& p, int64_t t) {
  const int b = (int)(t / p.step_T), i = (int)(t - (int64_t)b * p.step_T);
  const int pos = min(p.seq_lens[b], p.max_seq_len) - p.step_T + i;
  if (pos < 0) return -1;
  const int page = p.block_table[(int64_t)b * p.bt_stride + pos / kPageSize];
  return (unsigned)page < (unsigned)p.num_pages ? page * kPageSize + pos % kPageSize : -1;
}

// The input load does not wait for the slot: a job past the end, or of a
// skipped token, loads token 0 (always in range) and is dropped at the store.
// Both loads are unconditional (no branch around them), so the compiler can
// count the memory operations in flight and wait only for the ones it needs.
// side: also load the slot and block of the token on the other side of the
// pair (see finish_job), issued with the job's own loads.
template <typename InT>
__device__ __forceinline__ Job<InT> fetch_job(const AppendParams& p, const AppendTensor& T, int64_t i, int64_t n_jobs,
                                              bool side = false) {
  Job<InT> j;
  int64_t t;
  block_coords(i < n_jobs ? i : 0, p, t, j.h, j.b);
  j.live = i < n_jobs && t >= 0;
  const int64_t tt = j.live ? t : 0;
  j.t = tt;
  j.slot = p.slots ? p.slots[tt] : step_slot(p, tt);  // issued first: waiting for it never waits for the inputs
  const InT* x = reinterpret_cast<const InT*>(T.x) + (int64_t)j.h * kHeadDim + 16 * j.b;
  j.raw = load_raw<InT>(x + tt * p.token_stride);
  j.side_slot = -1;
  if (side) {
    // unconditional (waiting for the slots before loading measured slower)
    const int64_t t2 = (tt & 1) ? tt + 1 : tt - 1;
    const bool in = t2 >= 0 && t2 < p.num_tokens;
    const int64_t tc = in ? t2 : tt;
    const int32_t s2 = p.slots ? p.slots[tc] : step_slot(p, tc);
    j.side_slot = in ? s2 : -1;
    j.side_raw = load_raw<InT>(x + tc * p.token_stride);
  }
  return j;
}

// Lanes whose other-side token (t - 1 for even t, t + 1 for odd t) lies in
// another wave: token 4*tg of an even group tg (lane < 32) and token 4*tg + 3
// of an odd one.
__device__ __forceinline__ bool edge_lane() {
  const int lane = threadIdx.x & 63, tq = lane & 3;
  return (tq == 0 && lane < 32) || (tq == 3 && lane >= 32);
}

// which (0 = K, 1 = V) is uniform across the wave, and every lane of the wave
// runs this (lanes without a live job hold token 0 and store nothing).  A V
// block shares its bytes with the same block of the slot's pair partner
// (slot ^ 1).  The path exchanges codes with lane l ^ 1, the job of the
// neighbouring token t ^ 1 (same kv head and block); when that token holds the
// partner slot, the two lanes write the pair's bytes with plain stores.  Else,
// when the token on the other side (t - 1 for even t, t + 1 for odd t) holds
// it -- a run of consecutive slots that starts at an odd slot -- the codes
// come from that token's lane when it is in the same wave (lane l ^ 3 within
// a group of 4 tokens, l -/+ 29 across the wave's two groups); at a wave edge
// this lane quantizes that token's block too (the bytes that token's own lane
// computes), from inputs loaded with its own when the job was fetched with
// `side`, else loaded here.  Either way it writes its half as above.
// Otherwise this slot's nibbles are set alone.
template <typename InT, bool kRotK, bool kSide>
__device__ __forceinline__ void finish_job(const Job<InT>& j, const AppendTensor& T, const AppendParams& p, int which) {
  float x[16];
  widen<InT>(j.raw, x);
  if (kRotK && which == 0) hadamard_rotate_k<16, 8>(x, j.b);
  const bool ok = j.live && j.slot >= 0 && (int64_t)j.slot < (int64_t)p.num_pages * kPageSize;
  if (which == 0) {
    if (ok) store_k_block(T.codes, T.scales, p.H, j.slot, j.h, j.b, quantize_block16(x, T.g, T.r6));
    return;
  }
  const QuantBlock q = quantize_block16(x, T.g, T.r6);
  // a partner needs this lane's packed word of its own parity: word 1 from an even slot, word 0 from an odd one
  const int32_t my_slot = ok ? j.slot : -1;
  const uint32_t my_word = (j.slot & 1) ? q.packed[0] : q.packed[1];
  const int32_t other_slot = (int32_t)swz_xor1((uint32_t)my_slot);
  const uint32_t other = swz_xor1(my_word);
  const uint32_t other_sb = swz_xor1(q.sb);
  const int lane = threadIdx.x & 63, tq = lane & 3;
  int src = (tq == 1 || tq == 2) ? (lane ^ 3) : (tq == 0 ? lane - 29 : lane + 29);
  const bool side_in_wave = src >= 0 && src < 64;
  src = side_in_wave ? src : lane;
  const int32_t side_slot = __shfl(my_slot, src);
  const uint32_t side = (uint32_t)__shfl((int)my_word, src);
  const uint32_t side_sb = (uint32_t)__shfl((int)q.sb, src);
  if (!ok) return;
  if (other_slot == (j.slot ^ 1)) {
    store_v_pair(T.codes, T.scales, p.H, j.slot, j.h, j.b, q, other, other_sb);
    return;
  }
  if (side_in_wave) {
    if (side_slot == (j.slot ^ 1)) store_v_pair(T.codes, T.scales, p.H, j.slot, j.h, j.b, q, side, side_sb);
    else store_v_alone(T.codes, T.scales, p.H, j.slot, j.h, j.b, q);
    return;
  }
  const int64_t t2 = (j.t & 1) ? j.t + 1 : j.t - 1;
  RawBlock<InT> raw2 = j.side_raw;
  int32_t slot2 = j.side_slot;
  if (!kSide && t2 >= 0 && t2 < p.num_tokens) {
    slot2 = p.slots ? p.slots[t2] : step_slot(p, t2);
    if (slot2 == (j.slot ^ 1))
      raw2 = load_raw<InT>(reinterpret_cast<const InT*>(T.x) + t2 * p.token_stride + (int64_t)j.h * kHeadDim + 16 * j.b);
  }
  if (slot2 == (j.slot ^ 1)) {
    float x2[16];
    widen<InT>(raw2, x2);
    const QuantBlock q2 = quantize_block16(x2, T.g, T.r6);
    store_v_pair(T.codes, T.scales, p.H, j.slot, j.h, j.b, q, (j.slot & 1) ? q2.packed[1] : q2.packed[0], q2.sb);
    return;
  }
  store_v_alone(T.codes, T.scales, p.H, j.slot, j.h, j.b, q);
}

// One job per thread: a single load, quantize and store chain per thread.
// kRotK: K rows are Hadamard-rotated before quantization (the 8 blocks of a
// row sit in lanes l, l^4, .., l^28, so every lane of a 32-lane group takes
// part in the exchanges; idle lanes hold token 0 and skip the store).
template <typename InT, bool kRotK>
__global__ __launch_bounds__(256) void quantize_append_kernel(AppendParams p, int64_t n_jobs) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const AppendTensor& T = p.t[which];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_jobs) return;
  finish_job<InT, kRotK, true>(fetch_job<InT>(p, T, i, n_jobs, which == 1 && edge_lane()), T, p, which);
}

// Bulk rotated-K appends: a fixed grid of what the device holds at once walks the
// jobs with a stride that is a multiple of 128 (whole 16-token groups of one
// head, so every pass keeps the page-tile lane pattern), two jobs per step,
// and loads the next step's inputs before it quantizes the current ones, so
// each wave keeps reads in flight while it computes.  All lanes of a wave see
// the same trip count (jobs come in aligned groups of 128), so the lane
// exchanges of the rotated-K path stay uniform.
template <typename InT, bool kRotK>
__global__ __launch_bounds__(256) void quantize_append_stream_kernel(AppendParams p, int64_t n_jobs) {
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const AppendTensor& T = p.t[which];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_jobs) return;
  // two register sets, each loaded a step ahead of its use and consumed in
  // place (a copy of a set in flight would wait for its loads)
  Job<InT> a0 = fetch_job<InT>(p, T, i, n_jobs);
  Job<InT> a1 = fetch_job<InT>(p, T, i + stride, n_jobs);
  while (true) {
    const Job<InT> b0 = fetch_job<InT>(p, T, i + 2 * stride, n_jobs);
    const Job<InT> b1 = fetch_job<InT>(p, T, i + 3 * stride, n_jobs);
    finish_job<InT, kRotK, false>(a0, T, p, which);
    finish_job<InT, kRotK, false>(a1, T, p, which);
    if (i + 2 * stride >= n_jobs) break;  // uniform across the wave
    a0 = fetch_job<InT>(p, T, i + 4 * stride, n_jobs);
    a1 = fetch_job<InT>(p, T, i + 5 * stride, n_jobs);
    finish_job<InT, kRotK, false>(b0, T, p, which);
    finish_job<InT, kRotK, false>(b1, T, p, which);
    i += 4 * stride;
    if (i >= n_jobs) break;
  }
}

// blocks (16 values of one token and head) from which an append counts as bulk
constexpr int64_t kAppendBulkBlocks = 1 << 18;

// Workgroups of one tensor's streaming grid: half of what the device holds at
// once (K and V share the launch), so no workgroup waits for another to end.
template <typename Kernel>
hipError_t stream_groups(Kernel kernel, int64_t n_blocks, int64_t& groups) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
  if (e != hipSuccess) return e;
  groups = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * per_cu / 2, (n_blocks + 255) / 256));
  return hipSuccess;
}

}  // namespace

hipError_t launch_quantize_append(const AppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream) {
  // jobs: one per 16-value block, tokens rounded up to whole groups of 16 (a
  // multiple of 128 jobs, one group of one head)
  const int64_t n_blocks = (int64_t)((p.num_tokens + 15) / 16) * 16 * p.H * 8;
  if (n_blocks == 0) return hipSuccess;
  hipError_t err = hipSuccess;
  auto go = [&](auto in, auto rot) {
    using InT = decltype(in);
    constexpr bool K = decltype(rot)::value;
    if (K && n_blocks >= kAppendBulkBlocks) {
      // the rotation's arithmetic is what limits a bulk rotated append: overlap it with the next loads
      int64_t groups = 0;
      err = stream_groups(quantize_append_stream_kernel<InT, K>, n_blocks, groups);
      if (err != hipSuccess) return;
      hipLaunchKernelGGL((quantize_append_stream_kernel<InT, K>), dim3((unsigned)groups, 2, 1), dim3(256), 0, stream, p,
                         n_blocks);
    } else {
      // plain appends run at the memory system's rate with one job per thread
      hipLaunchKernelGGL((quantize_append_kernel<InT, K>), dim3((unsigned)((n_blocks + 255) / 256), 2, 1), dim3(256), 0,
                         stream, p, n_blocks);
    }
  };
  const bool bf16 = dtype == NVFP4_DTYPE_BF16;
  if (p.rot_k) {
    if (bf16) go(uint16_t{}, std::true_type{}); else go(float{}, std::true_type{});
  } else {
    if (bf16) go(uint16_t{}, std::false_type{}); else go(float{}, std::false_type{});
  }
  return err != hipSuccess ? err : hipGetLastError();
}

}  // namespace nvfp4kv
