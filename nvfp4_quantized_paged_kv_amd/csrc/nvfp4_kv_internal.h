// Internal declarations shared by the host shim and the gfx950 kernels of the
// NVFP4 paged KV-cache library (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_kv.h"

namespace nvfp4kv {

// Cache geometry (fixed by the public header).
constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kTileCodeBytes = 1024;  // 16 tokens x 64 code bytes, per (page, kv head)
constexpr int kTileScaleBytes = 128;  // 16 tokens x 8 E4M3 scale bytes
constexpr int kMxTileScaleBytes = 64; // MXFP4: 16 tokens x 4 E8M0 scale bytes
constexpr int kMaxGroup = 16;         // query heads per kv head handled by one MFMA tile

// One tensor (K or V) of a quantize-append call.
struct AppendTensor {
  const void* x;         // [num_tokens][H][128], token stride `token_stride` elements
  uint8_t* codes;        // code plane
  uint8_t* scales;       // scale plane
  float g;               // FP32 global scale
  double r6;             // 1/(6g) rounded to float64
};

struct AppendParams {
  AppendTensor t[2];     // [0] = K (token-major tile layout), [1] = V (decode-friendly tile layout)
  const int32_t* slots;  // [num_tokens], or nullptr: slots of a decode step's new tokens (below)
  int64_t token_stride;
  int32_t num_tokens;
  int32_t H;
  int32_t num_pages;
  int32_t rot_k;         // 1: Hadamard-rotate K rows before quantization
  // decode-step slots (slots == nullptr): token t = b*step_T + i sits at
  // position min(seq_lens[b], max_seq_len) - step_T + i (skipped when
  // negative), in page block_table[b*bt_stride + position/16] (skipped when
  // outside the cache) -- the positions the fused decode step appends at
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t bt_stride;
  int32_t step_T;
  int32_t max_seq_len;
};

hipError_t launch_quantize_append(const AppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream);

// MXFP4 quantize-append: [0] = K, [1] = V, the NVFP4 code layouts with 64-byte scale tiles.
struct MxAppendParams {
  const void* x[2];      // [num_tokens][H][128], token stride `token_stride` elements
  uint8_t* codes[2];
  uint8_t* scales[2];
  const int32_t* slots;  // [num_tokens]
  int64_t token_stride;
  int32_t num_tokens;
  int32_t H;
  int32_t num_pages;
  int32_t rot_k;         // 1: Hadamard-rotate K rows before quantization
};

hipError_t launch_mx_append(const MxAppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream);

struct DecodeParams {
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const void* q;           // [B][T][Hq][128]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* part;             // [B*H + num_groups][R][128 + 2]: unnormalised O, running max (log2), sum
  int32_t* counters;       // [B*H] arrival counters of split sequences; zero between calls
  float* out;              // [B][T][Hq][128]
  int32_t num_pages;
  int32_t H;
  int32_t G;
  int32_t T;               // query tokens per sequence
  int32_t R;               // query rows per (sequence, kv head) unit: G * T <= 16
  int32_t Hq;
  int32_t batch;
  int32_t bt_stride;
  int32_t max_seq_len;
  int32_t num_groups;      // workgroups of the launch
  float qk_scale_log2;     // sm_scale * k_global * log2(e)
  float k_global;
  float v_global;
  const void* k_new;       // decode step with its own append: [B][T][H][128] new K (q dtype), else null
  const void* v_new;
  int32_t mx;              // 1: the planes hold MXFP4 (E8M0 per 32 values, 64-byte scale tiles)
  int32_t rot_q;           // 1: the cache holds Hadamard-rotated K; rotate Q the same way
};

constexpr int kMaxDecodeBatch = 4096;  // sequences per decode call (prefix sums kept in LDS)
// Decode work balancing: each (sequence, kv head) unit counts as this many
// extra pages, the fixed cost of processing a unit piece (Q setup, pipeline
// fill, merges), so a share of many short units holds fewer pages.
#ifndef NVFP4_DECODE_UNIT_COST
#define NVFP4_DECODE_UNIT_COST 96
#endif
constexpr int kDecodeUnitCost = NVFP4_DECODE_UNIT_COST;

// Launch geometry and workspace of a decode call (shared by the workspace
// query and the launch).  Workspace = counters (B*H int32, padded to 256 B)
// followed by the split partials.
struct DecodeGeometry {
  int32_t num_groups;
  size_t counters_bytes;
  size_t workspace_bytes;
};
DecodeGeometry decode_geometry(int32_t batch, int32_t rows_per_unit, int32_t num_kv_heads, int32_t max_seq_len);

hipError_t launch_decode(const DecodeParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream);

struct DequantWsParams {
  const uint8_t* codes[2];
  const uint8_t* scales[2];
  uint8_t* ws[2];
  float g[2];
  float ws_scale[2];
  const int32_t* block_table;
  const int32_t* prefix_lens;
  const int32_t* ws_offsets;
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t max_prefix_len;
  int32_t ws_capacity;
  int32_t H;
  int32_t num_pages;
};

hipError_t launch_dequant_ws(const DequantWsParams& p, hipStream_t stream);

// FP8 rows of new tokens (K and V) into a workspace pair.
struct Fp8RowsParams {
  const void* x[2];      // K, V: [num_tokens][H][128], token stride `token_stride` elements
  uint8_t* ws[2];        // [ws_capacity][H][128]
  float ws_scale[2];
  double ws_rcp[2];      // 1/ws_scale rounded to float64
  const int32_t* rows;   // [num_tokens] workspace row per token (< 0: skip)
  int64_t token_stride;
  int32_t num_tokens;
  int32_t H;
  int32_t ws_capacity;
};

hipError_t launch_fp8_rows(const Fp8RowsParams& p, nvfp4_dtype_t dtype, hipStream_t stream);

// Causal attention of extend / prefill chunks over FP8 workspace rows.
struct ExtendParams {
  const void* q;               // [num_q_tokens][Hq][128]
  float* out;                  // [num_q_tokens][Hq][128]
  const uint8_t* ws_k;         // [ws_capacity][H][128] E4M3
  const uint8_t* ws_v;
  const int32_t* q_offsets;    // [num_seqs + 1]
  const int32_t* ws_offsets;   // [num_seqs]
  const int32_t* prefix_lens;  // [num_seqs]
  int32_t num_q_tokens;
  int32_t Hq;
  int32_t H;
  int32_t G;
  int32_t num_seqs;
  int32_t max_chunk;
  int32_t ws_capacity;
  float qk_scale_log2;         // sm_scale * k_ws_scale * log2(e)
  float v_scale;               // v_ws_scale
  int32_t splits;              // workgroups sharing one tile's keys (1: no split, outputs written directly)
  float* part;                 // splits > 1: [splits][num_q_tokens][Hq][kExtPartStride] partials (O, max, sum)
};

constexpr int kExtMaxSplits = 256;      // the merge takes one split per thread of a 256-thread workgroup
constexpr int kExtMinShareKeys = 1024;  // fewest keys a split workgroup takes
constexpr int kExtPartStride = 132;     // floats per (split, query token, head) partial: O[128], max (log2), sum, 2 pad

// Workgroups per tile for the split extend (1: none) and its workspace bytes.
struct ExtendGeometry {
  int32_t splits;
  size_t workspace_bytes;
};
ExtendGeometry extend_geometry(nvfp4_dtype_t q_dtype, int32_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t max_chunk, int32_t max_prefix);

hipError_t launch_extend(const ExtendParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream);
// the split extend's merge of p.splits partials in p.part into p.out
hipError_t launch_extend_merge(const ExtendParams& p, hipStream_t stream);
// the extend in FP8 arithmetic (Q and the softmax weights in E4M3, FP8 MFMA)
ExtendGeometry extend_f8_geometry(int32_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                  int32_t max_chunk, int32_t max_prefix);
hipError_t launch_extend_f8(const ExtendParams& p, nvfp4_dtype_t q_dtype, hipStream_t stream);

}  // namespace nvfp4kv
