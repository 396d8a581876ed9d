// Host side of the C ABI declared in include/nvfp4_kv.h: argument validation
// (pure host code, before any HIP call) and kernel launches on the caller's
// stream.  The library allocates nothing and never synchronizes.
#include <cmath>
#include <cstdint>

#include "decode_noalloc.h"
#include "mla_internal.h"
#include "nvfp4_kv.h"
#include "nvfp4_kv_internal.h"

using namespace nvfp4kv;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// FP32 scales the exact-rounding arguments of the kernels cover.
bool scale_ok(float s) { return std::isfinite(s) && s >= 0x1p-100f && s <= 0x1p100f; }

nvfp4_status_t check_layer(const nvfp4_kv_layer_t* L) {
  if (L == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if (L->head_dim != kHeadDim || L->page_size != kPageSize) return NVFP4_ERR_UNSUPPORTED;
  if (!L->k_codes || !L->k_scales || !L->v_codes || !L->v_scales) return NVFP4_ERR_INVALID_ARGUMENT;
  if (L->num_pages <= 0 || L->num_kv_heads <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((int64_t)L->num_pages * kPageSize > INT32_MAX) return NVFP4_ERR_UNSUPPORTED;  // slots are int32
  if (!aligned(L->k_codes, 16) || !aligned(L->v_codes, 16) || !aligned(L->k_scales, 4) || !aligned(L->v_scales, 4))
    return NVFP4_ERR_UNSUPPORTED;
  if (!scale_ok(L->k_global) || !scale_ok(L->v_global)) return NVFP4_ERR_INVALID_ARGUMENT;
  return NVFP4_OK;
}

bool dtype_ok(nvfp4_dtype_t d) { return d == NVFP4_DTYPE_F32 || d == NVFP4_DTYPE_BF16; }

nvfp4_status_t check_mx_layer(const mxfp4_kv_layer_t* L) {
  if (L == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if (L->head_dim != kHeadDim || L->page_size != kPageSize) return NVFP4_ERR_UNSUPPORTED;
  if (!L->k_codes || !L->k_scales || !L->v_codes || !L->v_scales) return NVFP4_ERR_INVALID_ARGUMENT;
  if (L->num_pages <= 0 || L->num_kv_heads <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((int64_t)L->num_pages * kPageSize > INT32_MAX) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(L->k_codes, 16) || !aligned(L->v_codes, 16) || !aligned(L->k_scales, 4) || !aligned(L->v_scales, 4))
    return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

nvfp4_status_t from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

}  // namespace

extern "C" {

NVFP4_API const char* nvfp4_status_string(nvfp4_status_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported shape, layout or alignment";
    case NVFP4_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

nvfp4_status_t append_impl(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new, nvfp4_dtype_t dtype,
                           int32_t num_tokens, int64_t token_stride_elems, const int32_t* slot_mapping, void* stream,
                           bool rot_k) {
  const nvfp4_status_t st = check_layer(layer);
  if (st != NVFP4_OK) return st;
  if (!dtype_ok(dtype) || num_tokens < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return NVFP4_OK;
  if (!k_new || !v_new || !slot_mapping) return NVFP4_ERR_INVALID_ARGUMENT;
  if (token_stride_elems < (int64_t)layer->num_kv_heads * kHeadDim) return NVFP4_ERR_INVALID_ARGUMENT;
  // the kernel indexes (group of 16 tokens, kv head) pairs in 31 bits
  if (((int64_t)num_tokens + 15) / 16 * layer->num_kv_heads >= ((int64_t)1 << 31)) return NVFP4_ERR_UNSUPPORTED;
  const int64_t esize = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || (token_stride_elems * esize) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  AppendParams p;
  p.t[0] = AppendTensor{k_new, layer->k_codes, layer->k_scales, layer->k_global, 1.0 / (6.0 * (double)layer->k_global)};
  p.t[1] = AppendTensor{v_new, layer->v_codes, layer->v_scales, layer->v_global, 1.0 / (6.0 * (double)layer->v_global)};
  p.slots = slot_mapping;
  p.block_table = p.seq_lens = nullptr;
  p.bt_stride = p.step_T = p.max_seq_len = 0;
  p.token_stride = token_stride_elems;
  p.num_tokens = num_tokens;
  p.H = layer->num_kv_heads;
  p.num_pages = layer->num_pages;
  p.rot_k = rot_k ? 1 : 0;
  return from_hip(launch_quantize_append(p, dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_kv_quantize_append(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                  nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                  const int32_t* slot_mapping, void* stream) {
  return append_impl(layer, k_new, v_new, dtype, num_tokens, token_stride_elems, slot_mapping, stream, false);
}

NVFP4_API nvfp4_status_t nvfp4_kv_quantize_append_hadamard(const nvfp4_kv_layer_t* layer, const void* k_new,
                                                           const void* v_new, nvfp4_dtype_t dtype, int32_t num_tokens,
                                                           int64_t token_stride_elems, const int32_t* slot_mapping,
                                                           void* stream) {
  return append_impl(layer, k_new, v_new, dtype, num_tokens, token_stride_elems, slot_mapping, stream, true);
}

// The decode kernel indexes the (sequence, kv head, page) work of a call, plus
// kDecodeUnitCost slots per unit, in 32 bits.
static bool decode_size_ok(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t slots = ((int64_t)max_seq_len + kPageSize - 1) / kPageSize + kDecodeUnitCost;
  return (int64_t)batch * num_kv_heads * slots <= (int64_t)1 << 30;
}

NVFP4_API size_t nvfp4_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t max_seq_len) {
  return nvfp4_paged_decode_multi_workspace_bytes(batch, 1, num_q_heads, num_kv_heads, max_seq_len);
}

NVFP4_API size_t nvfp4_paged_decode_multi_workspace_bytes(int32_t batch, int32_t q_per_seq, int32_t num_q_heads,
                                                          int32_t num_kv_heads, int32_t max_seq_len) {
  if (batch < 0 || batch > kMaxDecodeBatch || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return 0;
  if (q_per_seq < 1 || num_q_heads % num_kv_heads != 0) return 0;
  if ((int64_t)(num_q_heads / num_kv_heads) * q_per_seq > kMaxGroup) return 0;
  if (!decode_size_ok(batch, num_kv_heads, max_seq_len)) return 0;
  return decode_geometry(batch, num_q_heads / num_kv_heads * q_per_seq, num_kv_heads, max_seq_len).workspace_bytes;
}

}  // extern "C"

namespace {

// Decode of q_per_seq query tokens per sequence (1 for plain decode); with
// k_new / v_new the kernel first appends the q_per_seq new tokens itself.
// A decode step whose units hold more pages than this appends its new tokens
// with the append kernel and then decodes (two launches); shorter ones append
// inside the decode kernel.  Measured on MI355X with clocks in their sustained
// state (B=32, 8 kv heads, 64 q heads, 1 new token per sequence): the fused
// step takes 21.7 / 18.0 / 25.0 / 39.1 / 66.7 us at 512 / 1K / 2K / 4K / 8K
// tokens against 21.9 / 18.6 / 24.7 / 36.5 / 60.2 us for two launches, and
// 235 vs 217 us at 128K, 466 vs 423 us at 2M: the fused kernel's page loop
// runs about 9% slower (cause not found: the loop's compute blocks and waits
// match the plain kernel's), which only the saved launch outweighs.
constexpr int64_t kStepFusedMaxPages = 64;

nvfp4_status_t decode_impl(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new, const void* q,
                           nvfp4_dtype_t q_dtype, int32_t batch, int32_t q_per_seq, int32_t num_q_heads,
                           const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                           int32_t max_seq_len, float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream, bool mx = false, bool rot_q = false, bool use_scratch = false) {
  const nvfp4_status_t st = check_layer(layer);
  if (st != NVFP4_OK) return st;
  if (!dtype_ok(q_dtype) || batch < 0 || q_per_seq < 1 || num_q_heads <= 0 || max_seq_len < 0)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_q_heads % layer->num_kv_heads != 0) return NVFP4_ERR_INVALID_ARGUMENT;
  const int64_t G = num_q_heads / layer->num_kv_heads;
  if (G * q_per_seq > kMaxGroup || batch > kMaxDecodeBatch) return NVFP4_ERR_UNSUPPORTED;
  if ((int64_t)q_per_seq * num_q_heads * kHeadDim * 4 >= ((int64_t)1 << 31)) return NVFP4_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!decode_size_ok(batch, layer->num_kv_heads, max_seq_len)) return NVFP4_ERR_UNSUPPORTED;
  if (batch == 0) return NVFP4_OK;
  if (!q || !block_table || !seq_lens || !out) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((int64_t)block_table_stride * kPageSize < (int64_t)max_seq_len || block_table_stride < 0)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16)) return NVFP4_ERR_UNSUPPORTED;
  if ((k_new == nullptr) != (v_new == nullptr)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return NVFP4_ERR_UNSUPPORTED;
  const int32_t R = (int32_t)(G * q_per_seq);
  const DecodeGeometry geo = decode_geometry(batch, R, layer->num_kv_heads, max_seq_len);
  if (use_scratch) {
    // the library's own scratch: fixed counter region, partials after it
    const int64_t units = (int64_t)batch * layer->num_kv_heads;
    if (units * 4 > (int64_t)kNoAllocCounterBytes ||
        geo.workspace_bytes - geo.counters_bytes > kNoAllocScratchBytes - kNoAllocCounterBytes)
      return NVFP4_ERR_WORKSPACE_TOO_SMALL;
  } else {
    if (workspace_bytes < geo.workspace_bytes) return NVFP4_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned(workspace, 256)) return NVFP4_ERR_INVALID_ARGUMENT;
  }
  const double qk = (double)sm_scale * (double)layer->k_global * 1.4426950408889634;  // log2(e)
  if (!std::isfinite(qk)) return NVFP4_ERR_INVALID_ARGUMENT;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (use_scratch) {  // every argument is checked above; the first HIP call comes here
    void* sp = nullptr;
    const hipError_t e = noalloc_scratch(&sp, hs);
    if (e != hipSuccess) return from_hip(e);
    workspace = sp;
  }
  const uint8_t* ws_base = static_cast<uint8_t*>(workspace);
  const size_t part_offset = use_scratch ? kNoAllocCounterBytes : geo.counters_bytes;
  DecodeParams p;
  p.k_codes = layer->k_codes;
  p.k_scales = layer->k_scales;
  p.v_codes = layer->v_codes;
  p.v_scales = layer->v_scales;
  p.q = q;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.counters = static_cast<int32_t*>(workspace);
  p.part = reinterpret_cast<float*>(const_cast<uint8_t*>(ws_base) + part_offset);
  p.out = out;
  p.num_pages = layer->num_pages;
  p.H = layer->num_kv_heads;
  p.G = (int32_t)G;
  p.T = q_per_seq;
  p.R = R;
  p.Hq = num_q_heads;
  p.batch = batch;
  p.bt_stride = block_table_stride;
  p.max_seq_len = max_seq_len;
  p.num_groups = geo.num_groups;
  p.qk_scale_log2 = (float)qk;
  p.k_global = layer->k_global;
  p.v_global = layer->v_global;
  p.k_new = k_new;
  p.v_new = v_new;
  p.mx = mx ? 1 : 0;
  p.rot_q = rot_q ? 1 : 0;
  if (k_new && ((int64_t)max_seq_len + kPageSize - 1) / kPageSize > kStepFusedMaxPages) {
    // every argument is checked above: append the step's new tokens, then decode
    AppendParams a;
    a.t[0] = AppendTensor{k_new, layer->k_codes, layer->k_scales, layer->k_global, 1.0 / (6.0 * (double)layer->k_global)};
    a.t[1] = AppendTensor{v_new, layer->v_codes, layer->v_scales, layer->v_global, 1.0 / (6.0 * (double)layer->v_global)};
    a.slots = nullptr;
    a.token_stride = (int64_t)layer->num_kv_heads * kHeadDim;
    a.num_tokens = batch * q_per_seq;
    a.H = layer->num_kv_heads;
    a.num_pages = layer->num_pages;
    a.rot_k = 0;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.bt_stride = block_table_stride;
    a.step_T = q_per_seq;
    a.max_seq_len = max_seq_len;
    const hipError_t e = launch_quantize_append(a, q_dtype, hs);
    if (e != hipSuccess) return from_hip(e);
    p.k_new = p.v_new = nullptr;
  }
  return from_hip(launch_decode(p, q_dtype, hs));
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn(const nvfp4_kv_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  return decode_impl(layer, nullptr, nullptr, q, q_dtype, batch, 1, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, sm_scale, out, workspace, workspace_bytes, stream);
}

NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_noalloc(const nvfp4_kv_layer_t* layer, const void* q,
                                                         nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                         const int32_t* block_table, int32_t block_table_stride,
                                                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                         float* out, void* stream) {
  return decode_impl(layer, nullptr, nullptr, q, q_dtype, batch, 1, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, sm_scale, out, nullptr, 0, stream, false, false, true);
}

NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_hadamard(const nvfp4_kv_layer_t* layer, const void* q,
                                                          nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                          const int32_t* block_table, int32_t block_table_stride,
                                                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                          float* out, void* workspace, size_t workspace_bytes,
                                                          void* stream) {
  return decode_impl(layer, nullptr, nullptr, q, q_dtype, batch, 1, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, sm_scale, out, workspace, workspace_bytes, stream, false, true);
}

NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_multi(const nvfp4_kv_layer_t* layer, const void* q,
                                                       nvfp4_dtype_t q_dtype, int32_t batch, int32_t q_per_seq,
                                                       int32_t num_q_heads, const int32_t* block_table,
                                                       int32_t block_table_stride, const int32_t* seq_lens,
                                                       int32_t max_seq_len, float sm_scale, float* out,
                                                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(layer, nullptr, nullptr, q, q_dtype, batch, q_per_seq, num_q_heads, block_table,
                     block_table_stride, seq_lens, max_seq_len, sm_scale, out, workspace, workspace_bytes, stream);
}

NVFP4_API nvfp4_status_t nvfp4_paged_decode_step(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                 const void* q, nvfp4_dtype_t dtype, int32_t batch, int32_t q_per_seq,
                                                 int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new)) return NVFP4_ERR_INVALID_ARGUMENT;
  return decode_impl(layer, k_new, v_new, q, dtype, batch, q_per_seq, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, sm_scale, out, workspace, workspace_bytes, stream);
}

NVFP4_API nvfp4_status_t nvfp4_dequant_to_fp8_workspace(const nvfp4_kv_layer_t* layer, const int32_t* block_table,
                                                        int32_t block_table_stride, int32_t num_seqs,
                                                        const int32_t* prefix_lens, const int32_t* ws_offsets,
                                                        int32_t max_prefix_len, float k_ws_scale, float v_ws_scale,
                                                        uint8_t* ws_k, uint8_t* ws_v, int32_t ws_capacity_tokens,
                                                        void* stream) {
  const nvfp4_status_t st = check_layer(layer);
  if (st != NVFP4_OK) return st;
  if (num_seqs < 0 || max_prefix_len < 0 || ws_capacity_tokens < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!scale_ok(k_ws_scale) || !scale_ok(v_ws_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || max_prefix_len == 0) return NVFP4_OK;
  if (!block_table || !prefix_lens || !ws_offsets || !ws_k || !ws_v) return NVFP4_ERR_INVALID_ARGUMENT;
  if (block_table_stride < 0 || (int64_t)block_table_stride * kPageSize < (int64_t)max_prefix_len)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(ws_k, 16) || !aligned(ws_v, 16)) return NVFP4_ERR_UNSUPPORTED;
  DequantWsParams p;
  p.codes[0] = layer->k_codes;
  p.codes[1] = layer->v_codes;
  p.scales[0] = layer->k_scales;
  p.scales[1] = layer->v_scales;
  p.ws[0] = ws_k;
  p.ws[1] = ws_v;
  p.g[0] = layer->k_global;
  p.g[1] = layer->v_global;
  p.ws_scale[0] = k_ws_scale;
  p.ws_scale[1] = v_ws_scale;
  p.block_table = block_table;
  p.prefix_lens = prefix_lens;
  p.ws_offsets = ws_offsets;
  p.bt_stride = block_table_stride;
  p.num_seqs = num_seqs;
  p.max_prefix_len = max_prefix_len;
  p.ws_capacity = ws_capacity_tokens;
  p.H = layer->num_kv_heads;
  p.num_pages = layer->num_pages;
  return from_hip(launch_dequant_ws(p, static_cast<hipStream_t>(stream)));
}

NVFP4_API nvfp4_status_t nvfp4_fp8_rows_to_workspace(const void* k_new, const void* v_new, nvfp4_dtype_t dtype,
                                                     int32_t num_tokens, int64_t token_stride_elems,
                                                     int32_t num_kv_heads, const int32_t* ws_rows, float k_ws_scale,
                                                     float v_ws_scale, uint8_t* ws_k, uint8_t* ws_v,
                                                     int32_t ws_capacity_tokens, void* stream) {
  if (!dtype_ok(dtype) || num_tokens < 0 || num_kv_heads <= 0 || ws_capacity_tokens < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!scale_ok(k_ws_scale) || !scale_ok(v_ws_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0 || ws_capacity_tokens == 0) return NVFP4_OK;
  if (!k_new || !v_new || !ws_rows || !ws_k || !ws_v) return NVFP4_ERR_INVALID_ARGUMENT;
  if (token_stride_elems < (int64_t)num_kv_heads * kHeadDim) return NVFP4_ERR_INVALID_ARGUMENT;
  const int64_t esize = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || (token_stride_elems * esize) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(ws_k, 16) || !aligned(ws_v, 16)) return NVFP4_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * num_kv_heads * 8 / 256 >= ((int64_t)1 << 31)) return NVFP4_ERR_UNSUPPORTED;  // grid size
  Fp8RowsParams p;
  p.x[0] = k_new;
  p.x[1] = v_new;
  p.ws[0] = ws_k;
  p.ws[1] = ws_v;
  p.ws_scale[0] = k_ws_scale;
  p.ws_scale[1] = v_ws_scale;
  p.ws_rcp[0] = 1.0 / (double)k_ws_scale;
  p.ws_rcp[1] = 1.0 / (double)v_ws_scale;
  p.rows = ws_rows;
  p.token_stride = token_stride_elems;
  p.num_tokens = num_tokens;
  p.H = num_kv_heads;
  p.ws_capacity = ws_capacity_tokens;
  return from_hip(launch_fp8_rows(p, dtype, static_cast<hipStream_t>(stream)));
}

namespace {
// Checks the extend arguments and fills p (splits = 1, no workspace).
// NVFP4_OK with *empty set: nothing to compute.
nvfp4_status_t extend_params(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t num_seqs, const int32_t* q_offsets,
                             const int32_t* ws_offsets, const int32_t* prefix_lens, int32_t max_chunk_len,
                             const uint8_t* ws_k, const uint8_t* ws_v, int32_t ws_capacity_tokens, float k_ws_scale,
                             float v_ws_scale, float sm_scale, float* out, ExtendParams& p, bool* empty) {
  *empty = false;
  if (!dtype_ok(q_dtype) || num_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_seqs < 0 ||
      max_chunk_len < 0 || ws_capacity_tokens < 0)
    return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads != 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_q_heads / num_kv_heads > kMaxGroup) return NVFP4_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535 || num_seqs > 65535) return NVFP4_ERR_UNSUPPORTED;  // grid dimensions
  if (!scale_ok(k_ws_scale) || !scale_ok(v_ws_scale) || !std::isfinite(sm_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  const double qk = (double)sm_scale * (double)k_ws_scale * 1.4426950408889634;  // log2(e)
  if (!std::isfinite(qk) || !std::isfinite((float)qk)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || max_chunk_len == 0 || num_q_tokens == 0) {
    *empty = true;
    return NVFP4_OK;
  }
  if (!q || !q_offsets || !ws_offsets || !prefix_lens || !ws_k || !ws_v || !out) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(ws_k, 16) || !aligned(ws_v, 16)) return NVFP4_ERR_UNSUPPORTED;
  p.q = q;
  p.out = out;
  p.ws_k = ws_k;
  p.ws_v = ws_v;
  p.q_offsets = q_offsets;
  p.ws_offsets = ws_offsets;
  p.prefix_lens = prefix_lens;
  p.num_q_tokens = num_q_tokens;
  p.Hq = num_q_heads;
  p.H = num_kv_heads;
  p.G = num_q_heads / num_kv_heads;
  p.num_seqs = num_seqs;
  p.max_chunk = max_chunk_len;
  p.ws_capacity = ws_capacity_tokens;
  p.qk_scale_log2 = (float)qk;
  p.v_scale = v_ws_scale;
  p.splits = 1;
  p.part = nullptr;
  return NVFP4_OK;
}
}  // namespace

NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                               const int32_t* q_offsets, const int32_t* ws_offsets,
                                               const int32_t* prefix_lens, int32_t max_chunk_len,
                                               const uint8_t* ws_k, const uint8_t* ws_v, int32_t ws_capacity_tokens,
                                               float k_ws_scale, float v_ws_scale, float sm_scale, float* out,
                                               void* stream) {
  ExtendParams p;
  bool empty = false;
  const nvfp4_status_t st = extend_params(q, q_dtype, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, q_offsets,
                                          ws_offsets, prefix_lens, max_chunk_len, ws_k, ws_v, ws_capacity_tokens,
                                          k_ws_scale, v_ws_scale, sm_scale, out, p, &empty);
  if (st != NVFP4_OK || empty) return st;
  return from_hip(launch_extend(p, q_dtype, static_cast<hipStream_t>(stream)));
}

NVFP4_API size_t nvfp4_fp8_extend_attn_split_workspace_bytes(nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                              int32_t num_q_heads, int32_t num_kv_heads,
                                                              int32_t num_seqs, int32_t max_chunk_len,
                                                              int32_t max_prefix_len) {
  if (!dtype_ok(q_dtype) || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > kMaxGroup)
    return 0;
  return extend_geometry(q_dtype, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_chunk_len, max_prefix_len)
      .workspace_bytes;
}

NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn_split(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                     const int32_t* q_offsets, const int32_t* ws_offsets,
                                                     const int32_t* prefix_lens, int32_t max_chunk_len,
                                                     int32_t max_prefix_len, const uint8_t* ws_k, const uint8_t* ws_v,
                                                     int32_t ws_capacity_tokens, float k_ws_scale, float v_ws_scale,
                                                     float sm_scale, float* out, void* workspace,
                                                     size_t workspace_bytes, void* stream) {
  if (max_prefix_len < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  ExtendParams p;
  bool empty = false;
  const nvfp4_status_t st = extend_params(q, q_dtype, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, q_offsets,
                                          ws_offsets, prefix_lens, max_chunk_len, ws_k, ws_v, ws_capacity_tokens,
                                          k_ws_scale, v_ws_scale, sm_scale, out, p, &empty);
  if (st != NVFP4_OK || empty) return st;
  const ExtendGeometry geo =
      extend_geometry(q_dtype, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_chunk_len, max_prefix_len);
  if (geo.splits > 1) {
    if (workspace_bytes < geo.workspace_bytes) return NVFP4_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 16)) return NVFP4_ERR_UNSUPPORTED;
    p.splits = geo.splits;
    p.part = static_cast<float*>(workspace);
  }
  return from_hip(launch_extend(p, q_dtype, static_cast<hipStream_t>(stream)));
}

NVFP4_API size_t nvfp4_fp8_extend_attn_f8_workspace_bytes(nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                           int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                           int32_t max_chunk_len, int32_t max_prefix_len) {
  if (!dtype_ok(q_dtype) || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > kMaxGroup)
    return 0;
  return extend_f8_geometry(num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_chunk_len, max_prefix_len)
      .workspace_bytes;
}

NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn_f8(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                  const int32_t* q_offsets, const int32_t* ws_offsets,
                                                  const int32_t* prefix_lens, int32_t max_chunk_len,
                                                  int32_t max_prefix_len, const uint8_t* ws_k, const uint8_t* ws_v,
                                                  int32_t ws_capacity_tokens, float k_ws_scale, float v_ws_scale,
                                                  float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                                  void* stream) {
  if (max_prefix_len < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  ExtendParams p;
  bool empty = false;
  const nvfp4_status_t st = extend_params(q, q_dtype, num_q_tokens, num_q_heads, num_kv_heads, num_seqs, q_offsets,
                                          ws_offsets, prefix_lens, max_chunk_len, ws_k, ws_v, ws_capacity_tokens,
                                          k_ws_scale, v_ws_scale, sm_scale, out, p, &empty);
  if (st != NVFP4_OK || empty) return st;
  const ExtendGeometry geo =
      extend_f8_geometry(num_q_tokens, num_q_heads, num_kv_heads, num_seqs, max_chunk_len, max_prefix_len);
  if (geo.splits > 1) {
    if (workspace_bytes < geo.workspace_bytes) return NVFP4_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace) return NVFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 16)) return NVFP4_ERR_UNSUPPORTED;
    p.splits = geo.splits;
    p.part = static_cast<float*>(workspace);
  }
  return from_hip(launch_extend_f8(p, q_dtype, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- MXFP4

}  // extern "C"

namespace {

nvfp4_status_t mx_append_impl(const mxfp4_kv_layer_t* layer, const void* k_new, const void* v_new, nvfp4_dtype_t dtype,
                              int32_t num_tokens, int64_t token_stride_elems, const int32_t* slot_mapping, void* stream,
                              bool rot_k) {
  const nvfp4_status_t st = check_mx_layer(layer);
  if (st != NVFP4_OK) return st;
  if (!dtype_ok(dtype) || num_tokens < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return NVFP4_OK;
  if (!k_new || !v_new || !slot_mapping) return NVFP4_ERR_INVALID_ARGUMENT;
  if (token_stride_elems < (int64_t)layer->num_kv_heads * kHeadDim) return NVFP4_ERR_INVALID_ARGUMENT;
  if (((int64_t)num_tokens + 15) / 16 * layer->num_kv_heads >= ((int64_t)1 << 31)) return NVFP4_ERR_UNSUPPORTED;
  const int64_t esize = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || (token_stride_elems * esize) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  MxAppendParams p;
  p.x[0] = k_new;
  p.x[1] = v_new;
  p.codes[0] = layer->k_codes;
  p.codes[1] = layer->v_codes;
  p.scales[0] = layer->k_scales;
  p.scales[1] = layer->v_scales;
  p.slots = slot_mapping;
    p.token_stride = token_stride_elems;
  p.num_tokens = num_tokens;
  p.H = layer->num_kv_heads;
  p.num_pages = layer->num_pages;
  p.rot_k = rot_k ? 1 : 0;
  return from_hip(launch_mx_append(p, dtype, static_cast<hipStream_t>(stream)));
}

nvfp4_status_t mx_decode_impl(const mxfp4_kv_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype, int32_t batch,
                              int32_t num_q_heads, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out,
                              void* workspace, size_t workspace_bytes, void* stream, bool rot_q) {
  const nvfp4_status_t st = check_mx_layer(layer);
  if (st != NVFP4_OK) return st;
  // the decode path reads the same fields; MXFP4 has no tensor-wide scale
  const nvfp4_kv_layer_t as_layer{layer->k_codes,    layer->k_scales,  layer->v_codes,   layer->v_scales,
                                  layer->num_pages,  layer->num_kv_heads, layer->head_dim, layer->page_size,
                                  1.0f,              1.0f};
  return decode_impl(&as_layer, nullptr, nullptr, q, q_dtype, batch, 1, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, sm_scale, out, workspace, workspace_bytes, stream, true, rot_q);
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t mxfp4_kv_quantize_append(const mxfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                  nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                  const int32_t* slot_mapping, void* stream) {
  return mx_append_impl(layer, k_new, v_new, dtype, num_tokens, token_stride_elems, slot_mapping, stream, false);
}

NVFP4_API nvfp4_status_t mxfp4_kv_quantize_append_hadamard(const mxfp4_kv_layer_t* layer, const void* k_new,
                                                           const void* v_new, nvfp4_dtype_t dtype, int32_t num_tokens,
                                                           int64_t token_stride_elems, const int32_t* slot_mapping,
                                                           void* stream) {
  return mx_append_impl(layer, k_new, v_new, dtype, num_tokens, token_stride_elems, slot_mapping, stream, true);
}

NVFP4_API nvfp4_status_t mxfp4_paged_decode_attn(const mxfp4_kv_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  return mx_decode_impl(layer, q, q_dtype, batch, num_q_heads, block_table, block_table_stride, seq_lens, max_seq_len,
                        sm_scale, out, workspace, workspace_bytes, stream, false);
}

NVFP4_API nvfp4_status_t mxfp4_paged_decode_attn_hadamard(const mxfp4_kv_layer_t* layer, const void* q,
                                                          nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                          const int32_t* block_table, int32_t block_table_stride,
                                                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                          float* out, void* workspace, size_t workspace_bytes,
                                                          void* stream) {
  return mx_decode_impl(layer, q, q_dtype, batch, num_q_heads, block_table, block_table_stride, seq_lens, max_seq_len,
                        sm_scale, out, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

// ------------------------------------------------------ Sparse-MLA latent cache

namespace {

nvfp4_status_t check_mla_layer(const nvfp4_mla_layer_t* L) {
  if (L == nullptr) return NVFP4_ERR_INVALID_ARGUMENT;
  if (L->latent_dim != kMlaLatent || L->rope_dim != kMlaDim - kMlaLatent) return NVFP4_ERR_UNSUPPORTED;
  if (!L->codes || !L->scales || L->num_slots <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(L->codes, 16) || !aligned(L->scales, 4)) return NVFP4_ERR_UNSUPPORTED;
  if (!scale_ok(L->global_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

NVFP4_API nvfp4_status_t nvfp4_mla_quantize_append(const nvfp4_mla_layer_t* layer, const void* kv_new,
                                                   nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                   const int32_t* slot_mapping, void* stream) {
  const nvfp4_status_t st = check_mla_layer(layer);
  if (st != NVFP4_OK) return st;
  if (!dtype_ok(dtype) || num_tokens < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return NVFP4_OK;
  if (!kv_new || !slot_mapping) return NVFP4_ERR_INVALID_ARGUMENT;
  if (token_stride_elems < kMlaDim) return NVFP4_ERR_INVALID_ARGUMENT;
  const int64_t esize = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (!aligned(kv_new, 16) || (token_stride_elems * esize) % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
  MlaAppendParams p;
  p.x = kv_new;
  p.codes = layer->codes;
  p.scales = layer->scales;
  p.slots = slot_mapping;
  p.token_stride = token_stride_elems;
  p.num_tokens = num_tokens;
  p.num_slots = layer->num_slots;
  p.g = layer->global_scale;
  p.r6 = 1.0 / (6.0 * (double)layer->global_scale);
  return from_hip(launch_mla_append(p, dtype, static_cast<hipStream_t>(stream)));
}

static bool mla_shape_ok(int32_t num_q_tokens, int32_t num_q_heads, int32_t topk) {
  if (num_q_tokens < 0 || num_q_heads <= 0 || topk < 0) return false;
  if (num_q_heads % 16 != 0 || (num_q_heads > 64 && num_q_heads % 64 != 0)) return false;
  if (topk > (1 << 20)) return false;
  return true;
}

NVFP4_API size_t nvfp4_mla_sparse_decode_workspace_bytes(int32_t num_q_tokens, int32_t num_q_heads, int32_t topk) {
  if (!mla_shape_ok(num_q_tokens, num_q_heads, topk) || num_q_tokens == 0) return 0;
  const MlaGeometry geo = mla_geometry(num_q_tokens, num_q_heads, topk);
  if (geo.waves == 0 || (int64_t)num_q_tokens * geo.HB * geo.splits >= ((int64_t)1 << 31)) return 0;
  return geo.workspace_bytes;
}

NVFP4_API nvfp4_status_t nvfp4_mla_sparse_decode(const nvfp4_mla_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t num_q_tokens, int32_t num_q_heads, const int32_t* indices,
                                                 int32_t topk, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  const nvfp4_status_t st = check_mla_layer(layer);
  if (st != NVFP4_OK) return st;
  if (!dtype_ok(q_dtype) || num_q_tokens < 0 || num_q_heads <= 0 || topk < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (q_dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_UNSUPPORTED;
  if (!mla_shape_ok(num_q_tokens, num_q_heads, topk)) return NVFP4_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return NVFP4_ERR_INVALID_ARGUMENT;
  const double qk = (double)sm_scale * (double)layer->global_scale * 1.4426950408889634;  // log2(e)
  if (!std::isfinite(qk) || !std::isfinite((float)qk)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (num_q_tokens == 0) return NVFP4_OK;
  if (!q || !out || (topk > 0 && !indices)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16)) return NVFP4_ERR_UNSUPPORTED;
  const MlaGeometry geo = mla_geometry(num_q_tokens, num_q_heads, topk);
  if (geo.waves == 0 || (int64_t)num_q_tokens * geo.HB * geo.splits >= ((int64_t)1 << 31)) return NVFP4_ERR_UNSUPPORTED;
  if (geo.workspace_bytes > 0) {  // some list is split: the shares' partials
    if (workspace_bytes < geo.workspace_bytes) return NVFP4_ERR_WORKSPACE_TOO_SMALL;
    if (!workspace || !aligned(workspace, 256)) return NVFP4_ERR_INVALID_ARGUMENT;
  }
  MlaDecodeParams p;
  p.codes = layer->codes;
  p.scales = layer->scales;
  p.q = q;
  p.indices = indices;
  p.out = out;
  p.part = static_cast<float*>(workspace);
  p.num_slots = layer->num_slots;
  p.T = num_q_tokens;
  p.Hq = num_q_heads;
  p.topk = topk;
  p.HB = geo.HB;
  p.splits = geo.splits;
  p.per_split = geo.per_split;
  p.qk_scale_log2 = (float)qk;
  p.v_scale = layer->global_scale;
  return from_hip(launch_mla_decode(p, geo.waves, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
