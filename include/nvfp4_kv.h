/*
 * nvfp4_kv.h -- C ABI of the MI355X (gfx950) NVFP4 paged KV-cache library.
 *
 * NVFP4 stores each K/V value as a 4-bit E2M1 code (values +-{0, 0.5, 1, 1.5,
 * 2, 3, 4, 6}), every 16 consecutive values along head_dim share one FP8 E4M3
 * block scale, and each tensor has one FP32 global scale: 9/16 byte per value
 * (grer.cn blog "NVFP4 KV cache and the memory wall", section 2, two-level
 * scaling, and section 1 for the 9/16 byte accounting; cloud.tencent.com.cn
 * "NVFP4: breaking the memory wall of GPU inference", E2M1 encoding section).
 *
 * The entry points follow the cache data flows of section 3 of the same blog:
 * quantize-on-write of new K/V, decode attention that dequantizes inside the
 * kernel, extend-path dequantization into one FP8 workspace that is reused
 * across layers, and the FP8 attention of an extend / prefill chunk over that
 * workspace (with the chunk's own K/V stored as FP8 rows).
 *
 * Conventions for every function
 *   - All array arguments are DEVICE pointers unless marked "host".  The caller
 *     owns every buffer; the library never allocates, frees, synchronizes, or
 *     reads device memory from the host.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; results are visible after the caller's stream sync.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns a status and enqueues nothing.  A launch failure returns
 *     NVFP4_ERR_HIP.  Functions are stateless and thread-safe, except
 *     nvfp4_paged_decode_attn_noalloc, which uses a device scratch array the
 *     library holds per GPU (see there).
 *   - Supported shapes: head_dim 128 and page_size 16 only (others return
 *     NVFP4_ERR_UNSUPPORTED); at most 16 query heads per KV head.
 *   - Device-side index data (slot_mapping, block_table, seq_lens, prefix_lens,
 *     ws_offsets) is bounds-checked in the kernels: an out-of-range slot or page
 *     index is skipped (its tokens are ignored), never dereferenced.
 *
 * Cache layout (one layer; 16 token slots per page; slot s is page s/16,
 * offset o = s%16; tile (p, h) = page p, KV head h):
 *   k_codes  [num_pages][H][1024] u8: byte o*64 + d/2 of the tile holds dims
 *            d (even: low nibble) and d+1 (high nibble) of token o.
 *   k_scales [num_pages][H][128]  u8: byte o*8 + b = E4M3 scale of dims 16b..16b+15.
 *   v_codes  [num_pages][H][1024] u8: byte (o/4)*256 + (d/8)*16 + ((o/2)%2)*8
 *            + (d%2)*4 + (d%8)/2 holds dim d of tokens o (o even: low nibble)
 *            and o^1 (high nibble).
 *   v_scales [num_pages][H][128]  u8: byte (d/16)*16 + o.
 *   An E2M1 code is sign<<3 | magnitude code (0..7 <-> 0, .5, 1, 1.5, 2, 3, 4, 6).
 *   A value reads back as E2M1(code) * E4M3(scale) * global (k_global or v_global).
 */
#ifndef NVFP4_KV_H
#define NVFP4_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

/* The status and dtype enums are int-sized in C.  Seen from C++ they get int
 * as their fixed underlying type, so every int a C caller passes (an unknown
 * status for nvfp4_status_string, a bad dtype that the checks reject) is a
 * valid value of the type rather than undefined behaviour. */
#ifdef __cplusplus
#define NVFP4_ENUM_BASE : int
#else
#define NVFP4_ENUM_BASE
#endif

typedef enum nvfp4_status NVFP4_ENUM_BASE {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad scale, inconsistent sizes */
  NVFP4_ERR_UNSUPPORTED = 2,      /* head_dim != 128, page_size != 16, >16 q heads per kv head, alignment */
  NVFP4_ERR_WORKSPACE_TOO_SMALL = 3,
  NVFP4_ERR_HIP = 4               /* a HIP launch reported an error */
} nvfp4_status_t;

typedef enum nvfp4_dtype NVFP4_ENUM_BASE {
  NVFP4_DTYPE_F32 = 0,
  NVFP4_DTYPE_BF16 = 1
} nvfp4_dtype_t;

/* One layer's NVFP4 cache.  Plane pointers are device memory with the sizes
 * given in the layout above; code planes 16-byte aligned, scale planes 4-byte
 * aligned.  k_global / v_global are the FP32 per-tensor scales; they must be
 * finite with 2^-100 <= g <= 2^100. */
typedef struct nvfp4_kv_layer {
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;  /* must be 128 */
  int32_t page_size; /* must be 16 */
  float k_global;
  float v_global;
} nvfp4_kv_layer_t;

/* Quantize-on-append (blog section 3, first data flow: new K/V are written to
 * the cache as NVFP4; nmedialink.com "NVIDIA NVFP4: LLM memory doubled,
 * inference 3x", Fig. 3: new keys and values are quantized before they are
 * appended).  For each new token t < num_tokens with slot = slot_mapping[t]
 * (skipped when slot < 0 or slot >= num_pages*16), and each KV head h and
 * 16-value block b along head_dim:
 *   amax = max |x|,  bs = E4M3 nearest to amax/(6*g) (ties to even, saturating
 *   at 448, 0 below half the smallest step), code = sign(x) | E2M1 nearest to
 *   |x|/(bs*g) (ties to even, saturating at 6; magnitude 0 when bs = 0).
 *   k_new, v_new : [num_tokens][num_kv_heads][128] of `dtype`; consecutive tokens
 *                  are token_stride_elems elements apart (>= num_kv_heads*128);
 *                  16-byte aligned base and token stride.  Values must be finite.
 *   slot_mapping : [num_tokens] int32.
 * A slot that appears twice in one call ends with an unspecified mix of both
 * tokens' codes and scales.  num_tokens == 0 is a no-op.
 *   Supported: ceil(num_tokens/16) * num_kv_heads < 2^31. */
NVFP4_API nvfp4_status_t nvfp4_kv_quantize_append(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                  nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                  const int32_t* slot_mapping, void* stream);

/* Bytes of device workspace nvfp4_paged_decode_attn needs for these (host)
 * sizes (never 0 for batch > 0); 0 for batch 0 or sizes the call rejects. */
NVFP4_API size_t nvfp4_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t max_seq_len);

/* Decode attention over the paged NVFP4 cache, dequantizing inside the kernel
 * (blog section 3, third data flow: decode is bound by reading the cache, so
 * no separate dequant pass; the 4-bit values are widened in registers and the
 * block scale is applied there).  For each sequence b < batch and query head
 * j < num_q_heads, with KV head h = j / (num_q_heads / num_kv_heads):
 *   s_t = sm_scale * q[b][j] . K_hat[t]   for t < seq_lens[b],
 *   out[b][j] = sum_t softmax(s)_t * V_hat[t]            (fp32 accumulate)
 * where token t sits in slot block_table[b*block_table_stride + t/16]*16 + t%16
 * and K_hat/V_hat are the dequantized values.  seq_lens[b] == 0 gives zeros.
 *   q            : [batch][num_q_heads][128] of q_dtype (16-byte aligned).
 *   block_table  : [batch][block_table_stride] int32 page indices.
 *   seq_lens     : [batch] int32, each <= max_seq_len (larger values are
 *                  clamped to max_seq_len).
 *   max_seq_len  : host bound used to size the launch; block_table_stride must
 *                  be >= ceil(max_seq_len/16).
 *   out          : [batch][num_q_heads][128] float32.
 *   workspace    : >= nvfp4_paged_decode_workspace_bytes(...) bytes, 256-byte
 *                  aligned.  It holds one arrival counter per (sequence,
 *                  kv head) and the partial results of the (sequence, kv head)
 *                  pairs whose pages are shared by several workgroups.  It must be zero-filled once before its
 *                  first use; every call leaves the counters at zero again.
 *                  Calls that share a workspace must be ordered on one stream.
 *   Supported: batch <= 4096 and
 *              batch * num_kv_heads * (ceil(max_seq_len/16) + 96) <= 2^30. */
NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn(const nvfp4_kv_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): nvfp4_paged_decode_attn with its workspace taken from the
 * library's own device scratch instead of a caller buffer.  The call
 * allocates and frees nothing.
 * Scratch: one 8 MiB device array per GPU, held until the process ends --
 * 64 KiB of arrival counters (one int32 per (sequence, kv head)), then the
 * split partials.  The first call on a device looks the array up and clears
 * the counters with a fill kernel on `stream`; every call leaves them at zero
 * again.  Every call on a GPU shares that GPU's scratch and finds the last
 * call's partials in it: calls on one GPU must be ordered (one stream, or
 * synchronized); calls that overlap race.
 * Limit: batch * num_kv_heads <= 16384, and the partials must fit:
 *   nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, num_kv_heads,
 *   max_seq_len) - 256 * ceil(batch * num_kv_heads / 64) <= 8 MiB - 64 KiB
 * (e.g. up to 218 sequences of 8 kv heads at 8 query heads per kv head, any
 * context length).  Larger calls return NVFP4_ERR_WORKSPACE_TOO_SMALL before
 * any HIP call.  Other arguments, results and errors as nvfp4_paged_decode_attn. */
NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_noalloc(const nvfp4_kv_layer_t* layer, const void* q,
                                                         nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                         const int32_t* block_table, int32_t block_table_stride,
                                                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                         float* out, void* stream);

/* Decode of several new query tokens per sequence (multi-token or
 * speculative decoding).  It is the decode data flow of blog section 3 with q_per_seq query tokens
 * that share one pass over the cache: their G * q_per_seq query rows fill the
 * 16-row MFMA tile that plain decode fills only to G.  The q_per_seq new
 * tokens are already appended: query token i < q_per_seq of sequence b sits
 * at position seq_lens[b] - q_per_seq + i and attends over tokens
 * t <= that position (causal among the new tokens).
 *   q   : [batch][q_per_seq][num_q_heads][128] of q_dtype (16-byte aligned).
 *   out : [batch][q_per_seq][num_q_heads][128] float32.
 *   workspace: >= nvfp4_paged_decode_multi_workspace_bytes(batch, q_per_seq,
 *          num_q_heads, num_kv_heads, max_seq_len) bytes; the same contract as
 *          nvfp4_paged_decode_attn's (zero-filled once, left zeroed, calls
 *          that share it ordered on one stream).
 *   Other arguments as nvfp4_paged_decode_attn; seq_lens[b] < q_per_seq
 *   leaves the tokens with no key at zero output.
 *   Supported: (num_q_heads / num_kv_heads) * q_per_seq <= 16,
 *   q_per_seq * num_q_heads * 512 < 2^31, and the batch and size limits of
 *   nvfp4_paged_decode_attn.  q_per_seq == 1 is nvfp4_paged_decode_attn. */
NVFP4_API size_t nvfp4_paged_decode_multi_workspace_bytes(int32_t batch, int32_t q_per_seq, int32_t num_q_heads,
                                                          int32_t num_kv_heads, int32_t max_seq_len);
NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_multi(const nvfp4_kv_layer_t* layer, const void* q,
                                                       nvfp4_dtype_t q_dtype, int32_t batch, int32_t q_per_seq,
                                                       int32_t num_q_heads, const int32_t* block_table,
                                                       int32_t block_table_stride, const int32_t* seq_lens,
                                                       int32_t max_seq_len, float sm_scale, float* out,
                                                       void* workspace, size_t workspace_bytes, void* stream);

/* One decode step in one call: quantize-on-append of each sequence's
 * q_per_seq new tokens (blog section 3, first data flow) and the decode
 * attention over the cache that now holds them (third data flow), fused.
 * The new tokens of sequence b sit at positions
 * seq_lens[b] - q_per_seq + i, i < q_per_seq (seq_lens already counts them);
 * their slots come from block_table.  The result is the same as
 * nvfp4_kv_quantize_append of those tokens followed by
 * nvfp4_paged_decode_attn_multi: the same cache bytes and the same output.
 * Schedule: when a unit holds at most 64 pages (max_seq_len <= 1024) the
 * step is one launch -- the workgroup that reads a page holding a new token
 * quantizes and stores that token itself before it loads the page, so no
 * workgroup waits on another.  Longer units take two launches on `stream`
 * (the append kernel, with each new token's slot taken from block_table,
 * then the decode), which measured faster there.  Both give the same bytes
 * and output.
 *   k_new, v_new : [batch][q_per_seq][num_kv_heads][128] of dtype (the
 *                  query's dtype), 16-byte aligned.  Positions < 0
 *                  (seq_lens[b] < q_per_seq) and out-of-range page indices
 *                  are skipped.
 *   Other arguments and the workspace as nvfp4_paged_decode_attn_multi. */
NVFP4_API nvfp4_status_t nvfp4_paged_decode_step(const nvfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                 const void* q, nvfp4_dtype_t dtype, int32_t batch, int32_t q_per_seq,
                                                 int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream);

/* Extend-path dequantization into one FP8 workspace pair (blog section 3,
 * second data flow: cached NVFP4 pages are dequantized into a single FP8
 * workspace that every layer reuses; nmedialink.com, Fig. 3: values are taken
 * from NVFP4 back to FP8 before attention).  For extend sequence i < num_seqs
 * and cached token t < prefix_lens[i] (slot from block_table row i as above):
 *   ws_k[(ws_offsets[i] + t)][h][d] = sign(x) | E4M3 nearest to |x|/k_ws_scale
 *   (x = K_hat value; ties to even, saturating at 448; sign bit kept, so -0.0
 *   gives 0x80), and likewise ws_v with V_hat and v_ws_scale.
 *   prefix_lens : [num_seqs] int32;  ws_offsets : [num_seqs+1] int32 token
 *                 offsets into the workspace.
 *   max_prefix_len: host bound, >= every prefix_lens[i] (sizes the launch;
 *                 larger prefix_lens are clamped to it); block_table_stride
 *                 must be >= ceil(max_prefix_len/16).
 *   ws_k, ws_v  : [ws_capacity_tokens][num_kv_heads][128] uint8; rows at or
 *                 beyond ws_capacity_tokens are never written.
 *   k_ws_scale, v_ws_scale: finite, 2^-100 <= s <= 2^100. */
NVFP4_API nvfp4_status_t nvfp4_dequant_to_fp8_workspace(const nvfp4_kv_layer_t* layer, const int32_t* block_table,
                                                        int32_t block_table_stride, int32_t num_seqs,
                                                        const int32_t* prefix_lens, const int32_t* ws_offsets,
                                                        int32_t max_prefix_len, float k_ws_scale, float v_ws_scale,
                                                        uint8_t* ws_k, uint8_t* ws_v, int32_t ws_capacity_tokens,
                                                        void* stream);

/* FP8 rows of new tokens (blog section 3, first and second data flows: the
 * K/V of the tokens being prefilled or extended take part in attention as FP8;
 * only the cached prefix goes through the NVFP4 -> FP8 workspace).  Typical
 * use: an extend chunk's K/V go into the workspace rows right after its
 * prefix, with the workspace's own scales.  For token t < num_tokens with
 * 0 <= ws_rows[t] < ws_capacity_tokens, KV head h and dim d:
 *   ws_k[ws_rows[t]][h][d] = sign(x) | E4M3 nearest to |x| / k_ws_scale
 *   (x = k_new[t][h][d]; ties to even, saturating at 448: the rounding of
 *   nvfp4_dequant_to_fp8_workspace), and likewise ws_v from v_new.
 *   k_new, v_new : [num_tokens][num_kv_heads][128] of dtype, token stride
 *                  token_stride_elems >= num_kv_heads*128; 16-byte aligned
 *                  pointers and token rows.
 *   ws_rows      : [num_tokens] int32; other rows (< 0 or past the capacity)
 *                  are skipped.
 *   ws_k, ws_v   : [ws_capacity_tokens][num_kv_heads][128] uint8, 16-byte aligned.
 *   Non-finite inputs give unspecified bytes (written in bounds). */
NVFP4_API nvfp4_status_t nvfp4_fp8_rows_to_workspace(const void* k_new, const void* v_new, nvfp4_dtype_t dtype,
                                                     int32_t num_tokens, int64_t token_stride_elems,
                                                     int32_t num_kv_heads, const int32_t* ws_rows, float k_ws_scale,
                                                     float v_ws_scale, uint8_t* ws_k, uint8_t* ws_v,
                                                     int32_t ws_capacity_tokens, void* stream);

/* Causal attention of extend (or prefill) chunks over FP8 workspace rows
 * (blog section 3, second data flow: a chunked prefill / extend attends over
 * its cached prefix from the FP8 workspace; first data flow: the new tokens'
 * own K/V take part as FP8, causally as in prefill).  Sequence i < num_seqs
 * has prefix P_i = prefix_lens[i] and chunk C_i = q_offsets[i+1] -
 * q_offsets[i]; its K/V are workspace rows ws_offsets[i] + t, t < P_i + C_i
 * (the prefix from nvfp4_dequant_to_fp8_workspace, the chunk from
 * nvfp4_fp8_rows_to_workspace).  Query token j < C_i is row q_offsets[i] + j
 * of q; for query head qh and kv head h = qh / (num_q_heads/num_kv_heads):
 *   s_t = sm_scale * sum_d q[d] * E4M3(ws_k[row_t][h][d]) * k_ws_scale,  t <= P_i + j
 *   out[q_offsets[i] + j][qh][d] = sum_t softmax(s)_t * E4M3(ws_v[row_t][h][d]) * v_ws_scale
 * E4M3 values are widened exactly to f16 for f16 MFMA; softmax and
 * accumulation are fp32.
 *   q          : [num_q_tokens][num_q_heads][128] of q_dtype, 16-byte aligned.
 *   q_offsets  : [num_seqs+1] int32, nondecreasing (values are clamped to
 *                [0, num_q_tokens]); ws_offsets, prefix_lens: [num_seqs] int32.
 *   max_chunk_len: host bound >= every C_i (sizes the launch); query tokens
 *                of a chunk past it are not computed.
 *   ws_k, ws_v : [ws_capacity_tokens][num_kv_heads][128] uint8, 16-byte aligned;
 *                rows outside it read as zero bytes (memory-safe, results
 *                then unspecified).
 *   out        : [num_q_tokens][num_q_heads][128] float32; rows of tokens that
 *                belong to no chunk are not written.
 *   Supported: num_kv_heads <= 65535 and num_seqs <= 65535. */
NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                               const int32_t* q_offsets, const int32_t* ws_offsets,
                                               const int32_t* prefix_lens, int32_t max_chunk_len,
                                               const uint8_t* ws_k, const uint8_t* ws_v, int32_t ws_capacity_tokens,
                                               float k_ws_scale, float v_ws_scale, float sm_scale, float* out,
                                               void* stream);

/* The same attention with each chunk tile's keys divided among several
 * workgroups when the chunks alone are too few tiles to fill the GPU (short
 * extend chunks over long cached prefixes, as in speculative verification or
 * a small last prefill chunk).  Each workgroup keeps an unnormalised partial
 * output with its row maximum and row sum in `workspace`; a second kernel on
 * the same stream merges them (the usual log-sum-exp combination of softmax
 * pieces).  The result equals nvfp4_fp8_extend_attn's up to fp32 rounding
 * order.  Arguments are those of nvfp4_fp8_extend_attn plus:
 *   max_prefix_len : host bound on the prefixes P_i, used only to choose the
 *                    split (a larger P_i is still computed correctly).
 *   workspace      : device memory of at least
 *                    nvfp4_fp8_extend_attn_split_workspace_bytes(...) bytes,
 *                    16-byte aligned, owned by the caller, contents ignored
 *                    and overwritten; may be NULL when that size is 0 (no
 *                    split chosen: the call is then nvfp4_fp8_extend_attn).
 * Errors: those of nvfp4_fp8_extend_attn; INVALID_ARGUMENT for
 * max_prefix_len < 0 or a NULL workspace that is needed,
 * WORKSPACE_TOO_SMALL for workspace_bytes below the size, UNSUPPORTED for a
 * misaligned workspace.  Calls that share a workspace must not overlap. */
NVFP4_API size_t nvfp4_fp8_extend_attn_split_workspace_bytes(nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                              int32_t num_q_heads, int32_t num_kv_heads,
                                                              int32_t num_seqs, int32_t max_chunk_len,
                                                              int32_t max_prefix_len);
NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn_split(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                     const int32_t* q_offsets, const int32_t* ws_offsets,
                                                     const int32_t* prefix_lens, int32_t max_chunk_len,
                                                     int32_t max_prefix_len, const uint8_t* ws_k, const uint8_t* ws_v,
                                                     int32_t ws_capacity_tokens, float k_ws_scale, float v_ws_scale,
                                                     float sm_scale, float* out, void* workspace,
                                                     size_t workspace_bytes, void* stream);

/* The same extend attention in FP8 arithmetic, on gfx950's FP8 (E4M3) MFMA:
 * the workspace's E4M3 K and V bytes enter the matrix cores as they are
 * (blog section 3: extend attention consumes the FP8 workspace directly),
 * and so do Q and the softmax weights, each rounded to E4M3:
 *   c  = float32 of sm_scale * k_ws_scale * log2(e), u = float32(q * c);
 *   Q8 = E4M3(u * 2^-E) per (query token, query head) row, E the smallest
 *        integer with max|u| <= 448 * 2^E (round to nearest, ties to even);
 *   x_t = 2^E * sum_d Q8_d * E4M3(ws_k[row_t][h][d])  (base-2 logits, fp32
 *        accumulation);
 *   M  = ceil(max_t x_t);  W8_t = E4M3(2^(x_t - M + 8))  (at most 256; 2^(x_t - M)
 *        when |M| >= 2^27, where float32 cannot hold M - 8 exactly);
 *   out = v_ws_scale * sum_t W8_t * E4M3(ws_v[row_t][h][d]) / sum_t W8_t.
 * The kernel keeps an integer running maximum instead of M (rescales by
 * exact powers of two), so weights below 2^-14 of the row's largest can round
 * at a finer scale than M's; the accumulation error of the FP8 matrix cores
 * is within 2^-11 of the largest product per 64-term dot product.  Each
 * element of Q and of the weights carries up to 2^-4 relative rounding error:
 * this is a lower-precision contract than nvfp4_fp8_extend_attn's (about
 * 1e-2 of a row's largest value on the synthetic workloads, against 1e-3),
 * for about 4x less matrix-core work per key.  Arguments, layouts, errors and
 * the optional key split (with its workspace) are those of
 * nvfp4_fp8_extend_attn_split; the split sizes differ, so the workspace size
 * comes from nvfp4_fp8_extend_attn_f8_workspace_bytes. */
NVFP4_API size_t nvfp4_fp8_extend_attn_f8_workspace_bytes(nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                           int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                           int32_t max_chunk_len, int32_t max_prefix_len);
NVFP4_API nvfp4_status_t nvfp4_fp8_extend_attn_f8(const void* q, nvfp4_dtype_t q_dtype, int32_t num_q_tokens,
                                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                                  const int32_t* q_offsets, const int32_t* ws_offsets,
                                                  const int32_t* prefix_lens, int32_t max_chunk_len,
                                                  int32_t max_prefix_len, const uint8_t* ws_k, const uint8_t* ws_v,
                                                  int32_t ws_capacity_tokens, float k_ws_scale, float v_ws_scale,
                                                  float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                                  void* stream);

/* ------------------------------------------------------------------ MXFP4
 * The 4-bit format the NVFP4 pages compare against (nmedialink.com, accuracy
 * section and Fig. 6: NVFP4 KV caches score above MXFP4 ones, credited to the
 * finer blocks and the E4M3 scales; cloud.tencent.com.cn, E2M1 encoding and
 * two-level scaling section: MXFP4 shares one scale among 32 values).  The
 * scale rule is the OCP MX v1.0 one, which the pages do not spell out: per
 * 32 consecutive values along head_dim, X = 2^(floor(log2 amax) - 2) clamped
 * to 2^-127 .. 2^127 (2^-127 for amax = 0), stored as an E8M0 byte
 * (X = 2^(byte - 127)); code = sign(x) | E2M1 nearest to |x|/X (ties to even,
 * saturating at 6).  No tensor-wide scale.  17/32 byte per value.
 *
 * Layout: k_codes as the NVFP4 k_codes; v_codes keeps each token's nibbles
 * in bytes of its own (its two values share that token's E8M0 scale):
 *   v_codes  [num_pages][H][1024] u8: byte (o/4)*256 + (d/8)*16 + (o%4)*4 +
 *            (d%8)/2 holds dims d (low nibble, d even) and d+1 of token o.
 * A scale tile is 64 bytes:
 *   k_scales [num_pages][H][64] u8: byte o*4 + d/32 = E8M0 scale of dims
 *            32*(d/32) .. +31 of token o.
 *   v_scales [num_pages][H][64] u8: byte (d/32)*16 + o. */
typedef struct mxfp4_kv_layer {
  uint8_t* k_codes;  /* [num_pages][H][1024], 16-byte aligned */
  uint8_t* k_scales; /* [num_pages][H][64], 4-byte aligned */
  uint8_t* v_codes;
  uint8_t* v_scales;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;  /* must be 128 */
  int32_t page_size; /* must be 16 */
} mxfp4_kv_layer_t;

/* MXFP4 quantize-on-append: the data flow of nvfp4_kv_quantize_append with
 * the MXFP4 rounding above; arguments, skipping of bad slots, duplicate
 * slots, limits and errors as there.  Values must be finite. */
NVFP4_API nvfp4_status_t mxfp4_kv_quantize_append(const mxfp4_kv_layer_t* layer, const void* k_new, const void* v_new,
                                                  nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                  const int32_t* slot_mapping, void* stream);

/* Decode attention over MXFP4 pages: the computation, arguments, workspace
 * (nvfp4_paged_decode_workspace_bytes), limits and errors of
 * nvfp4_paged_decode_attn, with K_hat / V_hat the MXFP4 values.  Dequantized
 * values are exact in bf16 and the products run on bf16 MFMA with fp32
 * accumulation; P enters as a bf16 hi + lo pair. */
NVFP4_API nvfp4_status_t mxfp4_paged_decode_attn(const mxfp4_kv_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                                 int32_t block_table_stride, const int32_t* seq_lens,
                                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ Hadamard-rotated K
 * cloud.tencent.com.cn "NVFP4: breaking the memory wall of GPU inference",
 * E2M1 encoding and two-level scaling section, quantization tricks: an
 * orthogonal Hadamard transform applied before quantization spreads a local
 * outlier over the whole vector.  Here K rows are rotated before they are
 * quantized and the query is rotated the same way at decode time, so the
 * scores are unchanged:
 *   k' = H k / 16,  q' = H q / 8,  q'.k' = q.k,
 * H the 128-point Sylvester Walsh-Hadamard matrix, H[i][j] = (-1)^popcount(i & j)
 * (H H^T = 128 I; both scales are powers of two).  V is stored as usual.
 * k' is the float32 nearest to the exact H k / 16 whenever that sum is exact
 * in float64 (every 128-value row of bf16 values spanning at most 38
 * binades, of float32 values spanning at most 22); it is then quantized like
 * any K row, so the cache bytes equal those of the unrotated call on k'.
 * A cache written with a _hadamard append must be read with the _hadamard
 * decode of the same format; the global scale k_global is calibrated on k'.
 * The FP8 workspace, multi-token decode and the one-launch step read
 * unrotated caches only. */

/* nvfp4_kv_quantize_append with K rows rotated (k' above) before quantization. */
NVFP4_API nvfp4_status_t nvfp4_kv_quantize_append_hadamard(const nvfp4_kv_layer_t* layer, const void* k_new,
                                                           const void* v_new, nvfp4_dtype_t dtype, int32_t num_tokens,
                                                           int64_t token_stride_elems, const int32_t* slot_mapping,
                                                           void* stream);

/* nvfp4_paged_decode_attn over a cache of rotated K: each query row is
 * rotated (q' above, in fp32) and, no longer exact in 16 bits, enters the
 * MFMA as an f16 hi + lo pair.  Arguments, workspace, limits and errors as
 * nvfp4_paged_decode_attn. */
NVFP4_API nvfp4_status_t nvfp4_paged_decode_attn_hadamard(const nvfp4_kv_layer_t* layer, const void* q,
                                                          nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                          const int32_t* block_table, int32_t block_table_stride,
                                                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                          float* out, void* workspace, size_t workspace_bytes,
                                                          void* stream);

/* The same pair for MXFP4 caches. */
NVFP4_API nvfp4_status_t mxfp4_kv_quantize_append_hadamard(const mxfp4_kv_layer_t* layer, const void* k_new,
                                                           const void* v_new, nvfp4_dtype_t dtype, int32_t num_tokens,
                                                           int64_t token_stride_elems, const int32_t* slot_mapping,
                                                           void* stream);
NVFP4_API nvfp4_status_t mxfp4_paged_decode_attn_hadamard(const mxfp4_kv_layer_t* layer, const void* q,
                                                          nvfp4_dtype_t q_dtype, int32_t batch, int32_t num_q_heads,
                                                          const int32_t* block_table, int32_t block_table_stride,
                                                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                                          float* out, void* workspace, size_t workspace_bytes,
                                                          void* stream);

/* ------------------------------------------------- Sparse-MLA latent cache
 * grer.cn blog "NVFP4 KV cache and the memory wall", section 6 (closing
 * note): the serving engine's NVFP4 KV cache supports GQA and Sparse MLA
 * models.  An MLA cache holds one latent row per token, shared by every query
 * head: 512 latent values followed by 64 rotary-key values.  Rows are stored
 * as NVFP4 with the rule of nvfp4_kv_quantize_append applied to 36 blocks of
 * 16 consecutive values (one E4M3 scale per block, one FP32 global scale per
 * layer): 324 bytes per token, 9/16 byte per value.
 * Layout (slot s = page * page_size + offset, for any page size):
 *   codes  [num_slots][288] u8: byte j of a row holds values 2j (low nibble)
 *          and 2j+1 (high nibble).
 *   scales [num_slots][36]  u8: byte b = E4M3 scale of values 16b .. 16b+15.
 * A value reads back as E2M1(code) * E4M3(scale) * global_scale. */
typedef struct nvfp4_mla_layer {
  uint8_t* codes;      /* 16-byte aligned */
  uint8_t* scales;     /* 4-byte aligned */
  int32_t num_slots;
  int32_t latent_dim;  /* must be 512 */
  int32_t rope_dim;    /* must be 64 */
  float global_scale;  /* finite, 2^-100 <= g <= 2^100 */
} nvfp4_mla_layer_t;

/* Quantize-on-append of latent rows (blog section 3, first data flow, for the
 * MLA cache): row t < num_tokens of kv_new ([num_tokens][576] of dtype,
 * token_stride_elems >= 576 apart, 16-byte aligned base and stride, finite
 * values) goes to slot slot_mapping[t]; slots < 0 or >= num_slots are
 * skipped; the rounding is that of nvfp4_kv_quantize_append, block by block.
 * num_tokens == 0 is a no-op.  Supported: num_tokens * 18 < 2^31 * 256. */
NVFP4_API nvfp4_status_t nvfp4_mla_quantize_append(const nvfp4_mla_layer_t* layer, const void* kv_new,
                                                   nvfp4_dtype_t dtype, int32_t num_tokens, int64_t token_stride_elems,
                                                   const int32_t* slot_mapping, void* stream);

/* Bytes of device workspace nvfp4_mla_sparse_decode needs (host sizes): the
 * partial results of lists that the call splits over several workgroups (it
 * does so when few query tokens would leave CUs idle).  0 when no list is
 * split (the call then takes no workspace), for num_q_tokens == 0, and for
 * sizes the call rejects. */
NVFP4_API size_t nvfp4_mla_sparse_decode_workspace_bytes(int32_t num_q_tokens, int32_t num_q_heads, int32_t topk);

/* Sparse MLA decode over the NVFP4 latent cache (blog section 3, third data
 * flow, dequantizing inside the kernel; section 6: Sparse MLA).  For query
 * token t < num_q_tokens and head h < num_q_heads, over the entries j <
 * topk of indices[t][0..topk) that are cache slots (entries < 0 or >=
 * num_slots are skipped; an entry listed twice counts twice):
 *   s_j = sm_scale * sum_{d<576} q[t][h][d] * K_hat[slot_j][d]
 *   out[t][h][d] = sum_j softmax(s)_j * K_hat[slot_j][d],  d < 512 (fp32 accumulate)
 * A token with no valid entry gets zeros.  Dequantized values are exact in f16;
 * the products run on f16 MFMA, P as an f16 hi + lo pair.
 *   q       : [num_q_tokens][num_q_heads][576] bf16 (q_dtype must be BF16), 16-byte aligned.
 *   indices : [num_q_tokens][topk] int32 cache slots.
 *   out     : [num_q_tokens][num_q_heads][512] float32.
 *   workspace: >= nvfp4_mla_sparse_decode_workspace_bytes(...) bytes, 256-byte
 *            aligned, when that is not 0 (else ignored; may be NULL): the
 *            partial results of split lists, written and merged by the call (a
 *            second launch on `stream`); no initial contents needed; calls
 *            that share it must be ordered on one stream.
 *   Supported: num_q_heads a multiple of 16, and of 64 above 64; topk <= 2^20;
 *   q_dtype BF16.  Others return NVFP4_ERR_UNSUPPORTED. */
NVFP4_API nvfp4_status_t nvfp4_mla_sparse_decode(const nvfp4_mla_layer_t* layer, const void* q, nvfp4_dtype_t q_dtype,
                                                 int32_t num_q_tokens, int32_t num_q_heads, const int32_t* indices,
                                                 int32_t topk, float sm_scale, float* out, void* workspace,
                                                 size_t workspace_bytes, void* stream);

/* Static string for a status code. */
NVFP4_API const char* nvfp4_status_string(nvfp4_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_KV_H */
