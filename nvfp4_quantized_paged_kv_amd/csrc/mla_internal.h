// Internal declarations of the Sparse-MLA latent cache kernels (not part of
// the public C ABI): NVFP4 latent rows of 576 values, one per cache slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvfp4_kv.h"

namespace nvfp4kv {

constexpr int kMlaDim = 576;          // 512 latent + 64 rotary-key values per token row
constexpr int kMlaLatent = 512;       // values the output sums
constexpr int kMlaRowCodeBytes = 288; // E2M1 codes of one row
constexpr int kMlaRowScaleBytes = 36; // E4M3 scales of one row (36 blocks of 16)
constexpr int kMlaPartStride = kMlaLatent + 4;  // floats per (partial, head): O, running max (log2), sum, 2 pad

struct MlaAppendParams {
  const void* x;          // [num_tokens][576], token stride `token_stride` elements
  uint8_t* codes;         // [num_slots][288]
  uint8_t* scales;        // [num_slots][36]
  const int32_t* slots;   // [num_tokens]
  int64_t token_stride;
  int32_t num_tokens;
  int32_t num_slots;
  float g;                // FP32 global scale
  double r6;              // 1/(6g) rounded to float64
};

hipError_t launch_mla_append(const MlaAppendParams& p, nvfp4_dtype_t dtype, hipStream_t stream);

struct MlaDecodeParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const void* q;          // [T][Hq][576] bf16
  const int32_t* indices; // [T][topk] cache slots
  float* out;             // [T][Hq][512]
  float* part;            // [units * splits][heads per unit][516]: O, max, sum (rows 16-byte aligned)
  int32_t num_slots;
  int32_t T;
  int32_t Hq;
  int32_t topk;
  int32_t HB;             // head blocks per query token (units = T * HB)
  int32_t splits;         // workgroups per unit (each takes per_split list entries); > 1: a merge launch follows
  int32_t per_split;
  float qk_scale_log2;    // sm_scale * g * log2(e)
  float v_scale;          // g
};

// Launch geometry and workspace of a sparse-MLA decode call.
struct MlaGeometry {
  int32_t waves;          // waves per workgroup (16 heads each)
  int32_t HB;
  int32_t splits;
  int32_t per_split;
  size_t workspace_bytes; // partials of split lists (0 when no list is split)
};
MlaGeometry mla_geometry(int32_t T, int32_t Hq, int32_t topk);

hipError_t launch_mla_decode(const MlaDecodeParams& p, int32_t waves, hipStream_t stream);

}  // namespace nvfp4kv
