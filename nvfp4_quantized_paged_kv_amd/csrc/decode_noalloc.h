// Scratch of the allocation-free decode entry point (nvfp4_paged_decode_attn_noalloc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace nvfp4kv {

// A device array of kNoAllocScratchBytes per GPU: arrival counters in the
// first kNoAllocCounterBytes (one int32 per (sequence, kv head) unit), split
// partials after them.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr size_t kNoAllocCounterBytes = (size_t)64 << 10;

// The current device's scratch address: looked up with hipGetSymbolAddress,
// and its counters cleared by a fill kernel on `stream`, on the first call on
// that device; kept per device afterwards.
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);

}  // namespace nvfp4kv
