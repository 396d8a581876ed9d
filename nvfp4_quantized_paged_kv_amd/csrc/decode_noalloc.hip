// Device-resident scratch for the allocation-free decode entry point
// (nvfp4_paged_decode_attn_noalloc): the arrival counters and split partials
// that nvfp4_paged_decode_attn keeps in its caller's workspace live here in a
// fixed-size array in the library's code object instead, so the call needs no
// allocation from its caller.
//
// Layout: [0, kNoAllocCounterBytes) holds one int32 arrival counter per
// (sequence, kv head) unit -- zero between calls; the decode kernel leaves
// each counter it bumps at zero again -- and the rest holds the partials.
// The counter region is fixed, so a call of any geometry finds zeroed
// counters whatever the partials of earlier calls left behind.
//
// Each GPU holds its own copy of the array until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a stand-in
// for the device symbol): the device address comes from hipGetSymbolAddress,
// once per device with that device current, and is kept per device.
#include <mutex>

#include "decode_noalloc.h"

namespace nvfp4kv {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // clear the counters once, on the first caller's stream (a fill kernel,
    // not a memset, so that a captured first call records no memset node)
    constexpr int words = (int)(kNoAllocCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nvfp4kv
