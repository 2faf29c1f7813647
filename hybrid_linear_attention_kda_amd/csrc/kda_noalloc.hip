// Scratch for kda_prefill_noalloc: the matrix-core prefill's workspace (the chunk tile blocks its
// chunk-parallel kernel writes and its state pass reads, the pre-norm output o, the spare row slot)
// taken from a fixed array of the library instead of the caller's buffer, for callers that cannot
// allocate device memory.
//
// Host code never uses the array's name as an address: the name is a host-side stand-in.  The
// device address of each GPU's copy is looked up once per device (with that device current) and
// kept; every kernel argument uses that address.  The array is not cleared: the prefill writes
// every byte of it that it later reads within the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
