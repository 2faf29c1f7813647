// A streaming copy for measuring the HBM ceilings that the layer's bandwidth-bound kernels are
// reported against (a benchmark helper, not a step of the layer).  Each lane keeps four 16-byte
// non-temporal loads in flight, then stores them; a null source writes zeros (write-only).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kda_launch.h"

namespace kda {
namespace {

constexpr int MS_NT = 256;
constexpr int MS_UNROLL = 4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(MS_NT) void kda_stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                               long long n) {
  const long long stride = (long long)gridDim.x * MS_NT;
  long long i = (long long)blockIdx.x * MS_NT + threadIdx.x;
  for (; i + (MS_UNROLL - 1) * stride < n; i += MS_UNROLL * stride) {
    u32x4 v[MS_UNROLL];
#pragma unroll
    for (int u = 0; u < MS_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < MS_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(MS_NT) void kda_stream_fill_kernel(u32x4* __restrict__ dst, long long n) {
  const long long stride = (long long)gridDim.x * MS_NT;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (long long i = (long long)blockIdx.x * MS_NT + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(z, dst + i);
}

}  // namespace

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const long long n = (long long)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int cus = device_cus();
  const long long want = (n + (long long)MS_NT * MS_UNROLL - 1) / ((long long)MS_NT * MS_UNROLL);
  const unsigned grid = (unsigned)std::max<long long>(1, std::min<long long>(want, 8LL * cus));
  if (src != nullptr)
    kda_stream_copy_kernel<<<grid, MS_NT, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  else
    kda_stream_fill_kernel<<<grid, MS_NT, 0, s>>>(static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace kda
