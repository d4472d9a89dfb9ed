// Measurement utility: a plain streaming read of a device buffer, the achievable HBM read
// rate that the decode kernels are compared with (the second denominator of their
// roofline, next to the published peak).

#include <hip/hip_runtime.h>

#include "../../include/pkv.h"

#include "pkv_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 8;   // 16-byte loads in flight per thread per step

// Grid-stride sweep of 16-byte non-temporal loads; every thread folds what it read into
// one word (XOR of all words) so the loads cannot be dropped, and writes it to sink.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * kUnroll;
  unsigned acc = 0;
  for (size_t base = (size_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * blockDim.x;
      const u32x4 z = {0u, 0u, 0u, 0u};
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : z;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int32_t pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                   size_t sink_words, int32_t workgroups, hipStream_t stream) {
  if (!buf || !sink) return PKV_ERR_NULL;
  if (bytes == 0 || bytes % 16 || workgroups < 0 || workgroups > 65535) return PKV_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf) & 15u) return PKV_ERR_ALIGN;
  int wg = workgroups;
  if (wg == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return PKV_ERR_LAUNCH;
    wg = cus * 8;
  }
  if (sink_words < (size_t)wg * 256) return PKV_ERR_WORKSPACE;
  hipLaunchKernelGGL(stream_read_kernel, dim3(wg), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
