// A plain streaming read of a device buffer, for measurement: the HBM read
// bandwidth this GPU reaches with whole-line 16-byte non-temporal loads and
// no other work, the practical ceiling beside the nominal peak that the
// decode kernels' bytes per second are compared with.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_bench.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Workgroup w reads chunks w, w + gridDim.x, ... of kThreads * kUnroll
// 16-byte pieces each: within a chunk, load u of all threads is one
// contiguous 4 KiB run, so every wavefront instruction reads whole lines and
// a workgroup walks 32 KiB of consecutive memory per iteration.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                               int64_t n16, uint32_t* sink) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
  uint32_t acc = 0;
  const int64_t chunks = n16 / kChunk;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const uint4* p = buf + c * kChunk + threadIdx.x;
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + u * kThreads));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = chunks * kChunk + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(buf + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads alive; the store itself (almost) never happens
  if (acc == 0x9e3779b9u) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" pa_status pa_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                          int32_t workgroups, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) ||
      workgroups <= 0)
    return PA_EINVAL;
  if (bytes == 0) return PA_OK;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(buf),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_EHIP;
}
