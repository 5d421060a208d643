// Plain streaming read of a device buffer: the practical HBM read rate that
// the history scan's bandwidth is compared against (a measurement aid, not
// part of the attention path).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

// Every thread reads kProbeUnroll 16-byte words per step, the words of one
// step kProbeThreads apart (each load instruction of a wave covers 1 KB);
// the grid strides over the buffer.  The xor of the words goes to sink so
// the loads are not removed.
__global__ void __launch_bounds__(kProbeThreads) stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                                   uint32_t *sink) {
  const size_t step = (size_t)gridDim.x * kProbeThreads * kProbeUnroll;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x;
       i + (size_t)(kProbeUnroll - 1) * kProbeThreads < n16; i += step) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = p[i + (size_t)u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

int probe_threads() { return kProbeThreads; }

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4 *)buf, bytes / 16,
                     sink);
  return hipGetLastError();
}

}  // namespace oscar
