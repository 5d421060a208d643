// Benchmark helper, not part of liboscar.so: a plain streaming read of a
// device buffer, built into its own library (libbench_probe.so) that only the
// benchmark and its test load.  Its rate is the practical HBM read ceiling
// that the history scan's bandwidth is reported against, next to the
// published peak.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Every thread reads kProbeUnroll 16-byte words per step, the words of one
// step kProbeThreads apart (each load instruction of a wave covers 1 KB);
// the grid strides over the buffer.  The loads carry the non-temporal hint
// (a streaming read: 7.1 TB/s on MI355X against 6.3 TB/s without it).  The
// xor of the words goes to sink so the loads are not removed.
__global__ void __launch_bounds__(kProbeThreads) stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                                   uint32_t *sink) {
  const size_t step = (size_t)gridDim.x * kProbeThreads * kProbeUnroll;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x;
       i + (size_t)(kProbeUnroll - 1) * kProbeThreads < n16; i += step) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const u32x4 w = __builtin_nontemporal_load((const u32x4 *)&p[i + (size_t)u * kProbeThreads]);
      v[u] = make_uint4(w.x, w.y, w.z, w.w);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// One streaming read of `bytes` bytes of buf (16-byte aligned; a tail shorter
// than 32 KB may be skipped) by `grid` workgroups of 512 threads; sink is
// uint32 [grid * 512], overwritten with per-thread checksums.  Enqueued on
// `stream`.  Returns 0, -1 for bad arguments, or a hipError_t value.
int bench_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || grid < 1 || grid > 65536) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     (const uint4 *)buf, bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
