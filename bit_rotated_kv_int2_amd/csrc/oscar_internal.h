// Internal declarations shared by the translation units of liboscar.so.
// Geometry of the page block and the bf16 / metadata helpers used on the device.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kD = OSCAR_HEAD_DIM;          // head dimension
constexpr int kPageTokens = OSCAR_PAGE_TOKENS;
constexpr int kGroup = OSCAR_GROUP;
constexpr int kPageBytes = OSCAR_PAGE_BYTES;
constexpr int kKCodes = OSCAR_PAGE_KCODES;
constexpr int kVCodes = OSCAR_PAGE_VCODES;
constexpr int kKMeta = OSCAR_PAGE_KMETA;
constexpr int kVMeta = OSCAR_PAGE_VMETA;
constexpr int kMaxGroupHeads = 16;          // Hq / Hkv supported
constexpr int kPartStride = 132;            // floats per partial: m, l, 2 pad, o[128]
constexpr int kPartO = 4;                   // offset of o in a partial (16-byte aligned)
constexpr int kMaxPrefixPages = 131072;     // shared-prefix pages (128 chunks of at most 1024)
constexpr int kTileTokens = 16;             // BF16 window tokens per decode tile

// Bit reversal of a 7-bit channel index (d = 128).
__host__ __device__ constexpr int bitrev7(int p) {
  return ((p & 1) << 6) | ((p & 2) << 4) | ((p & 4) << 2) | (p & 8) | ((p & 16) >> 2) |
         ((p & 32) >> 4) | ((p & 64) >> 6);
}

// Metadata entry (4 bytes) of token slot t: slots t, t+16, t+32, t+48 are
// adjacent so a lane owning slot-column t&15 reads its four tokens with one
// 16-byte load.
__host__ __device__ constexpr int meta_entry(int slot) { return 4 * (slot & 15) + (slot >> 4); }
// Grid steps of the 8-bit metadata of a head with clip threshold tau: a
// group's zero is z8 * zero_step - tau, its scale s8 * scale_step.
__device__ __forceinline__ float meta_zero_step(float tau) { return __fdiv_rn(tau + tau, 255.0f); }
__device__ __forceinline__ float meta_scale_step(float tau) { return __fdiv_rn(tau + tau, 765.0f); }
// Byte (within a 16-byte V channel row) that holds token slot t; bits 2*(t&3).
__host__ __device__ constexpr int vcode_byte(int slot) { return 4 * ((slot >> 2) & 3) + (slot >> 4); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Orders LDS traffic between the lanes of one wave (compiler fence plus the
// hardware wait); waves never wait for each other here.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Cross-workgroup hand-off without cache flushes.  Partials and counters that
// another workgroup (possibly on another XCD, with its own L2) reads are moved
// with agent-scope relaxed atomics, which are coherent at the memory side;
// a writer waits for its stores to complete (vmcnt 0) before the counter
// increment, so no L2 write-back or invalidate is needed.
__device__ __forceinline__ void st_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Buffer resource of n bytes at p for 16-byte device-coherent loads
// (out-of-range offsets read 0); word 3 = raw 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float *p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), 0, (int)n, 0x00020000);
}
// Four floats at byte offset voff + soff of a buffer, device-coherent
// (cache policy SC1, as an agent-scope atomic load).
__device__ __forceinline__ float4 ld_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 16));
}
// Two adjacent floats (8-byte aligned) in one device-coherent load.
__device__ __forceinline__ float2 ld_coherent2(const float *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void stores_complete() { __builtin_amdgcn_s_waitcnt(0); }
// Returns true in every thread of the workgroup that arrives last of `total`
// at counter *c, and resets the counter for the next call.
__device__ __forceinline__ bool arrive_last(int *c, int total, int *flag_lds) {
  stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == total - 1;
    if (last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_lds = last;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// Everything a kernel needs from oscar_params / oscar_kv_pool / oscar_rotation,
// flattened into one by-value struct.
struct PoolView {
  uint16_t *sink_k, *sink_v, *recent_k, *recent_v;
  uint8_t *pages;
  const int32_t *block_table, *sink_slot;
  int32_t *seq_lens, *err, *app_cnt;
  int32_t batch, max_pages, n_pages, n_sink_slots;
  int32_t hkv, hq, sink, recent;
  float sm_scale;
};

struct RotView {
  const float *U_K, *U_V, *tau_K, *tau_V;
  const uint32_t *lev_K, *lev_V;   // codebooks (NULL: uniform grid)
};

// The codebook word (byte k = n_k) of KV head h, key or value tensor.
__device__ __forceinline__ uint32_t levels_of(const RotView &rv, int h, bool is_v) {
  const uint32_t *p = is_v ? rv.lev_V : rv.lev_K;
  return p ? p[h] : OSCAR_UNIFORM_LEVELS;
}

// Code of a normalised group value u = (x - zero) / scale: the nearest of the
// four levels n_k / 32, thresholds at the midpoints (n_k + n_{k+1}) / 64
// (exact in float32), a tie at the middle threshold going up and at the outer
// ones down.  On the uniform grid this is rint(u) clamped to [0, 3].
struct CodeThresholds {
  float t0, t1, t2;
};
__host__ __device__ inline CodeThresholds code_thresholds(uint32_t lev) {
  const float n0 = (float)(lev & 0xFFu), n1 = (float)((lev >> 8) & 0xFFu);
  const float n2 = (float)((lev >> 16) & 0xFFu), n3 = (float)(lev >> 24);
  return CodeThresholds{(n0 + n1) * (1.0f / 64.0f), (n1 + n2) * (1.0f / 64.0f), (n2 + n3) * (1.0f / 64.0f)};
}
__host__ __device__ inline uint32_t level_code(float u, const CodeThresholds &t) {
  return (uint32_t)(u > t.t0) + (uint32_t)(u >= t.t1) + (uint32_t)(u > t.t2);
}

// level_code(fl(a / s), th) for s > 0 as three comparisons of a with float
// cutoffs.  Each term of level_code is "fl(a / s) >= T" for one float T
// (u > t is u >= nextafter(t, +inf)).  Rounding is monotone, so the term
// holds from some float a on: fl(q) >= T exactly when q exceeds the
// midpoint m of prev(T) and T, or equals it and the tie goes to T (T has an
// even last bit).  m s is exact in float64 (25 x 24 significant bits), so
// the term is a >= B with B = m s, or a > B when the tie goes down, and the
// cutoff is the smallest float not below that bound.
__host__ __device__ inline uint32_t float_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
struct CodeCuts {
  double m[3];     // midpoints of prev(T) and T
  bool up[3];      // the tie at m rounds to T
};
__host__ __device__ inline CodeCuts code_cuts(const CodeThresholds &th) {
  const float T[3] = {nextafterf(th.t0, INFINITY), th.t1, nextafterf(th.t2, INFINITY)};
  CodeCuts c;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    c.m[j] = 0.5 * ((double)nextafterf(T[j], -INFINITY) + (double)T[j]);
    c.up[j] = (float_bits(T[j]) & 1u) == 0;
  }
  return c;
}
// Cutoff of term j for scale s > 0: the smallest float a with a >= m s (tie
// up) or a > m s (tie down).
__host__ __device__ inline float code_cut(const CodeCuts &c, int j, float s) {
  double b = c.m[j] * (double)s;
  if (!c.up[j]) b = nextafter(b, (double)INFINITY);
  float f = (float)b;
  if ((double)f < b) f = nextafterf(f, INFINITY);
  return f;
}

// Decode workspace carve-up (offsets in bytes from the workspace base).
struct DecodePlan {
  int n_splits;          // history splits per (sequence, kv head)
  int n_parts;           // partials per (sequence, kv head)
  int n_chunks;          // 16-token BF16 tiles (sink + recent window)
  int pages_per_split;
  int prefix_pages;      // shared-prefix pages (0: none)
  int n_prefix;          // shared-prefix chunks, one partial each per (sequence, kv head)
  int prefix_per_chunk;  // pages per shared-prefix chunk
  size_t off_counters;   // int [B*Hkv] completion counters, zero between calls
  size_t off_qconst;     // float [B*Hkv][GH][4] (VALU variant)
  size_t off_qrot;       // float [B*Hkv][GH][128] (VALU variant)
  size_t off_part;       // float partials [B*Hkv][n_parts][G][kPartStride]:
                         // history splits, shared-prefix chunks, BF16 tiles
  size_t off_pq;         // shared prefix: query operands [B*Hkv] (see prefix_prep_kernel)
  size_t total;
};

// blocks: scan workgroups the grid aims for (0 = the default, one per CU);
// prefix_pages: leading history pages shared by every sequence (0: none).
DecodePlan make_decode_plan(int batch, int hkv, int hq, int max_pages, int sink, int recent,
                            int variant, int blocks, int prefix_pages);

// Launchers (return hipError_t of the launches).
hipError_t launch_append(const PoolView &pv, const RotView &rv, const uint16_t *k_new,
                         const uint16_t *v_new, int n_new, hipStream_t s);
// ws: base of the plan's offsets; counters: the plan's completion counters
// (ws + plan.off_counters for a caller's workspace).
hipError_t launch_decode(const PoolView &pv, const RotView &rv, const uint16_t *q, float *out,
                         uint8_t *ws, int *counters, const DecodePlan &plan, int variant, hipStream_t s);
// Device address of the library's own decode buffer on the current device
// (OSCAR_NOALLOC_SCRATCH_BYTES): counters in the first noalloc_counter_bytes(),
// the rest free for one call's query operands and partials.  The first call
// on a device looks the address up and enqueues a clear of the counters on s.
hipError_t noalloc_scratch(hipStream_t s, uint8_t **base);
size_t noalloc_counter_bytes();

struct Bf16View {
  const uint16_t *k_pages, *v_pages;
  const int32_t *block_table, *seq_lens;
  int32_t *err;
  int32_t batch, max_pages, n_pages, hkv, hq;
  float sm_scale;
};
struct Bf16Plan {
  int n_splits, pages_per_split;
  size_t off_counters, off_part, total;
};
Bf16Plan make_bf16_plan(int batch, int hkv, int hq, int max_pages);
hipError_t launch_bf16_decode(const Bf16View &v, const uint16_t *q, float *out, uint8_t *ws,
                              const Bf16Plan &plan, hipStream_t s);

// Host Lloyd-Max codebook of one tensor (float64 iteration).
int calibrate_codebook_host(int d, int hkv, const float *U, const float *tau, const float *x_cal, int64_t n,
                            uint32_t *levels, char *err, size_t err_len);

// Host calibration (float64).
int calibrate_host(int d, int hkv, int hq, float sm_scale, const float *q_cal, int64_t n_q,
                   const float *k_cal, const float *v_cal, int64_t n_kv, double quantile_k,
                   double quantile_v, float *U_K, float *U_V, float *tau_K, float *tau_V,
                   char *err, size_t err_len);

}  // namespace oscar
