// Fused write path: rotate, clip, quantise, pack and demote tokens leaving the
// BF16 recent window into rotated-INT2 history pages.
//
// Sources: [A] youleyou.com article on OSCAR, token-pool paragraph under
// "OSCAR 的设计思路" (new tokens enter the recent window; the oldest recent
// token is rotated/clipped/quantised/packed by a fused kernel and demoted;
// four 2-bit codes per byte).  [B] MarkTechPost (zh) "Together AI 开源 OSCAR…",
// section "服务系统：混合精度缓存布局" (clip to the calibrated threshold, then
// per-token asymmetric INT2 with 64-channel groups) and section
// "OSCAR 有何不同做法" (R = U · H_Had · P_br).
//
// Arithmetic order (fixed so that codes and fp16 metadata are reproducible
// bit for bit by any implementation that follows it):
//   S1 y_j = sum_k x_k U[k][j], float64, k ascending (bf16 x float32
//      products are exact in float64, so fma == multiply-then-add);
//   S2 radix-2 butterfly, stages h = 1..64, (a, b) -> (a + b, a - b), float64;
//   S3 multiply by the float64 nearest to 1/sqrt(128);
//   S4 output channel p takes butterfly output bitrev(p);
//   S5 round to float32; S6 clamp to [-tau, tau];
//   S7 per 64-channel group: s = (max - min) / 3 (float32 IEEE),
//      scale = fp16(s), zero = fp16(min), code = clamp(rint((x - zero)/scale),
//      0, 3) in float32 with the stored values, all codes 0 if scale == 0.
#include "oscar_internal.h"

#pragma clang fp contract(off)

namespace oscar {
namespace {

constexpr int kChunk = 16;        // history slots per workgroup (aligned to 16)
constexpr int kThreads = 128;     // one thread per channel
constexpr double kInvSqrtD = 0x1.6a09e667f3bcdp-4;  // nearest double to 1/sqrt(128)

struct AppendArgs {
  PoolView pv;
  RotView rv;
  const uint16_t *k_new, *v_new;
  int n_new;
};

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// S6..S8 for output channel p of one token (this thread; the wave holds the
// 64 channels of one group): clamp, group scale/zero, code.  Lane 0 of the
// group writes the fp16 {scale, zero} pair to meta[group].
__device__ __forceinline__ uint32_t quantize_code(float v, float tau, int p, uint32_t *meta) {
  v = fminf(fmaxf(v, -tau), tau);
  const float mx = wave_max(v), mn = wave_min(v);
  const float s = __fdiv_rn(mx - mn, 3.0f);
  const uint16_t s16 = f32_to_f16_rn(s), z16 = f32_to_f16_rn(mn);
  const float sf = f16_to_f32(s16), zf = f16_to_f32(z16);
  uint32_t code = 0;
  if (sf != 0.0f) {
    float r = rintf(__fdiv_rn(v - zf, sf));
    r = fminf(fmaxf(r, 0.0f), 3.0f);
    code = (uint32_t)r;
  }
  if ((p & 63) == 0) meta[p >> 6] = (uint32_t)s16 | ((uint32_t)z16 << 16);
  return code;
}

// grid: (chunks, Hkv * 2, batch); block: 128 threads (thread j = channel j).
// Demotes every position x with max(S0, p0 - W) <= x < p0 + n_new - W.
__global__ void __launch_bounds__(kThreads) append_demote_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  const int b = blockIdx.z;
  const int h = blockIdx.y >> 1;
  const int is_v = blockIdx.y & 1;
  const int j = threadIdx.x;
  const int p0 = pv.seq_lens[b];
  if (p0 < 0) return;                                       // flagged by the store kernel
  const int L = p0 + a.n_new;
  const int xa = max(pv.sink, p0 - pv.recent);
  const int xb = L - pv.recent;
  if (xb <= xa) return;
  const int ha = xa - pv.sink, hb = xb - pv.sink;           // history index range
  const int c0 = (ha / kChunk) * kChunk + blockIdx.x * kChunk;
  const int t0 = max(c0, ha), t1 = min(c0 + kChunk, hb);
  if (t1 <= t0) return;
  const int nt = t1 - t0;

  const int page_idx = c0 / kPageTokens;
  if (page_idx >= pv.max_pages) {
    if (j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    return;
  }
  const int phys = pv.block_table[(size_t)b * pv.max_pages + page_idx];
  if (phys < 0 || phys >= pv.n_pages) {
    if (j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
    return;
  }

  __shared__ double xs[kChunk][kD];
  __shared__ double ys[kChunk][kD + 1];

  // Gather the bf16 sources: ring slot for old recent tokens, input otherwise.
  const uint16_t *ring = is_v ? pv.recent_v : pv.recent_k;
  const uint16_t *fresh = is_v ? a.v_new : a.k_new;
  for (int t = 0; t < nt; ++t) {
    const int x = t0 + t + pv.sink;
    uint16_t bits;
    if (x < p0)
      bits = ring[(((size_t)b * pv.hkv + h) * pv.recent + (x % pv.recent)) * kD + j];
    else
      bits = fresh[(((size_t)b * a.n_new + (x - p0)) * pv.hkv + h) * kD + j];
    xs[t][j] = (double)bf16_to_f32(bits);
  }
  __syncthreads();

  // S1: projection onto the eigenbasis, float64, k ascending.
  const float *U = (is_v ? a.rv.U_V : a.rv.U_K) + (size_t)h * kD * kD;
  double acc[kChunk];
#pragma unroll
  for (int t = 0; t < kChunk; ++t) acc[t] = 0.0;
  for (int k = 0; k < kD; ++k) {
    const double u = (double)U[k * kD + j];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) acc[t] = fma(xs[t][k], u, acc[t]);
  }
#pragma unroll
  for (int t = 0; t < kChunk; ++t) ys[t][j] = acc[t];
  __syncthreads();

  // S2: butterfly.  Thread j owns pair (j & 63) for tokens with parity j >> 6.
  for (int hs = 1; hs < kD; hs <<= 1) {
    const int pr = j & 63;
    const int i0 = (pr / hs) * (2 * hs) + (pr % hs);
    for (int t = j >> 6; t < nt; t += 2) {
      const double x0 = ys[t][i0], x1 = ys[t][i0 + hs];
      ys[t][i0] = x0 + x1;
      ys[t][i0 + hs] = x0 - x1;
    }
    __syncthreads();
  }

  // S3..S8 per token; thread j = output channel p, wave = quantisation group.
  const float tau = (is_v ? a.rv.tau_V : a.rv.tau_K)[h];
  const int p = j;
  uint8_t *page = pv.pages + ((size_t)phys * pv.hkv + h) * kPageBytes;
  uint32_t vbytes[4] = {0, 0, 0, 0};   // V: the 4 bytes of channel p this chunk touches
  uint32_t vmask[4] = {0, 0, 0, 0};
  for (int t = 0; t < nt; ++t) {
    const int slot = (t0 + t) % kPageTokens;
    const float v = (float)(ys[t][bitrev7(p)] * kInvSqrtD);
    const uint32_t code = quantize_code(v, tau, p, (uint32_t *)(page + (is_v ? kVMeta : kKMeta) + meta_entry(slot) * 8));
    if (!is_v) {
      // K codes: byte p/4 of the token row, four neighbouring lanes combine.
      uint32_t c = code << (2 * (p & 3));
      c |= __shfl_xor(c, 1, 64);
      c |= __shfl_xor(c, 2, 64);
      if ((p & 3) == 0) page[kKCodes + slot * 32 + (p >> 2)] = (uint8_t)c;
    } else {
      const int m = (slot >> 2) & 3;   // chunks are 16-aligned: slot >> 4 fixed
      vbytes[m] |= code << (2 * (slot & 3));
      vmask[m] |= 3u << (2 * (slot & 3));
    }
  }
  if (is_v) {
    const int a16 = (t0 % kPageTokens) >> 4;
    uint8_t *row = page + kVCodes + p * 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (!vmask[m]) continue;
      uint8_t *dst = row + 4 * m + a16;
      uint32_t val = vbytes[m];
      if (vmask[m] != 0xFF) val = (*dst & ~vmask[m]) | val;   // partial byte: keep other slots
      *dst = (uint8_t)val;
    }
  }
}

// Single-token append, one launch.  grid: (Hkv * 2, batch); block: 128
// (thread j = channel j).  Block (h, K|V) of sequence b stores the new token
// of head h (sink, or ring slot p0 mod W) and demotes the ring token that slot
// held when it leaves the window; the last of the sequence's 2 Hkv blocks
// (counted in app_cnt[b], which it resets) advances seq_lens[b].
__global__ void __launch_bounds__(kThreads) append_one_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  const int b = blockIdx.y, h = blockIdx.x >> 1, is_v = blockIdx.x & 1;
  const int j = threadIdx.x;
  const int p0 = pv.seq_lens[b];
  __shared__ double xs[kD];
  __shared__ double ys[kD];
  if (p0 >= 0) {
    const uint16_t nb = (is_v ? a.v_new : a.k_new)[((size_t)b * pv.hkv + h) * kD + j];
    bool demote = false;
    uint16_t old = 0;
    if (p0 < pv.sink) {
      const int ss = pv.sink_slot[b];
      if (ss >= 0 && ss < pv.n_sink_slots)
        (is_v ? pv.sink_v : pv.sink_k)[(((size_t)ss * pv.hkv + h) * pv.sink + p0) * kD + j] = nb;
      else if (blockIdx.x == 0 && j == 0 && pv.err)
        atomicOr(pv.err, OSCAR_DEVERR_SINKSLOT);
    } else {
      uint16_t *el = (is_v ? pv.recent_v : pv.recent_k) + (((size_t)b * pv.hkv + h) * pv.recent + p0 % pv.recent) * kD + j;
      demote = p0 - pv.recent >= pv.sink;   // the slot's token leaves the window
      if (demote) old = *el;
      *el = nb;
    }
    int phys = -1;
    if (demote) {
      const int page_idx = (p0 - pv.recent - pv.sink) / kPageTokens;
      if (page_idx >= pv.max_pages) {
        if (j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
      } else {
        phys = pv.block_table[(size_t)b * pv.max_pages + page_idx];
        if (phys < 0 || phys >= pv.n_pages) {
          if (j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
          phys = -1;
        }
      }
    }
    if (phys >= 0) {   // block-uniform
      const int slot = (p0 - pv.recent - pv.sink) % kPageTokens;
      // S1: thread j takes column j of U; all 128 loads are issued together
      const float *U = (is_v ? a.rv.U_V : a.rv.U_K) + (size_t)h * kD * kD + j;
      float u[kD];
#pragma unroll
      for (int k = 0; k < kD; ++k) u[k] = U[(size_t)k * kD];
      xs[j] = (double)bf16_to_f32(old);
      __syncthreads();
      double y = 0.0;
#pragma unroll
      for (int k = 0; k < kD; ++k) y = fma(xs[k], (double)u[k], y);
      // S2: butterfly; stages 1..32 inside the wave, stage 64 through LDS
#pragma unroll
      for (int hs = 1; hs < 64; hs <<= 1) {
        const double o = __shfl_xor(y, hs, 64);
        y = (j & hs) ? o - y : y + o;
      }
      ys[j] = y;
      __syncthreads();
      {
        const double o = ys[j ^ 64];
        y = (j & 64) ? o - y : y + o;
      }
      __syncthreads();
      ys[j] = y;
      __syncthreads();
      // S3..S8: thread j = output channel p
      const int p = j;
      const float tau = (is_v ? a.rv.tau_V : a.rv.tau_K)[h];
      uint8_t *page = pv.pages + ((size_t)phys * pv.hkv + h) * kPageBytes;
      const float v = (float)(ys[bitrev7(p)] * kInvSqrtD);
      const uint32_t code = quantize_code(v, tau, p, (uint32_t *)(page + (is_v ? kVMeta : kKMeta) + meta_entry(slot) * 8));
      if (!is_v) {
        uint32_t c = code << (2 * (p & 3));
        c |= __shfl_xor(c, 1, 64);
        c |= __shfl_xor(c, 2, 64);
        if ((p & 3) == 0) page[kKCodes + slot * 32 + (p >> 2)] = (uint8_t)c;
      } else {
        // one 2-bit field of a byte shared with three other slots
        uint8_t *dst = page + kVCodes + p * 16 + vcode_byte(slot);
        const uint32_t sh = 2 * (slot & 3);
        *dst = (uint8_t)((*dst & ~(3u << sh)) | (code << sh));
      }
    }
  }
  __syncthreads();
  if (j == 0) {
    const int n = atomicAdd(&pv.app_cnt[b], 1);
    if (n == 2 * pv.hkv - 1) {
      pv.app_cnt[b] = 0;
      if (p0 >= 0) pv.seq_lens[b] = p0 + 1;
      else if (pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    }
  }
}

// grid: (batch); block: 256.  Stores new tokens that stay BF16 (sink or the
// final recent window), then advances seq_lens.  Runs after the demote kernel
// on the same stream, so every ring slot has been read before it is reused.
__global__ void __launch_bounds__(256) append_store_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  const int b = blockIdx.x;
  const int p0 = pv.seq_lens[b];
  if (p0 < 0) {
    if (threadIdx.x == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    return;
  }
  const int L = p0 + a.n_new;
  const int sink_slot = pv.sink_slot[b];
  const bool sink_ok = sink_slot >= 0 && sink_slot < pv.n_sink_slots;
  if (!sink_ok && p0 < pv.sink && threadIdx.x == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_SINKSLOT);
  const int n_sink_new = max(0, min(a.n_new, pv.sink - p0));
  const int i_ring0 = max(n_sink_new, L - pv.recent - p0);
  // words of 8 bytes per token row: 128 bf16 = 32 x uint64
  const int words = kD / 4;
  for (int kv = 0; kv < 2; ++kv) {
    const uint64_t *src = (const uint64_t *)(kv ? a.v_new : a.k_new);
    uint64_t *sink = (uint64_t *)(kv ? pv.sink_v : pv.sink_k);
    uint64_t *ring = (uint64_t *)(kv ? pv.recent_v : pv.recent_k);
    if (sink_ok) {
      for (int e = threadIdx.x; e < n_sink_new * pv.hkv * words; e += blockDim.x) {
        const int w = e % words, h = (e / words) % pv.hkv, i = e / (words * pv.hkv);
        const int pos = p0 + i;
        sink[(((size_t)sink_slot * pv.hkv + h) * pv.sink + pos) * words + w] =
            src[(((size_t)b * a.n_new + i) * pv.hkv + h) * words + w];
      }
    }
    const int n_ring = a.n_new - i_ring0;
    for (int e = threadIdx.x; e < n_ring * pv.hkv * words; e += blockDim.x) {
      const int w = e % words, h = (e / words) % pv.hkv, i = i_ring0 + e / (words * pv.hkv);
      const int pos = p0 + i;
      ring[(((size_t)b * pv.hkv + h) * pv.recent + (pos % pv.recent)) * words + w] =
          src[(((size_t)b * a.n_new + i) * pv.hkv + h) * words + w];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) pv.seq_lens[b] = L;
}

}  // namespace

hipError_t launch_append(const PoolView &pv, const RotView &rv, const uint16_t *k_new,
                         const uint16_t *v_new, int n_new, hipStream_t s) {
  AppendArgs a{pv, rv, k_new, v_new, n_new};
  if (n_new == 1 && pv.app_cnt) {
    hipLaunchKernelGGL(append_one_kernel, dim3(pv.hkv * 2, pv.batch), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const int chunks = (n_new + kChunk - 1) / kChunk + 1;
  hipLaunchKernelGGL(append_demote_kernel, dim3(chunks, pv.hkv * 2, pv.batch), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_store_kernel, dim3(pv.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
