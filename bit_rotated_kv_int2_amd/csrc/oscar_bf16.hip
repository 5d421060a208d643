// In-house BF16 decode attention on a paged all-BF16 KV cache: the baseline
// every INT2 speedup is measured against (the pages compare OSCAR's INT2
// history against a BF16 KV cache: [A] youleyou.com article on OSCAR, section
// "系统加速效果"; [B] MarkTechPost (zh) "Together AI 开源 OSCAR…", section "结果").
//
// Split-K over 64-token pages, four waves per workgroup on interleaved pages.
//   QK on the matrix cores: v_mfma_f32_16x16x32_bf16, rows = query heads
//   (up to 16), columns = 16 tokens, K = 128 channels; the bf16 query and
//   keys are used as stored, products accumulate in float32.
//   PV on the VALU in float32: lane (c8, tq) owns channels 8 c8 .. 8 c8 + 7
//   and every fourth token, so each V row is read with 16-byte loads.
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

struct Bf16Args {
  Bf16View v;
  const uint16_t *q;
  float *part;
  int n_splits, pages_per_split;
};

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

template <int GH>   // GH >= G: heads per KV head, rounded up
__global__ void __launch_bounds__(256) bf16_decode_kernel(Bf16Args a) {
  const Bf16View &cv = a.v;
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int G = cv.hq / cv.hkv;
  const int L = cv.seq_lens[b];
  const int n_pages = (L + kPageTokens - 1) / kPageTokens;
  const int pg0 = split * a.pages_per_split;
  const int pg1 = min(n_pages, pg0 + a.pages_per_split);

  __shared__ float ps[4][kMaxGroupHeads][kPageTokens + 4];
  __shared__ float sm_m[4][kMaxGroupHeads], sm_l[4][kMaxGroupHeads];
  __shared__ float sm_o[4][kMaxGroupHeads][kD];

  // A operand: row = head (n), kgroup q, kstep ks: channels 32 q + 8 ks .. +8.
  v8bf Aq[4];
  {
    const int h = n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = {0, 0, 0, 0};
      if (h < G) u = *(const uint4 *)(a.q + ((size_t)b * cv.hq + kv * G + h) * kD + 32 * q + 8 * ks);
      Aq[ks] = as_v8bf(u);
    }
  }
  // running softmax per head (head = 4 q + i in the C layout, replicated)
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  // PV accumulators: lane (c8 = n, tq = q): channels 8 n .. 8 n + 7, all heads
  float o[GH][8];
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
  float mrow[GH];     // running max of every head, for PV rescaling
#pragma unroll
  for (int h = 0; h < GH; ++h) mrow[h] = -INFINITY;
  const float sl2 = cv.sm_scale * kLog2e;
  bool bad = false;

  for (int pgi = pg0 + wave; pgi < pg1; pgi += 4) {
    if (pgi >= cv.max_pages) {
      bad = true;
      break;
    }
    const int phys = cv.block_table[(size_t)b * cv.max_pages + pgi];
    if (phys < 0 || phys >= cv.n_pages) {
      bad = true;
      continue;
    }
    const int valid = min(kPageTokens, L - pgi * kPageTokens);
    const size_t base = ((size_t)phys * cv.hkv + kv) * kPageTokens * kD;
    const uint16_t *K = cv.k_pages + base;
    const uint16_t *V = cv.v_pages + base;

    // ---- logits: 4 tiles of 16 tokens ----
    float lg[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint16_t *kr = K + (size_t)(16 * tt + n) * kD + 32 * q;
      v4f C = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v8bf Bk = as_v8bf(*(const uint4 *)(kr + 8 * ks));
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aq[ks], Bk, C, 0, 0, 0);
      }
      const bool ok = (16 * tt + n) < valid;
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[tt][i] = ok ? C[i] * sl2 : -INFINITY;
    }
    // per head (row 4 q + i): page max over tokens (tt and 16 lanes n)
    float pm[4], e[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = fmaxf(fmaxf(lg[0][i], lg[1][i]), fmaxf(lg[2][i], lg[3][i]));
      v = fmaxf(v, __shfl_xor(v, 1, 64));
      v = fmaxf(v, __shfl_xor(v, 2, 64));
      v = fmaxf(v, __shfl_xor(v, 4, 64));
      v = fmaxf(v, __shfl_xor(v, 8, 64));
      const float mn = fmaxf(m[i], v);
      const float al = __builtin_amdgcn_exp2f(m[i] - mn);
      float s = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        e[tt][i] = __builtin_amdgcn_exp2f(lg[tt][i] - mn);
        s += e[tt][i];
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      s += __shfl_xor(s, 8, 64);
      l[i] = l[i] * al + s;
      m[i] = mn;
      pm[i] = mn;
      const int h = 4 * q + i;
      if (h < G) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ps[wave][h][16 * tt + n] = e[tt][i];
      }
    }
    // share the new running max of each head with the PV lanes
    wave_lds_sync();
    float mh[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      // head h lives in lanes 16 (h >> 2) .. in C row i = h & 3
      const int src = 16 * (h >> 2);
      const int i = h & 3;
      float v = (i == 0) ? pm[0] : (i == 1) ? pm[1] : (i == 2) ? pm[2] : pm[3];
      mh[h] = __shfl(v, src, 64);
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      if (h >= G) break;
      const float al = __builtin_amdgcn_exp2f(mrow[h] - mh[h]);
      mrow[h] = mh[h];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] *= al;
    }
    // ---- PV: lane (n = channel octet, q = token phase) ----
    for (int t = q; t < valid; t += 4) {
      const uint4 u = *(const uint4 *)(V + (size_t)t * kD + 8 * n);
      float vf[8];
      vf[0] = __uint_as_float(u.x << 16);
      vf[1] = __uint_as_float(u.x & 0xFFFF0000u);
      vf[2] = __uint_as_float(u.y << 16);
      vf[3] = __uint_as_float(u.y & 0xFFFF0000u);
      vf[4] = __uint_as_float(u.z << 16);
      vf[5] = __uint_as_float(u.z & 0xFFFF0000u);
      vf[6] = __uint_as_float(u.w << 16);
      vf[7] = __uint_as_float(u.w & 0xFFFF0000u);
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        if (h >= G) break;
        const float p = ps[wave][h][t];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = fmaf(p, vf[i], o[h][i]);
      }
    }
    wave_lds_sync();
  }
  if (bad && lane == 0 && cv.err) atomicOr(cv.err, OSCAR_DEVERR_PAGE);

  // combine: PV partial sums over the 4 token phases q, then the 4 waves
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    if (h >= G) break;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = o[h][i];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      o[h][i] = v;
    }
  }
  if (q == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      if (h >= G) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_o[wave][h][8 * n + i] = o[h][i];
    }
  }
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q + i;
      if (h < G) {
        sm_m[wave][h] = m[i];
        sm_l[wave][h] = l[i];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, c = idx % kD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float ov = 0.f, lv = 0.f;
    if (M > -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (sm_m[w][h] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
        ov += sc * sm_o[w][h][c];
        lv += sc * sm_l[w][h];
      }
    }
    float *dst = a.part + ((((size_t)b * cv.hkv + kv) * a.n_splits + split) * G + h) * kPartStride;
    if (c == 0) {
      dst[0] = M;   // log2 units
      dst[1] = lv;
    }
    dst[2 + c] = ov;
  }
}

// grid (Hq, batch), block 128: merge the split partials of one query head.
__global__ void __launch_bounds__(128) bf16_merge_kernel(Bf16View cv, const float *part, float *out,
                                                         int n_splits) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int G = cv.hq / cv.hkv;
  const int kv = hq / G, h = hq % G;
  auto P = [&](int s) { return part + ((((size_t)b * cv.hkv + kv) * n_splits + s) * G + h) * kPartStride; };
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, P(s)[0]);
  float o = 0.f, l = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float *p = P(s);
      if (p[0] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(p[0] - M);
      o += w * p[2 + c];
      l += w * p[1];
    }
  }
  out[((size_t)b * cv.hq + hq) * kD + c] = (l > 0.f) ? o / l : 0.f;
}

}  // namespace

Bf16Plan make_bf16_plan(int batch, int hkv, int hq, int max_pages) {
  (void)hq;
  Bf16Plan p{};
  const long work = (long)batch * hkv * (max_pages > 0 ? max_pages : 1);
  int pps = (int)((work + 2047) / 2048);
  pps = pps < 4 ? 4 : pps;
  p.pages_per_split = pps;
  p.n_splits = max_pages > 0 ? (max_pages + pps - 1) / pps : 1;
  p.off_part = 0;
  const int G = hq / hkv;
  p.total = ((size_t)batch * hkv * p.n_splits * G * kPartStride * sizeof(float) + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_bf16_decode(const Bf16View &v, const uint16_t *q, float *out, uint8_t *ws,
                              const Bf16Plan &plan, hipStream_t s) {
  float *part = (float *)(ws + plan.off_part);
  Bf16Args a{v, q, part, plan.n_splits, plan.pages_per_split};
  const dim3 grid(plan.n_splits, v.hkv, v.batch), block(256);
  const int G = v.hq / v.hkv;
  if (G <= 4) hipLaunchKernelGGL(bf16_decode_kernel<4>, grid, block, 0, s, a);
  else if (G <= 8) hipLaunchKernelGGL(bf16_decode_kernel<8>, grid, block, 0, s, a);
  else if (G <= 12) hipLaunchKernelGGL(bf16_decode_kernel<12>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(bf16_decode_kernel<16>, grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bf16_merge_kernel, dim3(v.hq, v.batch), dim3(128), 0, s, v, (const float *)part, out,
                     plan.n_splits);
  return hipGetLastError();
}

}  // namespace oscar
