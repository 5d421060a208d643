// In-house BF16 decode attention on a paged all-BF16 KV cache: the baseline
// every INT2 speedup is measured against (the pages compare OSCAR's INT2
// history with a BF16 KV cache: [A] youleyou.com article on OSCAR, section
// "系统加速效果"; [B] MarkTechPost (zh) "Together AI 开源 OSCAR…", section "结果").
//
// One launch: blocks of 256 threads over (sequence, KV head, split) of the
// 64-token pages; each wave takes every fourth page of its split and runs the
// shared BF16 chunk routine (bf16 MFMA logits, float32 VALU value sums).  The
// last block of a (sequence, KV head) merges the split partials and writes
// the output, so no second launch is needed.  Counters return to zero; the
// workspace must be zero-filled before its first use.
#include "oscar_wave.h"

namespace oscar {
namespace {

struct Bf16Args {
  Bf16View v;
  const uint16_t *q;
  float *out;
  float *part;      // [B*Hkv][n_splits][G][kPartStride]
  int *counters;    // [B*Hkv]
  int n_splits, pages_per_split;
};

template <int GH>
union Bf16BaseSmem {
  struct {
    float ps[4][GH][kPageTokens + 4];
    float m[4][GH], l[4][GH];
    float o[4][GH][kD];
  } w;
  struct {
    float ws[GH][256], M[GH], l[GH];
  } g;
};

template <int GH>
__global__ void __launch_bounds__(256) bf16_decode_kernel(Bf16Args a) {
  const Bf16View &cv = a.v;
  const int BH = cv.batch * cv.hkv;
  const int bh = blockIdx.x % BH, split = blockIdx.x / BH;
  const int b = bh / cv.hkv, kv = bh % cv.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = cv.hq / cv.hkv;
  const int L = max(0, cv.seq_lens[b]);
  const int n_pages = (L + kPageTokens - 1) / kPageTokens;
  const int pg0 = split * a.pages_per_split;
  const int pg1 = min(min(n_pages, pg0 + a.pages_per_split), cv.max_pages);
  if (n_pages > cv.max_pages && split == 0 && tid == 0 && cv.err) atomicOr(cv.err, OSCAR_DEVERR_LENGTH);
  __shared__ Bf16BaseSmem<GH> sm;

  v8bf Aq[4];
  load_bf16_query(a.q + ((size_t)b * cv.hq + (size_t)kv * G) * kD, G, Aq);
  float m[4], l[4], mrow[GH], o[GH][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    mrow[h] = -INFINITY;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[h][c] = 0.f;
  }
  const float sl2 = cv.sm_scale * kLog2e;
  bool bad = false;
  for (int pgi = pg0 + wave; pgi < pg1; pgi += 4) {
    const int phys = cv.block_table[(size_t)b * cv.max_pages + pgi];
    if (phys < 0 || phys >= cv.n_pages) {
      bad = true;
      continue;
    }
    const int valid = min(kPageTokens, L - pgi * kPageTokens);
    const size_t base = ((size_t)phys * cv.hkv + kv) * kPageTokens * kD;
    bf16_chunk<GH>(cv.k_pages + base, cv.v_pages + base, valid, G, Aq, sl2, m, l, mrow, o, sm.w.ps[wave]);
  }
  if (bad && lane == 0 && cv.err) atomicOr(cv.err, OSCAR_DEVERR_PAGE);
  float *parts = a.part + (size_t)bh * a.n_splits * G * kPartStride;
  bf16_block_combine<GH>(G, m, l, o, sm.w.m, sm.w.l, sm.w.o, parts + (size_t)split * G * kPartStride);

  __shared__ int last_flag;
  if (!arrive_last(&a.counters[bh], a.n_splits, &last_flag)) return;
  const int S = a.n_splits;
  for (int h = wave; h < G; h += 4) {
    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, ld_coherent(parts + ((size_t)s * G + h) * kPartStride));
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float lsum = 0.f;
    for (int s = lane; s < S; s += 64) {
      const float *p = parts + ((size_t)s * G + h) * kPartStride;
      const float m0 = ld_coherent(p);
      const float w = (M > -INFINITY && m0 > -INFINITY) ? exp2_fast(m0 - M) : 0.f;
      sm.g.ws[h][s] = w;
      lsum = fmaf(w, ld_coherent(p + 1), lsum);
    }
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
    if (lane == 0) {
      sm.g.M[h] = M;
      sm.g.l[h] = lsum;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, c = idx % kD;
    float o0 = 0.f, o1 = 0.f;
    const float *p = parts + (size_t)h * kPartStride + kPartO + c;
    const size_t st = (size_t)G * kPartStride;
    int s = 0;
    for (; s + 2 <= S; s += 2) {
      o0 = fmaf(sm.g.ws[h][s], ld_coherent(p + (size_t)s * st), o0);
      o1 = fmaf(sm.g.ws[h][s + 1], ld_coherent(p + (size_t)(s + 1) * st), o1);
    }
    if (s < S) o0 = fmaf(sm.g.ws[h][s], ld_coherent(p + (size_t)s * st), o0);
    const float den = sm.g.l[h];
    a.out[((size_t)b * cv.hq + (size_t)kv * G + h) * kD + c] = den > 0.f ? (o0 + o1) / den : 0.f;
  }
}

// workgroups the baseline's split grid aims for (four per CU)
constexpr int kBf16Blocks = 1024;

}  // namespace

Bf16Plan make_bf16_plan(int batch, int hkv, int hq, int max_pages) {
  Bf16Plan p{};
  const int G = hq / hkv;
  const int bh = batch * hkv;
  int S = (kBf16Blocks + bh - 1) / bh;
  const int max_by_pages = max_pages > 0 ? (max_pages + 3) / 4 : 1;
  S = S < 1 ? 1 : S;
  S = S > max_by_pages ? max_by_pages : S;
  S = S > 256 ? 256 : S;
  p.n_splits = S;
  p.pages_per_split = max_pages > 0 ? (max_pages + S - 1) / S : 1;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.off_counters = 0;
  p.off_part = al((size_t)bh * sizeof(int));
  p.total = al(p.off_part + (size_t)bh * S * G * kPartStride * sizeof(float));
  return p;
}

hipError_t launch_bf16_decode(const Bf16View &v, const uint16_t *q, float *out, uint8_t *ws,
                              const Bf16Plan &plan, hipStream_t s) {
  Bf16Args a{v, q, out, (float *)(ws + plan.off_part), (int *)(ws + plan.off_counters), plan.n_splits,
             plan.pages_per_split};
  const dim3 grid(v.batch * v.hkv * plan.n_splits), block(256);
  const int G = v.hq / v.hkv;
  if (G <= 4) hipLaunchKernelGGL(bf16_decode_kernel<4>, grid, block, 0, s, a);
  else if (G <= 8) hipLaunchKernelGGL(bf16_decode_kernel<8>, grid, block, 0, s, a);
  else if (G <= 12) hipLaunchKernelGGL(bf16_decode_kernel<12>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(bf16_decode_kernel<16>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
