// Decode attention over the mixed-precision pool: query pre-rotation, the
// BF16 sink/recent segment, a VALU INT2 history kernel, and the log-sum-exp
// merge that applies R_V^T once to the merged history output.
//
// Sources: [A] youleyou.com article on OSCAR, token-pool paragraph under
// "OSCAR 的设计思路" (decode splits the cache into a BF16 segment and an INT2
// segment; the INT2 kernel unpacks, restores scale/zero and accumulates in
// float; the BF16 kernel handles sink/recent; an online-softmax merge combines
// them).  [B] MarkTechPost (zh) "Together AI 开源 OSCAR…", section
// "服务系统：混合精度缓存布局" (read path dequantises and inverse-rotates inside
// the attention pass) and section "OSCAR 有何不同做法" (R = U · H_Had · P_br).
//
// Inverse rotation is factored: for a history token with rotated, dequantised
// x~, q · (x~ R^T) = (q R) · x~ and sum_t p_t x~_t R^T = (sum_t p_t x~_t) R^T,
// so the query is rotated once per step and R_V^T is applied once to the
// merged history output.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kInvSqrtDf = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Query pre-rotation: q~ = bitrev(FWHT(q U_K) / sqrt(d)), float32.
// Also the fixed-point copy used by the int8 MFMA kernel:
//   delta = max|q~| / 32639, qi = rint(q~ / delta) in [-32639, 32639],
//   qi = 256 * hi + lo with hi, lo signed bytes, Q_g = delta * sum_{c in g} qi.
// grid (Hq, batch), block 128.
// ---------------------------------------------------------------------------
struct QPrepArgs {
  PoolView pv;
  RotView rv;
  const uint16_t *q;
  float *qrot;       // [B][Hq][128]
  int8_t *qint;      // [B][Hkv][MT][2 ksteps][64 lanes][16]  (may be null)
  float *qconst;     // [B][Hq][4]
  int mtiles;
};

__global__ void __launch_bounds__(128) qprep_kernel(QPrepArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const int G = a.pv.hq / a.pv.hkv;
  const int kv = hq / G;
  __shared__ float qs[kD];
  __shared__ float ys[kD];
  __shared__ float red[2];
  qs[j] = bf16_to_f32(a.q[((size_t)b * a.pv.hq + hq) * kD + j]);
  __syncthreads();
  const float *U = a.rv.U_K + (size_t)kv * kD * kD;
  float y = 0.f;
  for (int k = 0; k < kD; ++k) y = fmaf(qs[k], U[k * kD + j], y);
  ys[j] = y;
  __syncthreads();
  for (int hs = 1; hs < kD; hs <<= 1) {
    float v = 0.f, w = 0.f;
    int i0 = 0;
    if (j < 64) {
      i0 = (j / hs) * (2 * hs) + (j % hs);
      v = ys[i0];
      w = ys[i0 + hs];
    }
    __syncthreads();
    if (j < 64) {
      ys[i0] = v + w;
      ys[i0 + hs] = v - w;
    }
    __syncthreads();
  }
  const float qr = ys[bitrev7(j)] * kInvSqrtDf;
  a.qrot[((size_t)b * a.pv.hq + hq) * kD + j] = qr;

  // fixed-point copy
  float m = fabsf(qr);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((j & 63) == 0) red[j >> 6] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  const float delta = m > 0.f ? m / 32639.0f : 1.0f;
  int qi = (int)rintf(qr / delta);
  qi = max(-32639, min(32639, qi));
  // group sums of qi (exact in int), per 64-channel group = per wave
  int gs = qi;
  for (int o = 32; o > 0; o >>= 1) gs += __shfl_xor(gs, o, 64);
  __syncthreads();
  if ((j & 63) == 0) red[j >> 6] = (float)gs;   // |sum| <= 64 * 32639 < 2^24: exact
  __syncthreads();
  if (j == 0) {
    float *qc = a.qconst + ((size_t)b * a.pv.hq + hq) * 4;
    qc[0] = delta;
    qc[1] = delta * red[0];
    qc[2] = delta * red[1];
    qc[3] = 0.f;
  }
  if (a.qint) {
    const int lo = (int)(int8_t)(qi & 0xFF);
    const int hi = (qi - lo) >> 8;
    // Operand layout for the QK MFMA (see oscar_decode_mfma.hip): M-tile
    // mt = hl / 4 holds rows r = 4 * (hl % 4) + 2 g + part; lane (r, kg) kstep
    // ks element e = 4 s + bb is channel 32 kg + 16 ks + 4 bb + s and is zero
    // unless that channel lies in group g.
    const int hl = hq % G;
    const int mt = hl >> 2;
    const int c = j;
    const int kg = c >> 5, ks = (c >> 4) & 1, bb = (c >> 2) & 3, s = c & 3;
    const int e = 4 * s + bb;
    const int g = c >> 6;
    int8_t *base = a.qint + (((size_t)b * a.pv.hkv + kv) * a.mtiles + mt) * 2 * 64 * 16;
    for (int part = 0; part < 2; ++part) {
      const int r = 4 * (hl & 3) + 2 * g + part;
      const int lane = r + 16 * kg;
      base[(ks * 64 + lane) * 16 + e] = (int8_t)(part == 0 ? hi : lo);
      // the same lane/element in the other group's rows is zero
      const int r0 = 4 * (hl & 3) + 2 * (1 - g) + part;
      base[(ks * 64 + r0 + 16 * kg) * 16 + e] = 0;
    }
  }
}

// Rows of M-tiles that belong to no head (G not a multiple of 4) must be zero.
__global__ void qint_zero_kernel(int8_t *qint, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) qint[i] = 0;
}

// ---------------------------------------------------------------------------
// Shared partial writer: (m, l, o[128]) per head, float.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float *part_ptr(float *base, int b, int kv, int hkv, int n, int idx, int G,
                                           int h) {
  return base + ((((size_t)b * hkv + kv) * n + idx) * G + h) * kPartStride;
}

// ---------------------------------------------------------------------------
// BF16 segment: sink (chunk 0 .. S0/64-1) and recent window chunks.
// grid (n_chunks, Hkv, batch), block 256 (wave w handles heads w, w+4, ...).
// Partials are in the original (unrotated) basis.
// ---------------------------------------------------------------------------
struct Bf16SegArgs {
  PoolView pv;
  const uint16_t *q;
  float *bpart;
  int n_chunks;
};

__global__ void __launch_bounds__(256) bf16_segment_kernel(Bf16SegArgs a) {
  const PoolView &pv = a.pv;
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int G = pv.hq / pv.hkv;
  const int L = pv.seq_lens[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint16_t ks[64][kD + 2];
  __shared__ uint16_t vs[64][kD + 2];
  __shared__ float qsh[kMaxGroupHeads][kD];
  __shared__ float ps[4][64];

  const int n_sink_chunks = pv.sink / 64;
  const int sink_len = min(L, pv.sink);
  const int r0 = max(pv.sink, L - pv.recent);
  int n = 0;                    // valid tokens in this chunk
  int pos0 = 0;
  bool from_sink = chunk < n_sink_chunks;
  if (from_sink) {
    pos0 = chunk * 64;
    n = max(0, min(64, sink_len - pos0));
  } else {
    pos0 = r0 + (chunk - n_sink_chunks) * 64;
    n = max(0, min(64, L - pos0));
  }
  const int slot = pv.sink_slot[b];
  if (from_sink && (slot < 0 || slot >= pv.n_sink_slots)) n = 0;

  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, c = e % kD;
    qsh[h][c] = bf16_to_f32(a.q[((size_t)b * pv.hq + kv * G + h) * kD + c]);
  }
  for (int e = tid; e < n * (kD / 2); e += 256) {
    const int t = e / (kD / 2), w = e % (kD / 2);
    const int pos = pos0 + t;
    size_t row;
    const uint32_t *K, *V;
    if (from_sink) {
      row = (((size_t)slot * pv.hkv + kv) * pv.sink + pos) * kD;
      K = (const uint32_t *)(pv.sink_k + row);
      V = (const uint32_t *)(pv.sink_v + row);
    } else {
      row = (((size_t)b * pv.hkv + kv) * pv.recent + (pos % pv.recent)) * kD;
      K = (const uint32_t *)(pv.recent_k + row);
      V = (const uint32_t *)(pv.recent_v + row);
    }
    const uint32_t kw = K[w], vw = V[w];
    ks[t][2 * w] = kw & 0xFFFF;
    ks[t][2 * w + 1] = kw >> 16;
    vs[t][2 * w] = vw & 0xFFFF;
    vs[t][2 * w + 1] = vw >> 16;
  }
  __syncthreads();

  for (int h = wave; h < G; h += 4) {
    float logit = -INFINITY;
    if (lane < n) {
      float acc = 0.f;
      for (int c = 0; c < kD; ++c) acc = fmaf(qsh[h][c], bf16_to_f32(ks[lane][c]), acc);
      logit = acc * pv.sm_scale;
    }
    float m = logit;
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float p = (lane < n) ? __expf(logit - m) : 0.f;
    float l = p;
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    ps[wave][lane] = p;
    wave_lds_sync();
    float o0 = 0.f, o1 = 0.f;
    for (int t = 0; t < n; ++t) {
      const float pt = ps[wave][t];
      o0 = fmaf(pt, bf16_to_f32(vs[t][2 * lane]), o0);
      o1 = fmaf(pt, bf16_to_f32(vs[t][2 * lane + 1]), o1);
    }
    float *dst = part_ptr(a.bpart, b, kv, pv.hkv, a.n_chunks, chunk, G, h);
    if (lane == 0) {
      dst[0] = (n > 0) ? m : -INFINITY;
      dst[1] = l;
    }
    dst[2 + 2 * lane] = o0;
    dst[3 + 2 * lane] = o1;
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// VALU INT2 history kernel (reference variant).
// grid (n_splits, Hkv, batch), block 256.  Wave w handles heads w, w+4, ...
// Per page: logits lane = token slot; PV lane = channel pair.
// Partials are in the rotated basis.
// ---------------------------------------------------------------------------
struct Int2Args {
  PoolView pv;
  const float *qrot;
  float *part;
  int n_splits, pages_per_split;
};

__global__ void __launch_bounds__(256) int2_valu_kernel(Int2Args a) {
  const PoolView &pv = a.pv;
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int G = pv.hq / pv.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = pv.seq_lens[b];
  const int n_hist = max(0, L - pv.sink - pv.recent);
  const int n_pages = (n_hist + kPageTokens - 1) / kPageTokens;
  const int pg0 = split * a.pages_per_split;
  const int pg1 = min(n_pages, pg0 + a.pages_per_split);

  __shared__ float qsh[kMaxGroupHeads][kD];
  __shared__ float qsum[kMaxGroupHeads][2];
  __shared__ __attribute__((aligned(16))) uint8_t pg[kPageBytes];
  __shared__ float ps[4][64];

  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, c = e % kD;
    qsh[h][c] = a.qrot[((size_t)b * pv.hq + kv * G + h) * kD + c];
  }
  __syncthreads();
  for (int h = wave; h < G; h += 4) {
    float s0 = qsh[h][lane], s1 = qsh[h][64 + lane];
    for (int o = 32; o > 0; o >>= 1) {
      s0 += __shfl_xor(s0, o, 64);
      s1 += __shfl_xor(s1, o, 64);
    }
    if (lane == 0) {
      qsum[h][0] = s0;
      qsum[h][1] = s1;
    }
  }

  constexpr int kHPW = kMaxGroupHeads / 4;   // heads per wave, max
  float m[kHPW], l[kHPW], o0[kHPW], o1[kHPW];
#pragma unroll
  for (int i = 0; i < kHPW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    o0[i] = 0.f;
    o1[i] = 0.f;
  }
  const float sl2 = pv.sm_scale * kLog2e;
  bool bad = false;

  for (int pgi = pg0; pgi < pg1; ++pgi) {
    if (pgi >= pv.max_pages) {
      bad = true;
      break;
    }
    const int phys = pv.block_table[(size_t)b * pv.max_pages + pgi];
    if (phys < 0 || phys >= pv.n_pages) {
      bad = true;
      continue;
    }
    const int valid = min(kPageTokens, n_hist - pgi * kPageTokens);
    __syncthreads();
    const uint4 *src = (const uint4 *)(pv.pages + ((size_t)phys * pv.hkv + kv) * kPageBytes);
    for (int e = tid; e < kPageBytes / 16; e += 256) ((uint4 *)pg)[e] = src[e];
    __syncthreads();

    // token slot = lane
    const uint32_t *krow = (const uint32_t *)(pg + kKCodes + lane * 32);
    const uint16_t *km = (const uint16_t *)(pg + kKMeta + meta_entry(lane) * 8);
    const float ks0 = f16_to_f32(km[0]), kz0 = f16_to_f32(km[1]);
    const float ks1 = f16_to_f32(km[2]), kz1 = f16_to_f32(km[3]);
#pragma unroll
    for (int i = 0; i < kHPW; ++i) {
      const int h = wave + 4 * i;
      if (h >= G) break;
      float d0 = 0.f, d1 = 0.f;
      for (int w = 0; w < 8; ++w) {
        const uint32_t word = krow[w];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float code = (float)((word >> (2 * q)) & 3);
          const int c = 16 * w + q;
          if (w < 4) d0 = fmaf(qsh[h][c], code, d0);
          else d1 = fmaf(qsh[h][c], code, d1);
        }
      }
      float logit = (ks0 * d0 + kz0 * qsum[h][0] + ks1 * d1 + kz1 * qsum[h][1]) * sl2;
      if (lane >= valid) logit = -INFINITY;
      float pm = logit;
      for (int o = 32; o > 0; o >>= 1) pm = fmaxf(pm, __shfl_xor(pm, o, 64));
      const float mn = fmaxf(m[i], pm);
      const float alpha = exp2f(m[i] - mn);
      const float p = (lane < valid) ? exp2f(logit - mn) : 0.f;
      float ls = p;
      for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
      l[i] = l[i] * alpha + ls;
      m[i] = mn;
      ps[wave][lane] = p;
      wave_lds_sync();
      // PV: lane owns channels 2 lane, 2 lane + 1 (same group)
      const int c0 = 2 * lane;
      const int g = c0 >> 6;
      const uint32_t *vr0 = (const uint32_t *)(pg + kVCodes + c0 * 16);
      const uint32_t *vr1 = (const uint32_t *)(pg + kVCodes + (c0 + 1) * 16);
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0[q] = vr0[q];
        w1[q] = vr1[q];
      }
      float a0 = o0[i] * alpha, a1 = o1[i] * alpha;
      for (int t = 0; t < valid; ++t) {
        const float pt = ps[wave][t];
        const uint16_t *vm = (const uint16_t *)(pg + kVMeta + meta_entry(t) * 8);
        const float s = f16_to_f32(vm[2 * g]), z = f16_to_f32(vm[2 * g + 1]);
        const int byte = vcode_byte(t), sh = 2 * (t & 3);
        const float cd0 = (float)((w0[byte >> 2] >> (8 * (byte & 3) + sh)) & 3);
        const float cd1 = (float)((w1[byte >> 2] >> (8 * (byte & 3) + sh)) & 3);
        const float ps_ = pt * s, pz = pt * z;
        a0 = fmaf(ps_, cd0, a0 + pz);
        a1 = fmaf(ps_, cd1, a1 + pz);
      }
      o0[i] = a0;
      o1[i] = a1;
      wave_lds_sync();
    }
  }
  if (bad && tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);

#pragma unroll
  for (int i = 0; i < kHPW; ++i) {
    const int h = wave + 4 * i;
    if (h >= G) break;
    float *dst = part_ptr(a.part, b, kv, pv.hkv, a.n_splits, split, G, h);
    if (lane == 0) {
      // logits were kept in log2 units; store natural-log max for the merge
      dst[0] = (l[i] > 0.f) ? m[i] / kLog2e : -INFINITY;
      dst[1] = l[i];
    }
    dst[2 + 2 * lane] = o0[i];
    dst[3 + 2 * lane] = o1[i];
  }
}

// ---------------------------------------------------------------------------
// Merge: history partials (rotated basis) -> apply R_V^T -> merge with the
// BF16 partials -> normalise.  grid (Hkv, batch), block 128 (thread = channel).
// ---------------------------------------------------------------------------
struct MergeArgs {
  PoolView pv;
  RotView rv;
  const float *part, *bpart;
  float *out;
  int n_splits, n_chunks;
};

__global__ void __launch_bounds__(128) merge_kernel(MergeArgs a) {
  const PoolView &pv = a.pv;
  const int kv = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const int G = pv.hq / pv.hkv;
  __shared__ float zs[kD];
  const float *U = a.rv.U_V + (size_t)kv * kD * kD;
  for (int h = 0; h < G; ++h) {
    // history partials
    float M = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s)
      M = fmaxf(M, part_ptr((float *)a.part, b, kv, pv.hkv, a.n_splits, s, G, h)[0]);
    float l = 0.f, o = 0.f;
    if (M > -INFINITY) {
      for (int s = 0; s < a.n_splits; ++s) {
        const float *p = part_ptr((float *)a.part, b, kv, pv.hkv, a.n_splits, s, G, h);
        if (p[0] == -INFINITY) continue;
        const float w = __expf(p[0] - M);
        l = fmaf(w, p[1], l);
        o = fmaf(w, p[2 + j], o);
      }
    }
    // o (rotated basis, channel j) -> R_V^T: permute, butterfly, U^T
    __syncthreads();
    zs[j] = o;
    __syncthreads();
    float zv = zs[bitrev7(j)];
    __syncthreads();
    zs[j] = zv;
    __syncthreads();
    for (int hs = 1; hs < kD; hs <<= 1) {
      float v = 0.f, w = 0.f;
      int i0 = 0;
      if (j < 64) {
        i0 = (j / hs) * (2 * hs) + (j % hs);
        v = zs[i0];
        w = zs[i0 + hs];
      }
      __syncthreads();
      if (j < 64) {
        zs[i0] = v + w;
        zs[i0 + hs] = v - w;
      }
      __syncthreads();
    }
    float oh = 0.f;
    const float *Urow = U + (size_t)j * kD;   // o[j] = sum_i z_i U[j][i]
    for (int i = 0; i < kD; ++i) oh = fmaf(zs[i], Urow[i], oh);
    oh *= kInvSqrtDf;

    // BF16 partials (original basis)
    float Mb = -INFINITY;
    for (int c = 0; c < a.n_chunks; ++c)
      Mb = fmaxf(Mb, part_ptr((float *)a.bpart, b, kv, pv.hkv, a.n_chunks, c, G, h)[0]);
    float lb = 0.f, ob = 0.f;
    if (Mb > -INFINITY) {
      for (int c = 0; c < a.n_chunks; ++c) {
        const float *p = part_ptr((float *)a.bpart, b, kv, pv.hkv, a.n_chunks, c, G, h);
        if (p[0] == -INFINITY) continue;
        const float w = __expf(p[0] - Mb);
        lb = fmaf(w, p[1], lb);
        ob = fmaf(w, p[2 + j], ob);
      }
    }
    const float Mt = fmaxf(M, Mb);
    float res = 0.f;
    if (Mt > -INFINITY) {
      const float wh = (M > -INFINITY) ? __expf(M - Mt) : 0.f;
      const float wb = (Mb > -INFINITY) ? __expf(Mb - Mt) : 0.f;
      const float den = wh * l + wb * lb;
      res = (wh * oh + wb * ob) / den;
    }
    a.out[((size_t)b * pv.hq + kv * G + h) * kD + j] = res;
  }
}

}  // namespace

// MFMA kernel launcher lives in oscar_decode_mfma.hip.
hipError_t launch_int2_mfma(const PoolView &pv, const uint8_t *qint, const float *qconst,
                            float *part, int n_splits, int pages_per_split, int mtiles,
                            hipStream_t s);

DecodePlan make_decode_plan(int batch, int hkv, int hq, int max_pages, int sink, int recent,
                            int variant) {
  DecodePlan p{};
  const int G = hq / hkv;
  const int mtiles = (G + 3) / 4;
  const long work = (long)batch * hkv * (max_pages > 0 ? max_pages : 1);
  // aim for ~2048 workgroups over the whole history
  int pps = (int)((work + 2047) / 2048);
  if (variant == 0) pps = (pps < 4) ? 4 : pps;
  pps = pps < 1 ? 1 : pps;
  p.pages_per_split = pps;
  p.n_splits = max_pages > 0 ? (max_pages + pps - 1) / pps : 1;
  p.n_bf16_chunks = sink / 64 + recent / 64;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  p.off_qrot = off;
  off = al(off + (size_t)batch * hq * kD * sizeof(float));
  p.off_qint = off;
  off = al(off + (size_t)batch * hkv * mtiles * 2 * 64 * 16);
  p.off_qconst = off;
  off = al(off + (size_t)batch * hq * 4 * sizeof(float));
  p.off_part = off;
  off = al(off + (size_t)batch * hkv * p.n_splits * G * kPartStride * sizeof(float));
  p.off_bpart = off;
  off = al(off + (size_t)batch * hkv * p.n_bf16_chunks * G * kPartStride * sizeof(float));
  p.total = off;
  return p;
}

hipError_t launch_decode(const PoolView &pv, const RotView &rv, const uint16_t *q, float *out,
                         uint8_t *ws, const DecodePlan &plan, int variant, hipStream_t s) {
  const int G = pv.hq / pv.hkv;
  const int mtiles = (G + 3) / 4;
  float *qrot = (float *)(ws + plan.off_qrot);
  int8_t *qint = (int8_t *)(ws + plan.off_qint);
  float *qconst = (float *)(ws + plan.off_qconst);
  float *part = (float *)(ws + plan.off_part);
  float *bpart = (float *)(ws + plan.off_bpart);
  hipError_t e;
  if (variant == 0 && (G % 4) != 0) {
    const size_t n = (size_t)pv.batch * pv.hkv * mtiles * 2 * 64 * 16;
    hipLaunchKernelGGL(qint_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, qint, n);
  }
  QPrepArgs qa{pv, rv, q, qrot, variant == 0 ? qint : nullptr, qconst, mtiles};
  hipLaunchKernelGGL(qprep_kernel, dim3(pv.hq, pv.batch), dim3(128), 0, s, qa);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  Bf16SegArgs ba{pv, q, bpart, plan.n_bf16_chunks};
  hipLaunchKernelGGL(bf16_segment_kernel, dim3(plan.n_bf16_chunks, pv.hkv, pv.batch), dim3(256), 0, s, ba);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (variant == 1) {
    Int2Args ia{pv, qrot, part, plan.n_splits, plan.pages_per_split};
    hipLaunchKernelGGL(int2_valu_kernel, dim3(plan.n_splits, pv.hkv, pv.batch), dim3(256), 0, s, ia);
  } else {
    e = launch_int2_mfma(pv, (const uint8_t *)qint, qconst, part, plan.n_splits, plan.pages_per_split,
                         mtiles, s);
    if (e != hipSuccess) return e;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  MergeArgs ma{pv, rv, part, bpart, out, plan.n_splits, plan.n_bf16_chunks};
  hipLaunchKernelGGL(merge_kernel, dim3(pv.hkv, pv.batch), dim3(128), 0, s, ma);
  return hipGetLastError();
}

}  // namespace oscar
