// Split-K INT2 history decode on CDNA4 matrix cores (v_mfma_i32_16x16x64_i8).
//
// Sources: [A] youleyou.com article on OSCAR, token-pool paragraph under
// "OSCAR 的设计思路" (INT2 segment: unpack, scale/zero restore, float
// accumulation; online-softmax merge of segments); [B] MarkTechPost (zh)
// "Together AI 开源 OSCAR…", section "服务系统：混合精度缓存布局" (per-token
// asymmetric INT2, 64-channel groups, packed codes read inside the attention
// pass) and section "结果" (decode is KV-bandwidth bound at long context).
//
// Why integer MFMA.  A history page of one KV head is 5120 bytes and asks for
// 2 * G * 128 multiply-adds per token; at G = 4 that is ~26 MACs per HBM byte,
// more than the VALU can issue per byte at full HBM rate.  Codes are exact
// small integers, so both contractions run as exact int8 x int8 -> int32
// products on the matrix cores, with the float operand split into two int8
// halves of a 15-bit fixed-point value (hi * 256 + lo):
//   logits: rows (head, group, hi|lo) x tokens, K = 128 channels;
//           row masking by group keeps the two scale groups apart;
//   values: rows (head, group, hi|lo) x channels, K = 64 tokens of a page;
//           the weight p_t * scale_t is quantised per page relative to its
//           maximum (exact integer accumulation, one float rescale per page).
// The only approximations are the 15-bit fixed-point query (relative error
// <= 2^-16 of its largest entry) and the 15-bit per-page weights.
//
// Lane roles (wave64, lane = n + 16 q):
//   QK  B operand: token 16 tt + n, channels of kgroup q (8 code bytes);
//       C: rows 4 q .. 4 q + 3 = (head 4 mt + q, {g0 hi, g0 lo, g1 hi, g1 lo}).
//   PV  B operand: channel 16 nt + n, the 16 tokens {16 bb + 4 q + s} held in
//       dword q of that channel's 16-byte row; A operand = the weights staged
//       through LDS; C rows as above, columns = channels.
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWScale = 32639.0f;   // 15-bit fixed point, hi byte <= 127

struct MfmaArgs {
  PoolView pv;
  const uint8_t *qint;    // [B][Hkv][MT][2][64][16] int8
  const float *qconst;    // [B][Hq][4] {delta, Q0, Q1, -}
  float *part;            // [B][Hkv][n_splits][G][kPartStride]
  int n_splits, pages_per_split;
};

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16 two-bit codes of a dword -> 4 dwords of int8 codes: reg s holds, in byte
// bb, the code at bits [8 bb + 2 s, 8 bb + 2 s + 2).
__device__ __forceinline__ v4i unpack16(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)((w >> 2) & 0x03030303u);
  r[2] = (int)((w >> 4) & 0x03030303u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 4, 64));
  v = fmaxf(v, __shfl_xor(v, 8, 64));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return f16_to_f32((uint16_t)(w & 0xFFFF)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return f16_to_f32((uint16_t)(w >> 16)); }

template <int MT>
__global__ void __launch_bounds__(256) int2_mfma_kernel(MfmaArgs a) {
  const PoolView &pv = a.pv;
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int G = pv.hq / pv.hkv;
  const int L = pv.seq_lens[b];
  const int n_hist = max(0, L - pv.sink - pv.recent);
  const int n_pages = (n_hist + kPageTokens - 1) / kPageTokens;
  const int pg0 = split * a.pages_per_split;
  const int pg1 = min(n_pages, pg0 + a.pages_per_split);

  __shared__ v4i wlds[4][MT][64];                       // per-wave PV A operand
  __shared__ float sm_m[4][MT * 4], sm_l[4][MT * 4], sm_z[4][MT * 4][2];
  __shared__ float sm_o[4][MT * 4][kD];

  // Query operands and constants.
  v4i Aq[MT][2];
  float dl[MT], Q0[MT], Q1[MT];
  const v4i *qsrc = (const v4i *)(a.qint + ((size_t)b * pv.hkv + kv) * MT * 2 * 64 * 16);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    Aq[mt][0] = qsrc[(mt * 2 + 0) * 64 + lane];
    Aq[mt][1] = qsrc[(mt * 2 + 1) * 64 + lane];
    const int h = 4 * mt + q;
    if (h < G) {
      const float *qc = a.qconst + ((size_t)b * pv.hq + kv * G + h) * 4;
      dl[mt] = qc[0];
      Q0[mt] = qc[1];
      Q1[mt] = qc[2];
    } else {
      dl[mt] = Q0[mt] = Q1[mt] = 0.f;
    }
  }

  float m[MT], lp[MT], zp0[MT], zp1[MT], acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    m[mt] = -INFINITY;
    lp[mt] = zp0[mt] = zp1[mt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = 0.f;
  }
  const float sl2 = pv.sm_scale * kLog2e;
  bool bad = false;

  for (int pgi = pg0 + wave; pgi < pg1; pgi += 4) {
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
    const uint8_t *P = pv.pages + ((size_t)phys * pv.hkv + kv) * kPageBytes;

    uint2 kc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) kc[tt] = *(const uint2 *)(P + kKCodes + (16 * tt + n) * 32 + 8 * q);
    const uint4 km0 = *(const uint4 *)(P + kKMeta + 32 * n);
    const uint4 km1 = *(const uint4 *)(P + kKMeta + 32 * n + 16);
    uint32_t vc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) vc[nt] = *(const uint32_t *)(P + kVCodes + (16 * nt + n) * 16 + 4 * q);
    const uint4 vm0 = *(const uint4 *)(P + kVMeta + 32 * n);
    const uint4 vm1 = *(const uint4 *)(P + kVMeta + 32 * n + 16);

    // metadata of this lane's tokens 16 tt + n: {s0, z0, s1, z1}
    const uint32_t kmw[8] = {km0.x, km0.y, km0.z, km0.w, km1.x, km1.y, km1.z, km1.w};
    const uint32_t vmw[8] = {vm0.x, vm0.y, vm0.z, vm0.w, vm1.x, vm1.y, vm1.z, vm1.w};

    // ---- logits (log2 units) ----
    float lg[MT][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const v4i B0 = unpack16(kc[tt].x);
      const v4i B1 = unpack16(kc[tt].y);
      const float ks0 = h2f_lo(kmw[2 * tt]), kz0 = h2f_hi(kmw[2 * tt]);
      const float ks1 = h2f_lo(kmw[2 * tt + 1]), kz1 = h2f_hi(kmw[2 * tt + 1]);
      const bool ok = (16 * tt + n) < valid;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4i C = {0, 0, 0, 0};
        C = mfma_i8(Aq[mt][0], B0, C);
        C = mfma_i8(Aq[mt][1], B1, C);
        const int x0 = C[0] * 256 + C[1];
        const int x1 = C[2] * 256 + C[3];
        const float r = dl[mt] * (ks0 * (float)x0 + ks1 * (float)x1) + kz0 * Q0[mt] + kz1 * Q1[mt];
        lg[mt][tt] = ok ? r * sl2 : -INFINITY;
      }
    }

    // ---- online softmax and weights ----
    float alpha[MT], wsc0[MT], wsc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float pm = fmaxf(fmaxf(lg[mt][0], lg[mt][1]), fmaxf(lg[mt][2], lg[mt][3]));
      pm = max16(pm);
      const float mn = fmaxf(m[mt], pm);
      alpha[mt] = __builtin_amdgcn_exp2f(m[mt] - mn);
      const float beta = __builtin_amdgcn_exp2f(pm - mn);
      m[mt] = mn;
      float e[4], w0[4], w1[4];
      float es = 0.f, ez0 = 0.f, ez1 = 0.f, wm0 = 0.f, wm1 = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const bool ok = (16 * tt + n) < valid;
        e[tt] = ok ? __builtin_amdgcn_exp2f(lg[mt][tt] - pm) : 0.f;
        const float vs0 = h2f_lo(vmw[2 * tt]), vz0 = h2f_hi(vmw[2 * tt]);
        const float vs1 = h2f_lo(vmw[2 * tt + 1]), vz1 = h2f_hi(vmw[2 * tt + 1]);
        w0[tt] = ok ? e[tt] * vs0 : 0.f;
        w1[tt] = ok ? e[tt] * vs1 : 0.f;
        es += e[tt];
        ez0 += ok ? e[tt] * vz0 : 0.f;
        ez1 += ok ? e[tt] * vz1 : 0.f;
        wm0 = fmaxf(wm0, w0[tt]);
        wm1 = fmaxf(wm1, w1[tt]);
      }
      lp[mt] = lp[mt] * alpha[mt] + beta * es;
      zp0[mt] = zp0[mt] * alpha[mt] + beta * ez0;
      zp1[mt] = zp1[mt] * alpha[mt] + beta * ez1;
      wm0 = max16(wm0);
      wm1 = max16(wm1);
      const float inv0 = wm0 > 0.f ? kWScale / wm0 : 0.f;
      const float inv1 = wm1 > 0.f ? kWScale / wm1 : 0.f;
      wsc0[mt] = beta * wm0 * (1.0f / kWScale);
      wsc1[mt] = beta * wm1 * (1.0f / kWScale);
      // 15-bit weights -> (hi, lo) bytes -> A operand rows (4 q + 2 g + part),
      // lane 4 q + 2 g + part + 16 (n >> 2), bytes 4 (n & 3) + tt.
      uint32_t hib[2] = {0, 0}, lob[2] = {0, 0};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int i0 = min(32639, (int)rintf(w0[tt] * inv0));
        const int i1 = min(32639, (int)rintf(w1[tt] * inv1));
        const int l0 = (int)(int8_t)(i0 & 0xFF), l1 = (int)(int8_t)(i1 & 0xFF);
        const int h0 = (i0 - l0) >> 8, h1 = (i1 - l1) >> 8;
        hib[0] |= (uint32_t)(h0 & 0xFF) << (8 * tt);
        lob[0] |= (uint32_t)(l0 & 0xFF) << (8 * tt);
        hib[1] |= (uint32_t)(h1 & 0xFF) << (8 * tt);
        lob[1] |= (uint32_t)(l1 & 0xFF) << (8 * tt);
      }
      uint32_t *wd = (uint32_t *)&wlds[wave][mt][0];
      const int lb = 16 * (n >> 2);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        wd[(4 * q + 2 * g + 0 + lb) * 4 + (n & 3)] = hib[g];
        wd[(4 * q + 2 * g + 1 + lb) * 4 + (n & 3)] = lob[g];
      }
    }
    wave_lds_sync();
    v4i Aw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) Aw[mt] = wlds[wave][mt][lane];
    wave_lds_sync();

    // ---- values ----
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const v4i Bv = unpack16(vc[nt]);
      const int g = nt >> 2;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4i C = {0, 0, 0, 0};
        C = mfma_i8(Aw[mt], Bv, C);
        const int x = g ? (C[2] * 256 + C[3]) : (C[0] * 256 + C[1]);
        acc[mt][nt] = acc[mt][nt] * alpha[mt] + (float)x * (g ? wsc1[mt] : wsc0[mt]);
      }
    }
  }
  if (bad && lane == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);

  // ---- combine the four waves of the block into one partial ----
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float l16 = sum16(lp[mt]);
    const float z0 = sum16(zp0[mt]);
    const float z1 = sum16(zp1[mt]);
    const int hh = 4 * mt + q;
    if (n == 0) {
      sm_m[wave][hh] = m[mt];
      sm_l[wave][hh] = l16;
      sm_z[wave][hh][0] = z0;
      sm_z[wave][hh][1] = z1;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) sm_o[wave][hh][16 * nt + n] = acc[mt][nt];
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, c = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (sm_m[w][h] == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
        o += sc * (sm_o[w][h][c] + sm_z[w][h][c >> 6]);
        l += sc * sm_l[w][h];
      }
    }
    float *dst = a.part + ((((size_t)b * pv.hkv + kv) * a.n_splits + split) * G + h) * kPartStride;
    if (c == 0) {
      dst[0] = (M > -INFINITY) ? M * (1.0f / kLog2e) : -INFINITY;
      dst[1] = l;
    }
    dst[2 + c] = o;
  }
}

}  // namespace

hipError_t launch_int2_mfma(const PoolView &pv, const uint8_t *qint, const float *qconst,
                            float *part, int n_splits, int pages_per_split, int mtiles,
                            hipStream_t s) {
  MfmaArgs a{pv, qint, qconst, part, n_splits, pages_per_split};
  const dim3 grid(n_splits, pv.hkv, pv.batch), block(256);
  switch (mtiles) {
    case 1: hipLaunchKernelGGL(int2_mfma_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(int2_mfma_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(int2_mfma_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(int2_mfma_kernel<4>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oscar
