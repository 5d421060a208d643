// Decode attention over the mixed-precision pool on CDNA4: two launches.
//
// Sources: [A] youleyou.com article on OSCAR, token-pool paragraph under
// "OSCAR 的设计思路" (INT2 segment: unpack, restore scale/zero, accumulate in
// float; BF16 segment for sink/recent; online-softmax merge); [B]
// MarkTechPost (zh) "Together AI 开源 OSCAR…", section
// "服务系统：混合精度缓存布局" (rotated INT2 history with per-token asymmetric
// 64-channel groups; the read path inverse-rotates inside attention), section
// "OSCAR 有何不同做法" (R = U · H_Had · P_br) and section "结果" (decode is
// KV-bandwidth bound at long context).
//
// pre  (grid B * Hkv, 256 threads): q~ = bitrev(FWHT(q U_K) / sqrt(d)) for
//   the G query heads of a KV head, as a 15-bit fixed-point value split into
//   the int8 operands of the logit MFMA, plus float copies for the VALU
//   reference.
// scan (grid B * Hkv * n_splits, NW waves per workgroup, one workgroup per CU
//   at batch 1): the NW waves take interleaved history pages of one split;
//   the 64-token BF16 chunks of the sink and the recent window are spread one
//   per wave over the first workgroups, each writing its own partial; the
//   last workgroup of a (sequence, KV head) merges the partials, applies
//   R_V^T to the history part and writes the output.
//
// History page arithmetic (per wave, 64 tokens of one KV head):
//   logits  v_mfma_i32_16x16x64_i8: rows (head, group, hi|lo) of the rotated
//           query, columns 16 tokens, K = 128 channels; rows are masked to
//           their group so the two scales stay apart;
//   values  v_mfma_i32_16x16x64_i8: rows (head, group, hi|lo) of the weights
//           w_t = 2^(l_t - m_ref) * scale_t quantised to 15 bits with a fixed
//           per-head scale (scales are bounded by 2 tau_V / 3 after clipping),
//           columns 16 channels, K = the 64 tokens; each page's exact int32
//           result is added to float accumulators.  m_ref moves (and the
//           running sums are rescaled) only when a logit exceeds it by more
//           than a factor 2, so no per-page max or scale reduction is needed.
//   Codes enter unscaled: the zero point is added as z * sum(q) (logits) and
//   sum(p * z) (values).
#include <mutex>
#include <type_traits>

#include "oscar_wave.h"

namespace oscar {
namespace {

// Value weights are 23-bit fixed point per page: u = round(w * kWScale / wmax)
// and u + 0x8080 = 65536 hi + 256 (mid + 128) + (lo + 128) with hi <= 127,
// i.e. u + 0x8080 < 2^23.  kWScale keeps a margin below 2^23 - 0x8080 - 1 =
// 8355711 because w * (kWScale / wmax) may round a few units above kWScale.
constexpr float kWScale = 8355000.0f;
// fma(w, kq, kWMagic) lies in [2^23, 2^24), where float32 spacing is 1: its
// low 23 bits are u + 0x8080 rounded to nearest, with no conversion.
constexpr float kWMagic = 8388608.0f + 32896.0f;   // 2^23 + 0x8080
constexpr float kInvSqrtDf = 0.08838834764831845f;
constexpr int kMaxSplits = 256;
constexpr int kMaxParts = 512;                 // history splits + BF16 tiles per (sequence, KV head)
constexpr int kMergeSlices = 6;                // partial slices of the merge (slices x G <= 24)
constexpr float kHeadroom = 1.0f;              // log2 headroom above m_ref

struct DecArgs {
  PoolView pv;
  RotView rv;
  const uint16_t *q;   // bf16 [B][Hq][d]
  float *out;          // fp32 [B][Hq][d]
  int *counters;       // [BH]
  float *qconst;       // [BH][GH][4]: delta, Q0, Q1 (VALU variant)
  float *qrot;         // [BH][GH][kD] float q~ (VALU variant)
  float *part;         // [BH][n_parts][G][kPartStride]: history splits, shared-prefix chunks, then
                       // (several M-tiles, VALU) BF16 tiles; one M-tile on MFMA folds its tiles
                       // into its split's partial
  int n_splits, n_chunks, pages_per_split, n_parts;
  int prefix_pages, n_prefix, prefix_per_chunk;   // shared prefix (0 pages: none)
  float *pq;           // shared prefix: query operands per (sequence, KV head)
};

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16 two-bit codes -> int8 operand: register s, byte bb = bits [8 bb + 2 s, +2).
__device__ __forceinline__ v4i unpack16(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)((w >> 2) & 0x03030303u);
  r[2] = (int)((w >> 4) & 0x03030303u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

// The same for value codes, with a mask and no shift where the field fits
// in a signed byte: register s holds code * 4^s for s = 0, 1, 2 (at most 48)
// and the plain code for s = 3.  The weights multiplied with register s are
// divided by 4^s beforehand (see int2_page).
__device__ __forceinline__ v4i unpack16_v(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)(w & 0x0C0C0C0Cu);
  r[2] = (int)(w & 0x30303030u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

// Every byte of w (a 2-bit code 0..3) replaced by byte `code` of the codebook
// word lut (its level n_code, <= 96): one v_perm_b32.
__device__ __forceinline__ int lut_bytes(int w, uint32_t lut) { return (int)__builtin_amdgcn_perm(0u, lut, (uint32_t)w); }
__device__ __forceinline__ v4i lut4(v4i r, uint32_t lut) {
  return v4i{lut_bytes(r[0], lut), lut_bytes(r[1], lut), lut_bytes(r[2], lut), lut_bytes(r[3], lut)};
}

// Byte i of a word as a float (one v_cvt_f32_ubyte<i>).
__device__ __forceinline__ float ubyte_f(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }

// Metadata grid steps of one KV head (zero z8 * a - tau, scale s8 * b).
struct MetaSteps {
  float ka, kb, ktau, va, vb, vtau;
};
__device__ __forceinline__ MetaSteps meta_steps(float tk, float tv) {
  return MetaSteps{meta_zero_step(tk), meta_scale_step(tk), tk, meta_zero_step(tv), meta_scale_step(tv), tv};
}
__device__ __forceinline__ MetaSteps meta_steps(const RotView &rv, int kv) {
  return meta_steps(rv.tau_K[kv], rv.tau_V[kv]);
}

// Byte 2 / byte 1 / byte 0 of four words gathered into one word (word i -> byte i).
__device__ __forceinline__ uint32_t gather_b2(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_amdgcn_perm(w1, w0, 0x0C0C0602u) | __builtin_amdgcn_perm(w3, w2, 0x06020C0Cu);
}
__device__ __forceinline__ uint32_t gather_b1(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_amdgcn_perm(w1, w0, 0x0C0C0501u) | __builtin_amdgcn_perm(w3, w2, 0x05010C0Cu);
}
__device__ __forceinline__ uint32_t gather_b0(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return __builtin_amdgcn_perm(w1, w0, 0x0C0C0400u) | __builtin_amdgcn_perm(w3, w2, 0x04000C0Cu);
}

// ===========================================================================
// pre kernel
// ===========================================================================
template <int MT, int GH>
struct QSmem {
  float ys[MT * 4][kD];
  v4i aq[MT * 2 * 64];     // int8 logit operands (hi/lo rows per head and group)
  float qc[GH][4];         // delta, Q0, Q1 (per-group sums of the fixed-point q~)
};

// Barrier among waves 0..3 of a workgroup (the other waves take no part): a
// shared counter, zero at the workgroup's first s_barrier, that each of the
// four waves raises by one and then polls until it reaches `target` (4 for
// the first such barrier, 8 for a second one, ...).
__device__ __forceinline__ void four_wave_sync(int *ctr, int target) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Query preparation for one (sequence, KV head): q~ = bitrev(FWHT(q U_K) /
// sqrt(d)) for its G query heads, then per head a 15-bit fixed-point copy
// split into hi/lo int8 bytes laid out as the A operand of the logit MFMA
// (rows: head h -> 4h + {group 0 hi, group 0 lo, group 1 hi, group 1 lo}).
// Results stay in `sm`; with `qrot` non-null the float q~ is also written
// there.  after_loads() runs on every thread once the global loads of the
// preparation (threads 0..255) have been consumed.
// With four_ctr null the whole workgroup (any multiple of 64 threads >= 256)
// takes part and synchronises with s_barrier.  Otherwise (G <= 4) waves 0..3
// alone finish the preparation, synchronising through four_wave_sync on
// *four_ctr, while every other wave returns right after after_loads(): a wave
// held up issuing page copies then delays no one.  The caller publishes the
// results with a barrier of its own (none is taken at the end here).
template <int MT, int GH, typename AfterLoads>
__device__ void query_prep(const DecArgs &a, int b, int kv, QSmem<MT, GH> &sm, float *qrot, AfterLoads after_loads,
                           int *four_ctr = nullptr) {
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = four_ctr ? 4 : blockDim.x >> 6;   // waves taking part
  const int G = pv.hq / pv.hkv;
  const float *U = a.rv.U_K + (size_t)kv * kD * kD;
  const uint16_t *qb = a.q + ((size_t)b * pv.hq + (size_t)kv * G) * kD;
  // y[h][j] = sum_k q[h][k] U[k][j]: threads 0..255 -> columns 4c..4c+3 and
  // rows k = 16 (t % 8) + i, i < 16; 8-lane reduction.  The 16 row loads of
  // U and the query rows of four heads (two 16-byte loads per head) are all
  // in flight at once: one memory round trip per four heads.
  if (tid < 256) {
    const int c = tid >> 3, kk = tid & 7;
    float4 u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = *(const float4 *)(U + (size_t)(16 * kk + i) * kD + 4 * c);
#pragma unroll
    for (int h0 = 0; h0 < GH; h0 += 4) {
      uint4 qv[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // heads past G load head G - 1 (in bounds) and are not stored
        const uint4 *qr = (const uint4 *)(qb + (size_t)min(h0 + j, G - 1) * kD + 16 * kk);
        qv[j][0] = qr[0];
        qv[j][1] = qr[1];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint4 &w4 = qv[j][i >> 3];
          const uint32_t w = (i & 6) == 0 ? w4.x : (i & 6) == 2 ? w4.y : (i & 6) == 4 ? w4.z : w4.w;
          const float qk = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
          y0 = fmaf(qk, u[i].x, y0);
          y1 = fmaf(qk, u[i].y, y1);
          y2 = fmaf(qk, u[i].z, y2);
          y3 = fmaf(qk, u[i].w, y3);
        }
        y0 += lane_xor<1>(y0);
        y1 += lane_xor<1>(y1);
        y2 += lane_xor<1>(y2);
        y3 += lane_xor<1>(y3);
        y0 += lane_xor<2>(y0);
        y1 += lane_xor<2>(y1);
        y2 += lane_xor<2>(y2);
        y3 += lane_xor<2>(y3);
        y0 += lane_xor<4>(y0);
        y1 += lane_xor<4>(y1);
        y2 += lane_xor<4>(y2);
        y3 += lane_xor<4>(y3);
        if (kk == 0 && h0 + j < G) {
          sm.ys[h0 + j][4 * c] = y0;
          sm.ys[h0 + j][4 * c + 1] = y1;
          sm.ys[h0 + j][4 * c + 2] = y2;
          sm.ys[h0 + j][4 * c + 3] = y3;
        }
      }
    }
  }
  after_loads();
  if (four_ctr && w >= 4) return;
  for (int e = tid; e < MT * 2 * 64 * 4; e += 64 * nw) ((uint32_t *)sm.aq)[e] = 0;
  if (four_ctr) four_wave_sync(four_ctr, 4);
  else __syncthreads();
  // one wave per head: Walsh-Hadamard butterfly (lane l holds elements l and
  // l + 64; stages 1..32 by lane exchange, stage 64 in registers), then the
  // rotated, permuted q~ -> fixed point -> operands
  for (int h = w; h < G; h += nw) {
    float x0 = sm.ys[h][lane], x1 = sm.ys[h][lane + 64];
    fwht_lane_stages(x0, x1, lane);
    sm.ys[h][lane] = x0 + x1;
    sm.ys[h][lane + 64] = x0 - x1;
    wave_lds_sync();
    const float v0 = sm.ys[h][bitrev7(lane)] * kInvSqrtDf;
    const float v1 = sm.ys[h][bitrev7(lane + 64)] * kInvSqrtDf;
    if (qrot) {
      qrot[(size_t)h * kD + lane] = v0;
      qrot[(size_t)h * kD + 64 + lane] = v1;
    }
    const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float delta = mx > 0.f ? mx / 32639.0f : 1.0f;
    const int q0 = max(-32639, min(32639, (int)rintf(v0 / delta)));
    const int q1 = max(-32639, min(32639, (int)rintf(v1 / delta)));
    const int s0 = wave_sum_i(q0), s1 = wave_sum_i(q1);
    if (lane == 0) {
      sm.qc[h][0] = delta;
      sm.qc[h][1] = delta * (float)s0;   // |sum| < 2^24: exact
      sm.qc[h][2] = delta * (float)s1;
      sm.qc[h][3] = 0.f;
    }
    const int mt = h >> 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = lane + 64 * half;
      const int qi = half ? q1 : q0;
      const int lo = (int)(int8_t)(qi & 0xFF);
      const int hi = (qi - lo) >> 8;
      // channel c -> kgroup c/32, kstep (c/16)%2, byte (c/4)%4 of register c%4
      const int kg = c >> 5, ks = (c >> 4) & 1, bb = (c >> 2) & 3, s = c & 3;
      const int g = c >> 6;
      int8_t *base = (int8_t *)(sm.aq + (mt * 2 + ks) * 64);
      const int r = 4 * (h & 3) + 2 * g;
      base[(r + 16 * kg) * 16 + 4 * s + bb] = (int8_t)hi;
      base[(r + 1 + 16 * kg) * 16 + 4 * s + bb] = (int8_t)lo;
    }
  }
  if (!four_ctr) __syncthreads();
}

// Query preparation for the VALU scan variant, which reads the float q~ and
// the per-head constants from the workspace.
template <int MT, int GH>
__global__ void __launch_bounds__(256) decode_pre_kernel(DecArgs a) {
  __shared__ QSmem<MT, GH> sm;
  const int bh = blockIdx.x;
  query_prep<MT, GH>(a, bh / a.pv.hkv, bh % a.pv.hkv, sm, a.qrot + (size_t)bh * GH * kD, [] {});
  const int G = a.pv.hq / a.pv.hkv;
  for (int e = threadIdx.x; e < G * 4; e += blockDim.x) a.qconst[(size_t)bh * GH * 4 + e] = (&sm.qc[0][0])[e];
}

// ===========================================================================
// scan kernel
// ===========================================================================
struct PageRegs {
  uint2 kc[4];
  uint4 km;          // metadata of tokens 16 tt + n, tt = 0..3: {s8_0, z8_0, s8_1, z8_1}
  uint32_t vc[8];
  uint4 vm;
};

__device__ __forceinline__ void load_page(PageRegs &r, const uint8_t *P, int n, int q) {
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) r.kc[tt] = *(const uint2 *)(P + kKCodes + (16 * tt + n) * 32 + 8 * q);
  r.km = *(const uint4 *)(P + kKMeta + 16 * n);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) r.vc[nt] = *(const uint32_t *)(P + kVCodes + (16 * nt + n) * 16 + 4 * q);
  r.vm = *(const uint4 *)(P + kVMeta + 16 * n);
}

template <int MT>
struct HistState {
  float mref[MT];          // log2-domain reference max (row-uniform)
  float lsum[MT], z0[MT], z1[MT];
  float facc[MT][8];       // value sums (rotated basis, relative to 2^mref)
};

template <int MT>
__device__ __forceinline__ void rescale(HistState<MT> &st, int mt, float alpha) {
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) st.facc[mt][nt] *= alpha;
  st.lsum[mt] *= alpha;
  st.z0[mt] *= alpha;
  st.z1[mt] *= alpha;
}

// Logit operands of one wave: the int8 query (A operand, hi/lo rows per
// group) and per-lane-row constants.  With metadata codes (s8, z8) of a
// token, its logit (log2 units) is
//   fma(fma(s8_0, x0, s8_1 x1), qa, fma(z8_0, qb0, fma(z8_1, qb1, qc)))
// where x_g is the integer dot product of group g, qa = delta b sl2,
// qb_g = Q_g a sl2 and qc = -tau (Q_0 + Q_1) sl2 (a, b: the head's zero and
// scale steps; delta: the query's fixed-point step; Q_g: its group sums).
template <int MT>
struct QueryOps {
  v4i A[MT][2];
  float qa[MT], qb0[MT], qb1[MT], qc[MT];
  uint32_t lutk, lutv;   // codebook words (LUT scans)
};

// One 64-token history page for MT M-tiles of 4 query heads.
//
// Logits: int8 MFMA of the 15-bit query (hi/lo rows, one per 64-channel
// group) against the unpacked K codes; scale and zero per token and group.
// Values: the weights w = 2^(l - m_ref) * scale_V of a head are quantised to
// 23 bits against the page's largest weight of that head, split into
// hi/mid/lo bytes (rows 4h, 4h+1, 4h+2 of the A operand of the token's
// 64-channel group; row 4h+3 stays zero) and multiplied with the unpacked V
// codes on the int8 MFMA.  Small weights must survive: at long context most
// of the softmax mass can sit in weights far below the page maximum.  The
// zero-point part sum(w * zero) stays in float.
// With LUT the codes stand for codebook levels: every unpacked code byte is
// replaced by its level n (<= 96) before the products, the 1/32 of the
// level grid is in qa and the page's weight step, and the value results are
// combined in float (an int32 of three byte planes could overflow).
template <int MT, bool FULL, bool LUT>
__device__ __forceinline__ void int2_page(const PageRegs &r, int valid, const QueryOps<MT> &qo, HistState<MT> &st,
                                          v4i *wl) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  // this lane's weights meet value-code register n % 4 (see unpack16_v)
  // (kWScale / 4^s for s = n % 4 < 3, else kWScale: exponent steps 0, 2, 4, 0)
  const float wsc = LUT ? kWScale : __int_as_float(__float_as_int(kWScale) - (int)(((0x00040200u >> (8 * (n & 3))) & 0xFFu) << 23));
  const uint32_t kmw[4] = {r.km.x, r.km.y, r.km.z, r.km.w};
  const uint32_t vmw[4] = {r.vm.x, r.vm.y, r.vm.z, r.vm.w};
  float lg[MT][4];
  // all products first, so that no logit waits on the product just issued
  v4i CK[4][MT];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    v4i B0 = unpack16(r.kc[tt].x);
    v4i B1 = unpack16(r.kc[tt].y);
    if constexpr (LUT) {
      B0 = lut4(B0, qo.lutk);
      B1 = lut4(B1, qo.lutk);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      CK[tt][mt] = mfma_i8(qo.A[mt][1], B1, mfma_i8(qo.A[mt][0], B0, v4i{0, 0, 0, 0}));
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const float s0 = ubyte_f(kmw[tt], 0), z0 = ubyte_f(kmw[tt], 1);
    const float s1 = ubyte_f(kmw[tt], 2), z1 = ubyte_f(kmw[tt], 3);
    const bool ok = FULL || (16 * tt + n) < valid;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i C = CK[tt][mt];
      const float x0 = (float)(C[0] * 256 + C[1]);
      const float x1 = (float)(C[2] * 256 + C[3]);
      const float v = fmaf(fmaf(s0, x0, s1 * x1), qo.qa[mt], fmaf(z0, qo.qb0[mt], fmaf(z1, qo.qb1[mt], qo.qc[mt])));
      lg[mt][tt] = ok ? v : -INFINITY;
    }
  }
  float pscale[MT];   // per-head dequantisation step of this page's weights
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // move the reference only when some logit exceeds it by the headroom
    float pm = fmaxf(fmaxf(lg[mt][0], lg[mt][1]), fmaxf(lg[mt][2], lg[mt][3]));
    if (__builtin_amdgcn_ballot_w64(pm > st.mref[mt] + kHeadroom)) {
      pm = row16_max(pm);
      const float mnew = fmaxf(st.mref[mt], pm);
      rescale<MT>(st, mt, exp2_fast(st.mref[mt] - mnew));
      st.mref[mt] = mnew;
    }
    float w0[4], w1[4];
    float es = 0.f, ez0 = 0.f, ez1 = 0.f, wmax = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      // masked tokens: e = 0, and their (unwritten) metadata is not used
      const bool ok = FULL || (16 * tt + n) < valid;
      const float e = exp2_fast(lg[mt][tt] - st.mref[mt]);
      const float vs0 = ubyte_f(vmw[tt], 0), vz0 = ubyte_f(vmw[tt], 1);
      const float vs1 = ubyte_f(vmw[tt], 2), vz1 = ubyte_f(vmw[tt], 3);
      es += e;
      ez0 = ok ? fmaf(e, vz0, ez0) : ez0;
      ez1 = ok ? fmaf(e, vz1, ez1) : ez1;
      w0[tt] = ok ? e * vs0 : 0.f;
      w1[tt] = ok ? e * vs1 : 0.f;
      wmax = fmaxf(wmax, fmaxf(w0[tt], w1[tt]));
    }
    st.lsum[mt] += es;
    st.z0[mt] += ez0;
    st.z1[mt] += ez1;
    wmax = row16_max(wmax);
    // approximate reciprocal: kq may exceed kWScale / wmax by an ulp, which
    // the margin in kWScale absorbs; pscale is exact in the same sense
    const float kq = wmax > 0.f ? wsc * __builtin_amdgcn_rcpf(wmax) : 0.f;
    pscale[mt] = wmax * (LUT ? 1.0f / (32.0f * kWScale) : 1.0f / kWScale);
    uint32_t u0[4], u1[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      u0[tt] = __float_as_uint(fmaf(w0[tt], kq, kWMagic));   // bytes 0..2 = u + 0x8080
      u1[tt] = __float_as_uint(fmaf(w1[tt], kq, kWMagic));
    }
    // lane (n, q): head q, tokens 16 tt + n -> A rows 4q + {hi, mid, lo},
    // lane group n / 4, bytes 4 (n % 4) + tt
    uint32_t *wd0 = (uint32_t *)(wl + (mt * 2 + 0) * 64);
    uint32_t *wd1 = (uint32_t *)(wl + (mt * 2 + 1) * 64);
    const int lb = 16 * (n >> 2), sub = n & 3;
    wd0[(4 * q + 0 + lb) * 4 + sub] = gather_b2(u0[0], u0[1], u0[2], u0[3]);
    wd0[(4 * q + 1 + lb) * 4 + sub] = gather_b1(u0[0], u0[1], u0[2], u0[3]) ^ 0x80808080u;
    wd0[(4 * q + 2 + lb) * 4 + sub] = gather_b0(u0[0], u0[1], u0[2], u0[3]) ^ 0x80808080u;
    wd1[(4 * q + 0 + lb) * 4 + sub] = gather_b2(u1[0], u1[1], u1[2], u1[3]);
    wd1[(4 * q + 1 + lb) * 4 + sub] = gather_b1(u1[0], u1[1], u1[2], u1[3]) ^ 0x80808080u;
    wd1[(4 * q + 2 + lb) * 4 + sub] = gather_b0(u1[0], u1[1], u1[2], u1[3]) ^ 0x80808080u;
  }
  wave_lds_sync();
  v4i Aw[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    Aw[mt][0] = wl[(mt * 2 + 0) * 64 + lane];
    Aw[mt][1] = wl[(mt * 2 + 1) * 64 + lane];
  }
  wave_lds_sync();
  // all products first, so that no value combine waits on the product just issued
  v4i C[8][MT];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const v4i Bv = LUT ? lut4(unpack16(r.vc[nt]), qo.lutv) : unpack16_v(r.vc[nt]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) C[nt][mt] = mfma_i8(Aw[mt][nt >> 2], Bv, v4i{0, 0, 0, 0});
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (LUT) {
        // each byte plane's sum (at most 128 * 96 * 64 in magnitude) is exact
        // in int32; the planes are weighted in float
        const float val = fmaf((float)C[nt][mt][0], 65536.0f, fmaf((float)C[nt][mt][1], 256.0f, (float)C[nt][mt][2]));
        st.facc[mt][nt] = fmaf(val, pscale[mt], st.facc[mt][nt]);
      } else {
        // sum over 64 tokens of u * code <= 8355000 * 3 * 64 < 2^31: exact in int32
        // two shift-adds; the empty asm (on a VALU result) keeps the compiler
        // from re-associating them into two shifts and a three-way add
        int t = (int)(((unsigned)C[nt][mt][0] << 8) + (unsigned)C[nt][mt][1]);
        asm("" : "+v"(t));
        const int val = (int)(((unsigned)t << 8) + (unsigned)C[nt][mt][2]);
        st.facc[mt][nt] = fmaf((float)val, pscale[mt], st.facc[mt][nt]);
      }
    }
  }
}

// VALU reference of the history scan: float32 FMAs on unpacked codes.
struct ValuWave {
  float *m, *l;          // [GH], wave-uniform values
  float (*acc)[64][2];   // [GH][lane][2]
};

// The reconstruction level of a code (byte `code` of the codebook word / 32;
// the code itself on the uniform grid).
__device__ __forceinline__ float level_f(uint32_t lut, uint32_t code) {
  return (float)((lut >> (8 * code)) & 0xFFu) * (1.0f / 32.0f);
}

template <bool FULL>
__device__ __forceinline__ void int2_page_valu(const uint8_t *P, int valid, int G, const float *qrot,
                                               const float (*qsum)[2], float sl2, const MetaSteps &ms,
                                               ValuWave st, float (*pw)[4], uint32_t lutk, uint32_t lutv) {
  const int lane = threadIdx.x & 63;
  const int t = lane;
  const uint4 k0 = *(const uint4 *)(P + kKCodes + t * 32);
  const uint4 k1 = *(const uint4 *)(P + kKCodes + t * 32 + 16);
  const uint32_t km = *(const uint32_t *)(P + kKMeta + meta_entry(t) * 4);
  const uint32_t vm = *(const uint32_t *)(P + kVMeta + meta_entry(t) * 4);
  const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
  const bool ok = FULL || t < valid;
  const float ks0 = ubyte_f(km, 0) * ms.kb, kz0 = ubyte_f(km, 1) * ms.ka - ms.ktau;
  const float ks1 = ubyte_f(km, 2) * ms.kb, kz1 = ubyte_f(km, 3) * ms.ka - ms.ktau;
  const float vs0 = ubyte_f(vm, 0) * ms.vb, vz0 = ubyte_f(vm, 1) * ms.va - ms.vtau;
  const float vs1 = ubyte_f(vm, 2) * ms.vb, vz1 = ubyte_f(vm, 3) * ms.va - ms.vtau;
  const int c0 = 2 * lane, g = lane >> 5;
  const uint4 r0 = *(const uint4 *)(P + kVCodes + c0 * 16);
  const uint4 r1 = *(const uint4 *)(P + kVCodes + (c0 + 1) * 16);
  const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    const float *qr = qrot + (size_t)h * kD;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float code = level_f(lutk, (kw[w] >> (2 * j)) & 3u);
        if (w < 4) d0 = fmaf(qr[16 * w + j], code, d0);
        else d1 = fmaf(qr[16 * w + j], code, d1);
      }
    }
    float lg = (ks0 * d0 + kz0 * qsum[h][0] + ks1 * d1 + kz1 * qsum[h][1]) * sl2;
    lg = ok ? lg : -INFINITY;
    float pm = lg;
    for (int o = 32; o > 0; o >>= 1) pm = fmaxf(pm, __shfl_xor(pm, o, 64));
    const float mh = st.m[h];
    const float mn = fmaxf(mh, pm);
    const float alpha = exp2_fast(mh - mn);
    const float p = ok ? exp2_fast(lg - mn) : 0.f;
    float ls = p;
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
    wave_lds_sync();
    if (lane == 0) {
      st.l[h] = st.l[h] * alpha + ls;
      st.m[h] = mn;
    }
    pw[t][0] = ok ? p * vs0 : 0.f;
    pw[t][1] = ok ? p * vz0 : 0.f;
    pw[t][2] = ok ? p * vs1 : 0.f;
    pw[t][3] = ok ? p * vz1 : 0.f;
    wave_lds_sync();
    float a0 = st.acc[h][lane][0] * alpha, a1 = st.acc[h][lane][1] * alpha;
    // token t = 16 bb + 4 j + s sits in word j, byte bb, bits 2 s of a V row
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int tt = 16 * bb + 4 * j + s4, sh = 8 * bb + 2 * s4;
          const float cd0 = level_f(lutv, (w0[j] >> sh) & 3u);
          const float cd1 = level_f(lutv, (w1[j] >> sh) & 3u);
          const float ps = pw[tt][2 * g], pz = pw[tt][2 * g + 1];
          a0 = fmaf(ps, cd0, a0 + pz);
          a1 = fmaf(ps, cd1, a1 + pz);
        }
      }
    }
    st.acc[h][lane][0] = a0;
    st.acc[h][lane][1] = a1;
    wave_lds_sync();
  }
}

// Waves per scan workgroup: 12 (three per SIMD) for one M-tile of heads, 8
// (two per SIMD) otherwise, so that one workgroup fills a CU; the VALU
// reference keeps per-wave value sums in LDS and uses 4.
template <int MT, bool MFMA>
constexpr int scan_waves() { return MFMA ? (MT == 1 ? 12 : 8) : 4; }

// History pages each MFMA wave keeps in flight as LDS DMA copies.
template <int MT>
constexpr int scan_prefetch() { return 2; }

// A running BF16 state (LDS, one M-tile of heads) is o[128 h + c] and 16
// floats st: m[h] (log2 units) at st[h], l[h] at st[4 + h], and a tile's m
// and l staged at st[8 + h], st[12 + h].  A wave's page buffers hold, once
// its pages are done, its history state (o, 128 floats per head) at kAccHist.
constexpr int kAccHist = 0, kAccFloats = 512;
constexpr int kStM = 0, kStL = 4, kStTm = 8, kStTl = 12;
// Waves that run the BF16 tiles (one M-tile of heads) before their pages,
// each into a BF16 state of its own outside the page buffers.
constexpr int kTileWaves = 4;

template <int MT, int GH, int NW, bool MFMA>
struct ScanSmem {
  static constexpr int PF = MFMA ? scan_prefetch<MT>() : 1;
  union WaveScratch {
    v4i wl[MT * 2 * 64];                   // PV A operands, one per channel group (MFMA)
    float pw[kPageTokens][4];              // p * scale, p * zero (VALU)
    float tile[GH][kD];                    // BF16 tile probabilities, then its o
  };
  struct EpiSmem {                         // split epilogue (one M-tile, after every wave's pages)
    float zs[GH][kD];                      // history sum, bit-reversal permuted, then butterflied
    float ot[GH][kD];                      // history sum in the original basis
    float ob[GH][kD];                      // BF16 tile sum
    float hm[GH], hl[GH], bm[GH], bl[GH];
  };
  union {
    WaveScratch wave[NW];
    QSmem<MT, GH> q;                       // query preparation, several M-tiles (before the scan)
    EpiSmem e;
  };
  // query preparation, one M-tile of heads: its own space (the tile waves
  // read it only after their tiles, while the other waves are scanning)
  struct NoQ {};
  std::conditional_t<MFMA && MT == 1, QSmem<MT, GH>, NoQ> q1;
  __device__ QSmem<MT, GH> &qprep() {
    if constexpr (MFMA && MT == 1) return q1;
    else return q;
  }
  float qsum[GH][2];                       // VALU: per-group sums of q~
  int prep_ctr, ready;                     // one M-tile: four_wave_sync counter; parts ready before the scan
  float m[NW][MT * 4], l[NW][MT * 4], z[NW][MT * 4][2];
  union {
    uint4 pbuf[MFMA ? NW : 1][PF][kPageBytes / 16];   // page copies (during the scan)
    float o[NW][MT * 4][kD];                          // per-wave value sums (after it)
  };
  float vacc[MFMA ? 1 : NW][GH][64][2];    // VALU: per-wave running sums
  float tacc[MFMA && MT == 1 ? kTileWaves : 1][kD * 4 + 16];   // BF16 states of the tile waves
};

// Page copies into LDS are issued as inline assembly so that the compiler
// does not treat every later LDS access as dependent on them (it would wait
// for all vector memory first); their completion is awaited explicitly with
// wait_pages().  Vector-memory loads complete in issue order, so waits the
// compiler places for its own loads stay correct (at worst longer).

// s_waitcnt immediate that waits for vector-memory count <= n only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most n pages' copies (5 loads each) are outstanding.
__device__ __forceinline__ void wait_pages(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait for this wave's LDS reads (a page buffer may then be refilled).
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One 1 KB LDS-DMA copy: lane i moves bytes [16 i, 16 i + 16).  src and lds
// are wave-uniform.  M0 (the LDS destination) is saved and restored inside
// the asm, so the compiler's own use of M0 is unaffected.  The readfirstlane
// builtin returns int: both halves of src go back through uint32_t so that
// the low half is zero-extended (a sign-extended low half would set every
// bit of the high half when its bit 31 is set).  The copy carries the
// non-temporal hint (nt): pages are read once per scan, and streaming reads
// with it measured 7.0 TB/s against 6.2 TB/s without on MI355X.
__device__ __forceinline__ void dma_1k(uint64_t src, uint32_t lds, uint32_t lane_off) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(src >> 32));
  src = ((uint64_t)hi << 32) | (uint64_t)lo;
  lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(lane_off), "s"(src)
      : "memory");
}

// Copy one 4608-byte page to LDS: four 1 KB DMA copies (kilobyte j of the
// page from base + 1024 j to lds + 1024 j; lane_off = 16 lane) and one
// 512-byte copy of the metadata tail.
__device__ __forceinline__ void dma_page(uint64_t base, uint32_t lds, uint32_t lane_off) {
  static_assert(kPageBytes == 4 * 1024 + 512, "a page is four 1 KB copies and a 512-byte tail");
#pragma unroll
  for (int j = 0; j < 4; ++j) dma_1k(base + 1024u * j, lds + 1024u * j, lane_off);
  // tail: lanes 0..31 move 16 bytes each (the instruction still counts once
  // in vmcnt, so a page is five copies either way)
  if (lane_off < 512u) dma_1k(base + 4096u, lds + 4096u, lane_off);
}

template <int GH>
struct MergeSmem {
  float ml[kMaxParts * GH][2];  // (m, l) of partial p, head h at p * G + h: history splits, then BF16 tiles
  float wgt[kMaxParts][GH];     // merge weight of every partial
  float hs[GH][4];              // per head: history scale, tile scale, 1 / denominator
  float zs[GH][kD];             // weighted history sum, bit-reversal permuted
  float ot[GH][kD];             // history output in the original basis
  float ob[GH][kD];             // weighted BF16 tile sum
  alignas(16) float red[2][kMergeSlices * 4 * kD];   // per-slice sums (history, tiles)
};

// Plain merge of partials already in the original basis (see merge_plain).
template <int GH>
struct PlainMergeSmem {
  float wgt[kMaxSplits][GH];
  float inv[GH];
  alignas(16) float red[kMergeSlices][GH * kD];
};

template <int MT, int GH, int NW, bool MFMA>
union ScanUnion {
  ScanSmem<MT, GH, NW, MFMA> s;
  MergeSmem<GH> g;
  PlainMergeSmem<GH> pm;
};

// BF16 window tiles: 16 tokens each, sink tiles first (kSinkTiles = sink / 16),
// then the recent ring.  tile_source gives tile u's K and V rows and its
// number of valid tokens (0: nothing to do).
struct TileSrc {
  const uint16_t *K, *V;
  int valid;
};
// A sequence's length and sink slot, loaded once for all its tiles (each
// tile's row loads then cost one memory round trip, not two).
struct TileCtx {
  int L, slot;
};
__device__ __forceinline__ TileCtx tile_ctx(const PoolView &pv, int b) {
  return TileCtx{max(0, pv.seq_lens[b]), pv.sink_slot[b]};
}
__device__ __forceinline__ void tile_source(const PoolView &pv, const TileCtx &tc, int b, int kv, int u, TileSrc &t) {
  const int lane = threadIdx.x & 63;
  const int L = tc.L;
  const int n_sink_tiles = pv.sink / kTileTokens;
  const bool sink_tile = u < n_sink_tiles;
  size_t row;
  if (sink_tile) {
    const int slot = tc.slot;
    const bool slot_ok = slot >= 0 && slot < pv.n_sink_slots;
    if (!slot_ok && L > 0 && lane == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_SINKSLOT);
    t.valid = slot_ok ? max(0, min(kTileTokens, min(L, pv.sink) - u * kTileTokens)) : 0;
    row = (((size_t)max(slot, 0) * pv.hkv + kv) * pv.sink + (size_t)u * kTileTokens) * kD;
  } else {
    // recent ring: valid slots are [a0, a0 + nr) mod W, a prefix of every
    // tile (a0 is 0 mod 64 while the ring is filling; all slots once full)
    const int r0 = max(pv.sink, L - pv.recent);
    const int nr = max(0, L - r0);
    const int a0 = r0 % pv.recent;
    const int lo = (u - n_sink_tiles) * kTileTokens, hi = lo + kTileTokens;
    const int e1 = min(a0 + nr, pv.recent);
    const int e2 = max(0, a0 + nr - pv.recent);
    t.valid = max(0, min(hi, e1) - max(lo, a0)) + max(0, min(hi, e2) - lo);
    row = (((size_t)b * pv.hkv + kv) * pv.recent + lo) * kD;
  }
  // the four base pointers are first pinned in scalar registers: a choice
  // between the struct fields themselves was compiled into an indexed copy
  // of the struct in scratch memory, one more memory round trip per tile
  uint64_t sk = (uint64_t)(uintptr_t)pv.sink_k, sv = (uint64_t)(uintptr_t)pv.sink_v;
  uint64_t rk = (uint64_t)(uintptr_t)pv.recent_k, rv = (uint64_t)(uintptr_t)pv.recent_v;
  asm volatile("" : "+s"(sk), "+s"(sv), "+s"(rk), "+s"(rv));
  t.K = reinterpret_cast<const uint16_t *>(sink_tile ? sk : rk) + row;
  t.V = reinterpret_cast<const uint16_t *>(sink_tile ? sv : rv) + row;
}

// One wave computes one tile from its loaded rows: (m, l) per head (log2
// units, row-uniform for head 4 q + i) and o = sum over the four token
// phases of p V, staged in scratch[h][c] (original basis).
template <int GH>
__device__ __forceinline__ void bf16_tile_finish(const DecArgs &a, const TileRegs &r, int valid, const v8bf (&Aq)[4],
                                 float (*scratch)[kD], float (&m)[4], float (&l)[4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int G = a.pv.hq / a.pv.hkv;
  float o[GH][8];
  bf16_tile_math<GH>(r, valid, G, Aq, a.pv.sm_scale * kLog2e, m, l, o, scratch);
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    if (h < G) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v = o[h][c];
        v += lane_xor<16>(v);
        v += lane_xor<32>(v);
        if (q == 0) scratch[h][8 * n + c] = v;
      }
    }
  }
  wave_lds_sync();
}

// The same for tile u, loads included; returns its number of valid tokens
// (with none, m = -inf, l = 0 and nothing is staged).
template <int GH>
__device__ __forceinline__ int bf16_tile_compute(const DecArgs &a, const TileCtx &tc, int b, int kv, int u,
                                                 float (*scratch)[kD], float (&m)[4], float (&l)[4]) {
  const PoolView &pv = a.pv;
  TileSrc t;
  tile_source(pv, tc, b, kv, u, t);
  if (t.valid == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
    return 0;
  }
  TileRegs r;
  bf16_tile_load(t.K, t.V, t.valid, r);
  v8bf Aq[4];
  load_bf16_query(a.q + ((size_t)b * pv.hq + (size_t)kv * (pv.hq / pv.hkv)) * kD, pv.hq / pv.hkv, Aq);
  bf16_tile_finish<GH>(a, r, t.valid, Aq, scratch, m, l);
  return t.valid;
}

// One BF16 tile as its own (m, l, o) partial, written with coherent stores.
template <int GH>
__device__ void bf16_tile_partial(const DecArgs &a, const TileCtx &tc, int b, int kv, int u, float (*scratch)[kD],
                                  float *dst) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int G = a.pv.hq / a.pv.hkv;
  float m[4], l[4];
  const int valid = bf16_tile_compute<GH>(a, tc, b, kv, u, scratch, m, l);
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q + i;
      if (h < G) {
        st_coherent(dst + (size_t)h * kPartStride, m[i]);
        st_coherent(dst + (size_t)h * kPartStride + 1, l[i]);
      }
    }
  }
  for (int e = lane; e < G * kD; e += 64)
    st_coherent(dst + (size_t)(e / kD) * kPartStride + kPartO + e % kD, valid ? scratch[e / kD][e % kD] : 0.f);
  wave_lds_sync();
}


// Fold a tile staged by bf16_tile_finish (m, l per head, o in scratch) into
// the running state (o, st), online-softmax style.
template <int GH>
__device__ __forceinline__ void bf16_fold_staged(int G, const float (&m)[4], const float (&l)[4], float (*scratch)[kD],
                                                 float *o, float *st) {
  static_assert(GH == 4, "one M-tile of heads");
  const int lane = threadIdx.x & 63;
  // heads 0..3 are the C rows of lane group 0 (the other rows are padding)
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[kStTm + i] = m[i];
      st[kStTl + i] = l[i];
    }
  }
  wave_lds_sync();
  float al[4], be[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float ma = st[kStM + h], mt = st[kStTm + h];
    const float mx = fmaxf(ma, mt);   // finite: the tile has a valid token
    al[h] = ma > -INFINITY ? exp2_fast(ma - mx) : 0.f;
    be[h] = exp2_fast(mt - mx);
    if (lane == h) st[kStL + h] = fmaf(st[kStL + h], al[h], st[kStTl + h] * be[h]);
  }
  wave_lds_sync();
  if (lane < 4) st[kStM + lane] = fmaxf(st[kStM + lane], st[kStTm + lane]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + 64 * j, h = e >> 7;
    if (h < G) o[e] = fmaf(o[e], al[h], scratch[h][e & (kD - 1)] * be[h]);
  }
  wave_lds_sync();
}

// Tile u of one (sequence, KV head) folded into a wave's running BF16 state.
template <int GH>
__device__ __forceinline__ void bf16_tile_fold(const DecArgs &a, const TileCtx &tc, int b, int kv, int u,
                                               float (*scratch)[kD], float *o, float *st) {
  float m[4], l[4];
  if (bf16_tile_compute<GH>(a, tc, b, kv, u, scratch, m, l))
    bf16_fold_staged<GH>(a.pv.hq / a.pv.hkv, m, l, scratch, o, st);
}

// Combine the NW waves' history state into the split's partial.
template <int MT, int GH, int NW, bool MFMA>
__device__ void write_split_partial(ScanSmem<MT, GH, NW, MFMA> &sm, int G, float *dst, bool with_z) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, c = idx % kD;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
    float o = 0.f, l = 0.f;
    if (M > -INFINITY) {
      for (int w = 0; w < NW; ++w) {
        if (sm.m[w][h] == -INFINITY) continue;
        const float sc = exp2_fast(sm.m[w][h] - M);
        const float ov = MFMA ? sm.o[w][h][c] : sm.vacc[MFMA ? 0 : w][h][c >> 1][c & 1];
        o += sc * (with_z ? ov + sm.z[w][h][c >> 6] : ov);
        l += sc * sm.l[w][h];
      }
    }
    float *d = dst + (size_t)h * kPartStride;
    if (c == 0) {
      st_coherent(d, M);
      st_coherent(d + 1, l);
    }
    st_coherent(d + kPartO + c, o);
  }
}

// History page pipeline of one wave over the pages [pg0, pg1) of one
// (sequence, KV head): the wave takes pages first + i * NW, i < npg, with up
// to PF page copies in flight (LDS DMA).  The block-table entries of a span
// of kBtSpan pages are loaded together, 64 per register (lane k of bt0 holds
// the entry of the next page index with remainder k mod 64; bt1 and bt2 the
// following 64 each, shifted down every 64 pages).  One span covers every
// page of a wave up to 2.1 M tokens of history per workgroup, so the refill
// (which drains the wave's copies) is rare.
constexpr int kBtSpan = 192;
// Complete the loads of the block-table registers and redefine them through
// an empty asm: later reads of them (one readlane per page) then carry no
// compiler wait.  Without this the compiler, unable to prove across the
// loop that a refill load has landed, waits for every outstanding
// vector-memory operation, page copies included, at each page issue.
template <typename P>
__device__ __forceinline__ void bt_settle(P &p) {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" : "+v"(p.bt0), "+v"(p.bt1), "+v"(p.bt2));
}
// The same for the block-table registers and two loaded floats together.
template <typename P>
__device__ __forceinline__ void bt_settle(P &p, float &x, float &y) {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" : "+v"(p.bt0), "+v"(p.bt1), "+v"(p.bt2), "+v"(x), "+v"(y));
}

template <int NW, int PF>
struct PagePipe {
  const int32_t *btw;
  const uint8_t *pbase;
  size_t pstride;
  uint4 (*bufs)[kPageBytes / 16];
  uint32_t lds0;
  int bt0, bt1, bt2;
  int first, npg, issued;
  uint32_t inflight;   // bit j: page i + j (i = next page consumed) has a copy in flight
  bool bad;
};

// Block-table entries of the span starting at page index j (loads only).
template <int NW, int PF>
__device__ __forceinline__ void bt_load(PagePipe<NW, PF> &p, int j, int lane) {
  const int i = j + lane;
  p.bt0 = i < p.npg ? p.btw[(size_t)i * NW] : -1;
  p.bt1 = i + 64 < p.npg ? p.btw[(size_t)(i + 64) * NW] : -1;
  p.bt2 = i + 128 < p.npg ? p.btw[(size_t)(i + 128) * NW] : -1;
}

// Issues the first block-table loads without waiting for them: a bt_settle
// of p must come before pipe_prologue.
template <int NW, int PF>
__device__ __forceinline__ void pipe_init(PagePipe<NW, PF> &p, const PoolView &pv, int b, int kv, int pg0, int pg1,
                                          uint4 (*bufs)[kPageBytes / 16], int wave, int lane) {
  p.first = pg0 + wave;
  p.npg = p.first < pg1 ? (pg1 - p.first + NW - 1) / NW : 0;
  p.btw = pv.block_table + (size_t)b * pv.max_pages + p.first;
  bt_load(p, 0, lane);   // settled by the caller
  p.pbase = pv.pages + (size_t)kv * kPageBytes;
  p.pstride = (size_t)pv.hkv * kPageBytes;
  p.bufs = bufs;
  p.lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)bufs[0];
  p.issued = 0;
  p.inflight = 0;
  p.bad = false;
}

// Start the copy of page j (j < npg) into buffer j % PF; false if its
// block-table entry is out of range (then nothing is copied).
template <int NW, int PF>
__device__ __forceinline__ bool pipe_issue(PagePipe<NW, PF> &p, const PoolView &pv, int j, int lane) {
  if ((j & 63) == 0 && j > 0) {
    if (j % kBtSpan == 0) {
      bt_load(p, j, lane);
      bt_settle(p);
    } else {   // next 64 entries of the span
      p.bt0 = p.bt1;
      p.bt1 = p.bt2;
    }
  }
  const int ph = __builtin_amdgcn_readlane(p.bt0, j & 63);
  const bool ok = ph >= 0 && ph < pv.n_pages;
  if (ok) {
    const uint64_t base = (uint64_t)(uintptr_t)(p.pbase + (size_t)ph * p.pstride);
    dma_page(base, p.lds0 + (uint32_t)(j % PF) * kPageBytes, 16u * lane);
  } else {
    p.bad = true;
  }
  return ok;
}

template <int NW, int PF>
__device__ __forceinline__ void pipe_prologue(PagePipe<NW, PF> &p, const PoolView &pv, int lane) {
  for (; p.issued < PF && p.issued < p.npg; ++p.issued)
    if (pipe_issue(p, pv, p.issued, lane)) p.inflight |= 1u << p.issued;
}

// One page of the pipeline: wait for its copy, read it, refill the pipeline
// and fold the page into the state.  A page whose copy was never issued (its
// block-table entry is out of range) is skipped.
template <int MT, int NW, int PF, bool FULL, bool LUT>
__device__ __forceinline__ void pipe_step(PagePipe<NW, PF> &p, const PoolView &pv, int i, int n_hist,
                                          const QueryOps<MT> &qo, HistState<MT> &st, v4i *wl, int lane) {
  const int n = lane & 15, q = lane >> 4;
  const bool ok = p.inflight & 1u;
  PageRegs cur;
  // copies issued after page i that may still be outstanding
  wait_pages(__builtin_popcount(p.inflight >> 1));
  load_page(cur, (const uint8_t *)p.bufs[i % PF], n, q);   // in bounds also when page i was skipped
  wait_lds_reads();
  p.inflight >>= 1;
  if (p.issued < p.npg) {
    if (pipe_issue(p, pv, p.issued, lane)) p.inflight |= 1u << (PF - 1);
    ++p.issued;
  }
  if (ok) {
    const int valid = FULL ? kPageTokens : min(kPageTokens, n_hist - (p.first + i * NW) * kPageTokens);
    int2_page<MT, FULL, LUT>(cur, valid, qo, st, wl);
  }
}

// Consume every page of the pipeline (the prologue must have been issued).
// Only the last page of the history can be partly filled, so every page of
// the wave but possibly its last runs the full-page path.
template <int MT, int NW, int PF, bool LUT>
__device__ __forceinline__ void pipe_scan(PagePipe<NW, PF> &p, const PoolView &pv, int n_hist, const QueryOps<MT> &qo,
                                          HistState<MT> &st, v4i *wl, int lane) {
  const int full_pages = n_hist / kPageTokens;   // global pages [0, full_pages) hold 64 tokens
  const int nfull = min(p.npg, max(0, (full_pages - p.first + NW - 1) / NW));
  int i = 0;
  for (; i < nfull; ++i) pipe_step<MT, NW, PF, true, LUT>(p, pv, i, n_hist, qo, st, wl, lane);
  for (; i < p.npg; ++i) pipe_step<MT, NW, PF, false, LUT>(p, pv, i, n_hist, qo, st, wl, lane);
}

// Dynamic page order within a workgroup (48 to kDynMaxPages pages, one
// M-tile of heads): the block-table entries of the workgroup's pages sit in
// LDS and each wave takes the next page index from a shared counter
// whenever it frees a buffer, so the waves of a SIMD (which otherwise
// finish in age order, the oldest having issue priority) all run until the
// pages are gone.
constexpr int kDynMaxPages = 2048;
struct DynPages {
  int next_page;
  int bt[kDynMaxPages];   // block-table entries of pages pg0 + i
};

// Consume pages in the order the counter hands them out.  The wave starts
// with the prologue's two copies (pages wave and wave + NW, both full) and
// takes indices from dp->next_page (initialised to NW * PF) until they reach
// nfull, the workgroup's full pages.  Each index is drawn one page ahead, so
// the counter's round trip overlaps the page's compute, and its
// block-table entry is read together with the page.  Returns true on the
// wave that drew index nfull: it owns the workgroup's partly filled last
// page, if any.
template <int MT, int NW, int PF, bool LUT>
__device__ __forceinline__ bool pipe_scan_dyn(PagePipe<NW, PF> &p, const PoolView &pv, int nfull, DynPages *dp,
                                              const QueryOps<MT> &qo, HistState<MT> &st, v4i *wl, int lane) {
  static_assert(PF == 2, "the dynamic order is written for two page buffers");
  const int n = lane & 15, q = lane >> 4;
  bool own_tail = false;
  bool have_cur = true, have_nxt = true;
  int c = 0;   // buffer of the page consumed next; the other holds the one after it
  int jn = 0;  // the index drawn for the next refill
  if (lane == 0) jn = atomicAdd(&dp->next_page, 1);
  while (have_cur) {
    // copies issued after this page that may still be outstanding
    wait_pages(__builtin_popcount(p.inflight >> 1));
    PageRegs cur;
    load_page(cur, (const uint8_t *)p.bufs[c], n, q);
    const int j = __builtin_amdgcn_readfirstlane(jn);
    const bool have_new = j < nfull;
    const int ph = __builtin_amdgcn_readfirstlane(dp->bt[have_new ? j : 0]);
    wait_lds_reads();   // buffer c is read: it may be refilled
    const bool ok = p.inflight & 1u;
    p.inflight >>= 1;
    own_tail = own_tail || j == nfull;
    if (have_new) {
      if (ph >= 0 && ph < pv.n_pages) {
        dma_page((uint64_t)(uintptr_t)(p.pbase + (size_t)ph * p.pstride), p.lds0 + (uint32_t)c * kPageBytes,
                 16u * lane);
        p.inflight |= 1u << (PF - 1);
      } else {
        p.bad = true;
      }
      if (lane == 0) jn = atomicAdd(&dp->next_page, 1);
    }
    if (ok) int2_page<MT, true, LUT>(cur, kPageTokens, qo, st, wl);
    have_cur = have_nxt;
    have_nxt = have_new;
    c ^= 1;
  }
  return own_tail;
}

template <int MT>
__device__ __forceinline__ void hist_reset(HistState<MT> &st) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.mref[mt] = -INFINITY;
    st.lsum[mt] = st.z0[mt] = st.z1[mt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.facc[mt][nt] = 0.f;
  }
}

// Query operands of one head group into registers, from prepared LDS copies
// (qc[h] = {delta, Q_0, Q_1}), with the K metadata steps of the KV head
// folded in (see QueryOps).
template <int MT, int GH, bool LUT>
__device__ __forceinline__ void load_query_ops(const v4i *aq, const float (*qc)[4], int G, float sl2,
                                               const MetaSteps &ms, int lane, QueryOps<MT> &qo) {
  const int q = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    qo.A[mt][0] = aq[(mt * 2 + 0) * 64 + lane];
    qo.A[mt][1] = aq[(mt * 2 + 1) * 64 + lane];
    const int h = min(4 * mt + q, GH - 1);
    const bool hv = 4 * mt + q < G;
    const float q0 = hv ? qc[h][1] * sl2 : 0.f, q1 = hv ? qc[h][2] * sl2 : 0.f;
    qo.qa[mt] = hv ? qc[h][0] * sl2 * ms.kb * (LUT ? 1.0f / 32.0f : 1.0f) : 0.f;
    qo.qb0[mt] = q0 * ms.ka;
    qo.qb1[mt] = q1 * ms.ka;
    qo.qc[mt] = -ms.ktau * (q0 + q1);
  }
}

// Every wave's history state -> one (m, l, o) partial of the workgroup.
// The page buffers must be idle (sm.o aliases them).
template <int MT, int GH, int NW>
__device__ void flush_partial(ScanSmem<MT, GH, NW, true> &sm, HistState<MT> &st, int G, const MetaSteps &ms,
                              float *dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // value sums are kept in metadata code units: sum w s8 code and sum w z8
    // become sum w (s8 b) code and sum w (z8 a - tau)
    const float l16 = row16_sum(st.lsum[mt]);
    const float z0 = row16_sum(st.z0[mt]);
    const float z1 = row16_sum(st.z1[mt]);
    const int hh = 4 * mt + q;
    if (n == 0) {
      sm.m[wave][hh] = st.mref[mt];
      sm.l[wave][hh] = l16;
      sm.z[wave][hh][0] = fmaf(z0, ms.va, -ms.vtau * l16);
      sm.z[wave][hh][1] = fmaf(z1, ms.va, -ms.vtau * l16);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) sm.o[wave][hh][16 * nt + n] = st.facc[mt][nt] * ms.vb;
  }
  __syncthreads();
  write_split_partial<MT, GH, NW, true>(sm, G, dst, true);
}

// End of a split for one M-tile of heads (G <= 4).  Each wave, once its
// pages are done, stores its history state in its own (now idle) page
// buffers and loads its share of U_V (the last 512 threads, one quarter row
// each).  Then the workgroup combines the waves' history states and the
// tile waves' BF16 states, takes the history sum out of the rotated basis
// (bit reversal, Walsh-Hadamard butterfly, U_V^T / sqrt(d): R_V^T is linear,
// so applying it to every split's sum equals applying it once to the merged
// sum) and adds the BF16 part.  With one split the output is written here;
// otherwise one (m, l, o) partial in the original basis goes to dst.
template <int GH, int NW>
__device__ void split_epilogue(const DecArgs &a, int b, int kv, int split, ScanSmem<1, GH, NW, true> &sm,
                               const HistState<1> &st, const MetaSteps &ms, float *dst) {
  static_assert(GH == 4 && NW * 64 >= 512 + 256, "one M-tile of heads, 12 waves");
  constexpr int NT = NW * 64;
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = pv.hq / pv.hkv;
  const int S = a.n_splits;
  static_assert(sizeof(sm.pbuf[0]) >= kAccFloats * sizeof(float), "wave state fits in its page buffers");
  float *reg = reinterpret_cast<float *>(&sm.pbuf[wave][0][0]);
  // 1) this wave's history state: o = facc b_V + zero-point sums, per head q
  {
    const float l16 = row16_sum(st.lsum[0]);
    const float z0 = row16_sum(st.z0[0]), z1 = row16_sum(st.z1[0]);
    const float zz0 = fmaf(z0, ms.va, -ms.vtau * l16), zz1 = fmaf(z1, ms.va, -ms.vtau * l16);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) reg[kAccHist + q * kD + 16 * nt + n] = fmaf(st.facc[0][nt], ms.vb, nt < 4 ? zz0 : zz1);
    if (n == 0) {
      sm.m[wave][q] = st.mref[0];
      sm.l[wave][q] = l16;
    }
  }
  // 2) U_V rows for step 4: thread t >= NT - 512 owns row (t - (NT - 512)) / 4,
  // columns 32 ((t - (NT - 512)) % 4) .. + 32; the loads overlap the wait
  // for the other waves and the combine
  const int ut = tid - (NT - 512);
  const bool uown = ut >= 0;
  const int krow = (uown ? ut : 0) >> 2, upart = (uown ? ut : 0) & 3;
  float4 u[8];
  if (uown) {
    const float4 *urow = (const float4 *)(a.rv.U_V + ((size_t)kv * kD + krow) * kD + 32 * upart);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = urow[i];
  }
  __syncthreads();
  // 3) combine the waves (history: rotated basis, permuted for the butterfly)
  for (int idx = tid; idx < G * kD; idx += NT) {
    const int h = idx >> 7, c = idx & (kD - 1);
    float M = -INFINITY, Mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTileWaves; ++t) Mb = fmaxf(Mb, sm.tacc[t][4 * kD + kStM + h]);
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
    float o = 0.f, l = 0.f, ob = 0.f, lb = 0.f;
#pragma unroll
    for (int t = 0; t < kTileWaves; ++t) {
      const float mt = sm.tacc[t][4 * kD + kStM + h];
      if (mt > -INFINITY) {
        const float sc = exp2_fast(mt - Mb);
        ob = fmaf(sc, sm.tacc[t][idx], ob);
        lb = fmaf(sc, sm.tacc[t][4 * kD + kStL + h], lb);
      }
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm.m[w][h];
      if (mw > -INFINITY) {
        const float sc = exp2_fast(mw - M);
        o = fmaf(sc, reinterpret_cast<const float *>(&sm.pbuf[w][0][0])[kAccHist + idx], o);
        l = fmaf(sc, sm.l[w][h], l);
      }
    }
    sm.e.zs[h][bitrev7(c)] = o;   // (o P)[j] = o[bitrev(j)]
    sm.e.ob[h][c] = ob;
    if (c == 0) {
      sm.e.hm[h] = M;
      sm.e.hl[h] = l;
      sm.e.bm[h] = Mb;
      sm.e.bl[h] = lb;
    }
  }
  __syncthreads();
  // 4) Walsh-Hadamard butterfly per head (one wave each), then U_V^T
  if (wave < G) {
    float x0 = sm.e.zs[wave][lane], x1 = sm.e.zs[wave][lane + 64];
    fwht_lane_stages(x0, x1, lane);
    sm.e.zs[wave][lane] = x0 + x1;
    sm.e.zs[wave][lane + 64] = x0 - x1;
  }
  __syncthreads();
  if (uown) {
    for (int h = 0; h < G; ++h) {
      const float4 *zr = (const float4 *)(&sm.e.zs[h][32 * upart]);
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float4 za = zr[i], zb = zr[i + 1];
        sa = fmaf(za.x, u[i].x, fmaf(za.y, u[i].y, fmaf(za.z, u[i].z, fmaf(za.w, u[i].w, sa))));
        sb = fmaf(zb.x, u[i + 1].x, fmaf(zb.y, u[i + 1].y, fmaf(zb.z, u[i + 1].z, fmaf(zb.w, u[i + 1].w, sb))));
      }
      float sum = sa + sb;
      sum += lane_xor<1>(sum);
      sum += lane_xor<2>(sum);
      if (upart == 0) sm.e.ot[h][krow] = sum * kInvSqrtDf;
    }
  }
  __syncthreads();
  // 5) history and BF16 parts together
  for (int idx = tid; idx < G * kD; idx += NT) {
    const int h = idx >> 7, c = idx & (kD - 1);
    const float Mh = sm.e.hm[h], Mb = sm.e.bm[h], Mt = fmaxf(Mh, Mb);
    const float ah = Mh > -INFINITY ? exp2_fast(Mh - Mt) : 0.f;
    const float ab = Mb > -INFINITY ? exp2_fast(Mb - Mt) : 0.f;
    const float l = fmaf(ah, sm.e.hl[h], ab * sm.e.bl[h]);
    const float o = fmaf(ah, sm.e.ot[h][c], ab * sm.e.ob[h][c]);
    if (S == 1 && a.n_prefix == 0) {
      a.out[((size_t)b * pv.hq + (size_t)kv * G + h) * kD + c] = l > 0.f ? o / l : 0.f;
    } else {
      float *d = dst + (size_t)h * kPartStride;
      if (c == 0) {
        st_coherent(d, Mt);
        st_coherent(d + 1, l);
      }
      st_coherent(d + kPartO + c, o);
    }
  }
}

template <int MT, int GH, int NW, bool DYN, bool LUT>
__device__ void run_scan_mfma(const DecArgs &a, int b, int kv, int split, float *dst,
                              ScanSmem<MT, GH, NW, true> &sm, DynPages *dp) {
  constexpr int PF = ScanSmem<MT, GH, NW, true>::PF;
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = pv.hq / pv.hkv;
  const int bh = b * pv.hkv + kv;
  const int L = pv.seq_lens[b];
  const int n_hist = max(0, L - pv.sink - pv.recent);
  const int n_pages = (n_hist + kPageTokens - 1) / kPageTokens;
  const int pg0 = a.prefix_pages + split * a.pages_per_split;   // the shared prefix has a scan of its own
  const int pg1 = min(min(n_pages, pg0 + a.pages_per_split), pv.max_pages);
  if (n_pages > pv.max_pages && split == 0 && tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);

  // Vector-memory loads complete in issue order, so a load issued after the
  // page copies waits for them.  Every load whose value is used after the
  // copies start is therefore issued first and completed in one round trip:
  // the clip thresholds, the first block-table entries and (threads
  // 0..255) the query preparation's loads.  The waves without preparation
  // work start their copies as soon as those land (the tile waves of one
  // M-tile of heads after their tiles).
  float tk = a.rv.tau_K[kv], tv = a.rv.tau_V[kv];
  const uint32_t lutk = LUT ? levels_of(a.rv, kv, false) : OSCAR_UNIFORM_LEVELS;
  const uint32_t lutv = LUT ? levels_of(a.rv, kv, true) : OSCAR_UNIFORM_LEVELS;
  const TileCtx tc{max(0, L), pv.sink_slot[b]};
  const int S = a.n_splits;
  PagePipe<NW, PF> pipe;
  pipe_init(pipe, pv, b, kv, pg0, pg1, sm.pbuf[wave], wave, lane);
  // several M-tiles: long scans (16 pages per wave and more) take every BF16
  // tile after the pages, short ones four of them first (on waves 0..3)
  const int npg_wg = pg1 - pg0;
  const bool long_scan = npg_wg >= 16 * NW;
  const int early = (MT == 1 || long_scan) ? 0 : 4;
  // one M-tile of heads: the last kTileWaves waves run every BF16 tile first,
  // from the start (a tile needs the query only in its original basis, and
  // its loads then go out ahead of the wave's page copies), each wave into a
  // running state of its own outside the page buffers, and then join the
  // page stream
  const int tw = MT == 1 ? wave - (NW - kTileWaves) : -1;   // this wave's tile-wave index, or < 0
  // where the workgroup has two rounds of prologue pages or more and its
  // block-table entries fit in LDS, pages are handed out dynamically
  const bool dyn = DYN && npg_wg >= 2 * NW * PF && npg_wg <= kDynMaxPages;
  // pages [pg0, pg0 + nfull) hold 64 tokens (only the history's last page can hold fewer)
  const int nfull = max(0, min(pg1, n_hist / kPageTokens) - pg0);
  // threads that load the workgroup's block-table entries into LDS (the
  // tile waves do not)
  constexpr int kBtThreads = 64 * (MT == 1 ? NW - kTileWaves : NW);
  constexpr int kDynPer = (kDynMaxPages + kBtThreads - 1) / kBtThreads;
  int dbt[kDynPer];
  if (dyn && tid < kBtThreads) {
    const int32_t *row = pv.block_table + (size_t)b * pv.max_pages + pg0;
#pragma unroll
    for (int r = 0; r < kDynPer; ++r) {
      const int i = tid + r * kBtThreads;
      dbt[r] = i < npg_wg ? row[i] : -1;
    }
  }
  // block-table entries to LDS and the prologue copies of waves 4.. once the
  // first loads have landed (published by the barrier or readiness count
  // that follows the preparation)
  auto after_loads = [&] {
    bt_settle(pipe, tk, tv);
    if (dyn) {
#pragma unroll
      for (int r = 0; r < kDynPer; ++r) {
        const int i = tid + r * kBtThreads;
        if (i < npg_wg) dp->bt[i] = dbt[r];
      }
      if (tid == 0) dp->next_page = NW * PF;
    }
    if (wave >= 4) pipe_prologue(pipe, pv, lane);
  };
  QSmem<MT, GH> &qs = sm.qprep();
  if constexpr (MT == 1) {
    // No barrier between the start and the pages: waves 0..3 prepare the
    // query (synchronising among themselves), waves 4..7 start their copies,
    // the tile waves run their tiles and then start their copies.  Waves
    // 0..7 each raise sm.ready once their part (query operands of their head,
    // block-table entries) is in LDS; every wave waits for all eight before
    // it reads the query operands.  Both counters start at zero.
    if (tid == 0) {
      sm.prep_ctr = 0;
      sm.ready = 0;
    }
    __syncthreads();
    if (tw >= 0) {
      // tiles u = split + S k with k = tw mod kTileWaves, one after the other
      float *to = &sm.tacc[tw][0], *tst = &sm.tacc[tw][4 * kD];
#pragma unroll
      for (int j = 0; j < 8; ++j) to[lane + 64 * j] = 0.f;
      if (lane < 4) {
        tst[kStM + lane] = -INFINITY;
        tst[kStL + lane] = 0.f;
      }
      wave_lds_sync();
      for (int u = split + S * tw; u < a.n_chunks; u += S * kTileWaves)
        bf16_tile_fold<GH>(a, tc, b, kv, u, sm.wave[wave].tile, to, tst);
      bt_settle(pipe, tk, tv);
      pipe_prologue(pipe, pv, lane);
    } else {
      query_prep<MT, GH>(a, b, kv, qs, nullptr, after_loads, &sm.prep_ctr);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_fetch_add(&sm.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    while (__hip_atomic_load(&sm.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NW - kTileWaves)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    query_prep<MT, GH>(a, b, kv, qs, nullptr, after_loads);
  }
  const MetaSteps ms = meta_steps(tk, tv);
  QueryOps<MT> qo;
  load_query_ops<MT, GH, LUT>(qs.aq, qs.qc, G, pv.sm_scale * kLog2e, ms, lane, qo);
  qo.lutk = lutk;
  qo.lutv = lutv;
  // several M-tiles: the query scratch is reused by the weights and the BF16 tiles
  if constexpr (MT != 1) __syncthreads();
  // Several M-tiles, BF16 tiles u = split + S k of this workgroup: on short
  // scans (under 16 pages per wave) tiles k < 4 run first on waves 3..0 (the
  // preparing waves, whose history pages are the last to arrive, and which
  // finish their pages before the others); the rest run after the history
  // pages, from the last wave down.  An early tile goes before the wave's
  // page copies: its loads would otherwise complete behind them.  Long
  // scans: every tile runs after the pages on waves 0..3, which finish their
  // pages well before the younger waves of their SIMDs (the oldest wave has
  // issue priority), so the tiles hide behind the remaining page stream.
  // (The tile scratch overlaps the query scratch, which is dead after the
  // barrier above.)
  float *parts = a.part + (size_t)bh * a.n_parts * G * kPartStride;
  if (wave < 4) {
    const int u = split + S * (early - 1 - wave);
    if (wave < early && u < a.n_chunks)
      bf16_tile_partial<GH>(a, tc, b, kv, u, sm.wave[wave].tile, parts + (size_t)(S + a.n_prefix + u) * G * kPartStride);
    // the preparing waves start their copies only now: issuing them inside
    // the preparation would stall those waves (the CU accepts copy requests
    // at the memory rate) and with them every wave waiting on the preparation
    pipe_prologue(pipe, pv, lane);
  }
  HistState<MT> st;
  hist_reset(st);
  v4i *wl = sm.wave[wave].wl;
  // rows 4h + 3 of the weight operands stay zero; the rest is rewritten per page
#pragma unroll
  for (int i = 0; i < MT * 2; ++i) wl[i * 64 + lane] = v4i{0, 0, 0, 0};
  if (dyn) {
    if (pipe_scan_dyn<MT, NW, PF, LUT>(pipe, pv, nfull, dp, qo, st, wl, lane) && nfull < npg_wg) {
      // the partly filled last page, on the wave that drew its index (its
      // buffers are idle: every copy it issued has been consumed)
      const int ph = __builtin_amdgcn_readfirstlane(dp->bt[nfull]);
      if (ph >= 0 && ph < pv.n_pages) {
        dma_page((uint64_t)(uintptr_t)(pipe.pbase + (size_t)ph * pipe.pstride), pipe.lds0, 16u * lane);
        wait_pages(0);
        PageRegs cur;
        load_page(cur, (const uint8_t *)pipe.bufs[0], lane & 15, lane >> 4);
        wait_lds_reads();
        int2_page<MT, false, LUT>(cur, n_hist - (pg0 + nfull) * kPageTokens, qo, st, wl);
      } else {
        pipe.bad = true;
      }
    }
  } else {
    pipe_scan<MT, NW, PF, LUT>(pipe, pv, n_hist, qo, st, wl, lane);
  }
  if (pipe.bad && lane == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
  if constexpr (MT == 1) {
    split_epilogue<GH, NW>(a, b, kv, split, sm, st, ms, dst);
    return;
  }
  for (int u = split + S * early; u < a.n_chunks; u += S) {
    const int k = u / S - early;
    if ((long_scan ? k % 4 : NW - 1 - k % NW) == wave)
      bf16_tile_partial<GH>(a, tc, b, kv, u, sm.wave[wave].tile, parts + (size_t)(S + a.n_prefix + u) * G * kPartStride);
  }
  flush_partial<MT, GH, NW>(sm, st, G, ms, dst);
}

template <int MT, int GH, int NW>
__device__ void run_scan_valu(const DecArgs &a, int b, int kv, int split, float *dst,
                              ScanSmem<MT, GH, NW, false> &sm) {
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = pv.hq / pv.hkv;
  const int bh = b * pv.hkv + kv;
  const int L = pv.seq_lens[b];
  const int n_hist = max(0, L - pv.sink - pv.recent);
  const int n_pages = (n_hist + kPageTokens - 1) / kPageTokens;
  const int pg0 = a.prefix_pages + split * a.pages_per_split;   // the shared prefix has a scan of its own
  const int pg1 = min(min(n_pages, pg0 + a.pages_per_split), pv.max_pages);
  if (n_pages > pv.max_pages && split == 0 && tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
  const float *qrot = a.qrot + (size_t)bh * GH * kD;
  for (int h = wave; h < G; h += NW) {
    float s0 = qrot[h * kD + lane], s1 = qrot[h * kD + 64 + lane];
    for (int o = 32; o > 0; o >>= 1) {
      s0 += __shfl_xor(s0, o, 64);
      s1 += __shfl_xor(s1, o, 64);
    }
    if (lane == 0) {
      sm.qsum[h][0] = s0;
      sm.qsum[h][1] = s1;
    }
  }
  for (int e = tid; e < NW * MT * 4; e += blockDim.x) {
    sm.m[e / (MT * 4)][e % (MT * 4)] = -INFINITY;
    sm.l[e / (MT * 4)][e % (MT * 4)] = 0.f;
  }
  for (int e = tid; e < NW * GH * 64 * 2; e += blockDim.x) (&sm.vacc[0][0][0][0])[e] = 0.f;
  __syncthreads();
  const ValuWave st{sm.m[wave], sm.l[wave], sm.vacc[wave]};
  const float sl2 = pv.sm_scale * kLog2e;
  const MetaSteps ms = meta_steps(a.rv, kv);
  const uint32_t lutk = levels_of(a.rv, kv, false), lutv = levels_of(a.rv, kv, true);
  const int32_t *btab = pv.block_table + (size_t)b * pv.max_pages;
  bool bad = false;
  for (int pg = pg0 + wave; pg < pg1; pg += NW) {
    const int ph = btab[pg];
    if (ph < 0 || ph >= pv.n_pages) {
      bad = true;
      continue;
    }
    const uint8_t *P = pv.pages + ((size_t)ph * pv.hkv + kv) * kPageBytes;
    const int valid = min(kPageTokens, n_hist - pg * kPageTokens);
    if (valid == kPageTokens) int2_page_valu<true>(P, valid, G, qrot, sm.qsum, sl2, ms, st, sm.wave[wave].pw, lutk, lutv);
    else int2_page_valu<false>(P, valid, G, qrot, sm.qsum, sl2, ms, st, sm.wave[wave].pw, lutk, lutv);
  }
  if (bad && lane == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
  __syncthreads();
  write_split_partial<MT, GH, NW, false>(sm, G, dst, false);
}

// Merge of one (sequence, KV head), by the last workgroup to finish its
// split: log-sum-exp merge of the history splits (rotated basis), then P, H
// and U_V^T once; merge of the BF16 tiles; combine and normalise.  Partials
// written by other workgroups are read with device-coherent loads, issued in
// batches so that the merge costs a few memory round trips, not one per
// partial.  The U_V rows are loaded once the partial loads are out, by
// threads that do not compute the per-head weights, so that their latency
// overlaps the weights and the weighted sums.
template <int GH, int NT>
__device__ void merge_item(const DecArgs &a, int b, int kv, const float *hist, int n_hist_parts, const float *tiles,
                           int n_tile_parts, MergeSmem<GH> &sm) {
  // (head, channel quad) items per thread when each item takes all partials
  // (quads padded to whole waves)
  constexpr int kItems = ((GH * (kD / 4) + 63) / 64 * 64 + NT - 1) / NT;
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int G = pv.hq / pv.hkv;
  const int S = n_hist_parts, P = n_hist_parts + n_tile_parts;
  // partial p: history split p < S, else BF16 tile p - S; [G][kPartStride]
  // each.  A buffer resource per segment; the partial's offset (p is
  // wave-uniform) goes in the scalar offset, the lane's (head, channels)
  // offset in the vector offset.
  const int pstride = G * kPartStride;
  const __amdgpu_buffer_rsrc_t rs_hist = coherent_rsrc(hist, (uint32_t)(S * pstride * 4));
  const __amdgpu_buffer_rsrc_t rs_tile = coherent_rsrc(tiles, (uint32_t)(n_tile_parts * pstride * 4));
  // 16 bytes at float offset off of partial p (p wave-uniform)
  auto part4 = [&](int p, uint32_t off) -> float4 {
    return p < S ? ld_coherent4(rs_hist, 4u * off, (uint32_t)(p * pstride * 4))
                 : ld_coherent4(rs_tile, 4u * off, (uint32_t)((p - S) * pstride * 4));
  };
  // U_V rows for step 4: the last kUT threads own row k = t' / kLPR
  // (t' = t - (NT - kUT)), channels kCPL (t' % kLPR) .. + kCPL.  With 12
  // waves these are waves 4..11, so waves 0..3 are free for step 2.
  constexpr int kUT = NT >= 512 ? 512 : 256;
  constexpr int kLPR = kUT / kD, kCPL = kD / kLPR;
  const int ut = tid - (NT - kUT);
  const bool uown = ut >= 0;
  const int krow = (ut >= 0 ? ut : 0) / kLPR, upart = (ut >= 0 ? ut : 0) % kLPR;
  const float4 *urow = (const float4 *)(a.rv.U_V + (size_t)kv * kD * kD + (size_t)krow * kD + kCPL * upart);
  float4 u[kCPL / 4];
  // 1) one round of device-coherent loads: the first kPer partials of each
  // thread's slice (thread -> head, channel quad, slice; 16 bytes each) into
  // registers, and the (m, l) headers of every partial into LDS.  Further
  // rounds (only when P > kPer * slices) reload values in step 3.  The quads
  // of a slice are padded to whole waves, so the slice (and with it the
  // partial index) is wave-uniform; padding lanes load head 0 and are idle.
  constexpr int kPer = 9;   // one round covers 6 x 9 = 54 partials at G = 4 (32 splits + 20 tiles at batch 1)
  const int nq = G * (kD / 4);
  const int nqp = (nq + 63) & ~63;
  const int nsl = min(kMergeSlices, min(max(1, NT / nqp), 24 / G));
  const int nitem = nqp * nsl;   // <= kItems * NT
  const int rounds = (P + nsl * kPer - 1) / (nsl * kPer);
  float4 val[kItems][kPer];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int e = tid + it * NT;
    if (e >= nitem) break;
    const int qd = e % nqp;
    const int sl = __builtin_amdgcn_readfirstlane(e / nqp);
    const uint32_t off = qd < nq ? (uint32_t)((qd >> 5) * kPartStride + kPartO + 4 * (qd & 31)) : (uint32_t)kPartO;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = sl + nsl * j;
      val[it][j] = p < P ? part4(p, off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  for (int e = tid; e < P * G; e += blockDim.x) {   // partial e / G, head e % G
    const float2 hv = ld_coherent2(e < S * G ? hist + (size_t)e * kPartStride : tiles + (size_t)(e - S * G) * kPartStride);
    sm.ml[e][0] = hv.x;
    sm.ml[e][1] = hv.y;
  }
  __syncthreads();
  // U_V rows once every wave has issued its partial loads (the memory
  // pipeline serves a CU's loads in order, so earlier they would delay the
  // loads that step 2 waits for); they are needed only in step 4
  asm volatile("" ::: "memory");
  if (uown) {
#pragma unroll
    for (int i = 0; i < kCPL / 4; ++i) u[i] = urow[i];
  }
  // 2) per head: maxima, weights, denominators
  for (int h = wave; h < G; h += nwaves) {
    float Mh = -INFINITY, Mb = -INFINITY;
    for (int p = lane; p < P; p += 64) {
      const float m = sm.ml[p * G + h][0];
      if (p < S) Mh = fmaxf(Mh, m);
      else Mb = fmaxf(Mb, m);
    }
    Mh = wave_max(Mh);
    Mb = wave_max(Mb);
    float lh = 0.f, lb = 0.f;
    for (int p = lane; p < P; p += 64) {
      const float m = sm.ml[p * G + h][0];
      const float ref = p < S ? Mh : Mb;
      const float w = m > -INFINITY ? exp2_fast(m - ref) : 0.f;
      sm.wgt[p][h] = w;
      if (p < S) lh = fmaf(w, sm.ml[p * G + h][1], lh);
      else lb = fmaf(w, sm.ml[p * G + h][1], lb);
    }
    lh = wave_sum(lh);
    lb = wave_sum(lb);
    if (lane == 0) {
      const float Mt = fmaxf(Mh, Mb);
      const float ah = Mh > -INFINITY ? exp2_fast(Mh - Mt) : 0.f;
      const float ab = Mb > -INFINITY ? exp2_fast(Mb - Mt) : 0.f;
      const float den = ah * lh + ab * lb;
      sm.hs[h][0] = ah;
      sm.hs[h][1] = ab;
      sm.hs[h][2] = den > 0.f ? 1.0f / den : 0.f;
    }
  }
  __syncthreads();
  // 3) weighted sums per slice (first round from registers, further rounds
  // reload), then the slices are added in a fixed order
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int e = tid + it * NT;
    if (e >= nitem) break;
    const int qd = e % nqp;
    const int sl = __builtin_amdgcn_readfirstlane(e / nqp);
    const bool act = qd < nq;
    const int h = act ? qd >> 5 : 0, c = 4 * (qd & 31);
    const uint32_t off = (uint32_t)(h * kPartStride + kPartO + c);
    float4 hs4 = make_float4(0.f, 0.f, 0.f, 0.f), bs4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < rounds; ++r) {
      const int p_base = nsl * kPer * r;
      float4 v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int p = p_base + sl + nsl * j;
        v[j] = r == 0 ? val[it][j] : (p < P ? part4(p, off) : make_float4(0.f, 0.f, 0.f, 0.f));
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int p = p_base + sl + nsl * j;
        if (p < P) {
          const float w = sm.wgt[p][h];
          float4 &acc = p < S ? hs4 : bs4;
          acc.x = fmaf(w, v[j].x, acc.x);
          acc.y = fmaf(w, v[j].y, acc.y);
          acc.z = fmaf(w, v[j].z, acc.z);
          acc.w = fmaf(w, v[j].w, acc.w);
        }
      }
    }
    if (act) {
      *(float4 *)(sm.red[0] + (size_t)sl * G * kD + h * kD + c) = hs4;
      *(float4 *)(sm.red[1] + (size_t)sl * G * kD + h * kD + c) = bs4;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, c = idx % kD;
    float acc_h = 0.f, acc_b = 0.f;
    for (int sl = 0; sl < nsl; ++sl) {
      acc_h += sm.red[0][(size_t)sl * G * kD + idx];
      acc_b += sm.red[1][(size_t)sl * G * kD + idx];
    }
    sm.zs[h][bitrev7(c)] = acc_h;   // (o P)[j] = o[bitrev(j)]
    sm.ob[h][c] = acc_b;
  }
  __syncthreads();
  // Walsh-Hadamard butterfly of each head's permuted sum, one wave per head:
  // lane l holds elements l and l + 64 (stage 64 in registers, the rest by
  // lane exchanges)
  for (int h = wave; h < G; h += nwaves) {
    float x0 = sm.zs[h][lane], x1 = sm.zs[h][lane + 64];
    fwht_lane_stages(x0, x1, lane);
    sm.zs[h][lane] = x0 + x1;
    sm.zs[h][lane + 64] = x0 - x1;
  }
  __syncthreads();
  // 4) o_hist[h][k] = sum_j z[h][j] U_V[k][j] / sqrt(d)
  // two partial sums per head (independent FMA chains), then the kLPR
  // lanes of a row are added
  if (uown) {
    for (int h = 0; h < G; ++h) {
      const float4 *zr = (const float4 *)(&sm.zs[h][kCPL * upart]);
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int i = 0; i < kCPL / 4; i += 2) {
        const float4 za = zr[i], zb = zr[i + 1];
        const float4 ua = u[i], ub = u[i + 1];
        sa = fmaf(za.x, ua.x, fmaf(za.y, ua.y, fmaf(za.z, ua.z, fmaf(za.w, ua.w, sa))));
        sb = fmaf(zb.x, ub.x, fmaf(zb.y, ub.y, fmaf(zb.z, ub.z, fmaf(zb.w, ub.w, sb))));
      }
      float s = sa + sb;
      s += lane_xor<1>(s);
      if constexpr (kLPR == 4) s += lane_xor<2>(s);
      if (upart == 0) sm.ot[h][krow] = s * kInvSqrtDf;
    }
  }
  __syncthreads();
  // 5) combine and normalise
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, c = idx % kD;
    const float res = (sm.hs[h][0] * sm.ot[h][c] + sm.hs[h][1] * sm.ob[h][c]) * sm.hs[h][2];
    a.out[((size_t)b * pv.hq + (size_t)kv * G + h) * kD + c] = res;
  }
}

// Merge of the S partials of one (sequence, KV head) whose splits have
// already left the rotated basis and folded in the BF16 tiles: a plain
// log-sum-exp merge, by the last workgroup to finish.  Waves 0..G-1 form one
// head's weights each; meanwhile every thread has its first kPer partial
// loads (16 bytes each, device-coherent) in flight.
template <int GH, int NT>
__device__ void merge_plain(const DecArgs &a, int b, int kv, const float *parts, int S, PlainMergeSmem<GH> &sm) {
  constexpr int kPer = 8;
  const PoolView &pv = a.pv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = pv.hq / pv.hkv;
  const int pstride = G * kPartStride;
  const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(parts, (uint32_t)(S * pstride * 4));
  // thread -> (head, channel quad) item of slice sl (quads padded to whole
  // waves, so the slice is wave-uniform); slice sl takes partials sl + nsl j
  const int nq = G * (kD / 4);
  const int nqp = (nq + 63) & ~63;
  const int nsl = min(kMergeSlices, max(1, NT / nqp));
  const bool item = tid < nqp * nsl;
  const int qd = tid % nqp;
  const int sl = __builtin_amdgcn_readfirstlane(tid / nqp);
  const bool act = item && qd < nq;
  const int h = act ? qd >> 5 : 0, c = 4 * (qd & 31);
  const uint32_t off = 4u * (uint32_t)(h * kPartStride + kPartO + c);
  float4 v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = sl + nsl * j;
    v[j] = item && p < S ? ld_coherent4(rs, off, (uint32_t)(p * pstride * 4)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (wave < G) {
    float mx = -INFINITY;
    float2 ml[kMaxSplits / 64];
#pragma unroll
    for (int r = 0; r < kMaxSplits / 64; ++r) {
      const int p = lane + 64 * r;
      ml[r] = p < S ? ld_coherent2(parts + (size_t)p * pstride + (size_t)wave * kPartStride) : make_float2(-INFINITY, 0.f);
      mx = fmaxf(mx, ml[r].x);
    }
    mx = wave_max(mx);
    float den = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxSplits / 64; ++r) {
      const int p = lane + 64 * r;
      const float w = ml[r].x > -INFINITY ? exp2_fast(ml[r].x - mx) : 0.f;
      if (p < S) sm.wgt[p][wave] = w;
      den = fmaf(w, ml[r].y, den);
    }
    den = wave_sum(den);
    if (lane == 0) sm.inv[wave] = den > 0.f ? 1.0f / den : 0.f;
  }
  __syncthreads();
  if (item) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < S; p0 += nsl * kPer) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int p = p0 + sl + nsl * j;
        if (p0 > 0)
          v[j] = p < S ? ld_coherent4(rs, off, (uint32_t)(p * pstride * 4)) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int p = p0 + sl + nsl * j;
        if (p < S) {
          const float w = sm.wgt[p][h];
          acc.x = fmaf(w, v[j].x, acc.x);
          acc.y = fmaf(w, v[j].y, acc.y);
          acc.z = fmaf(w, v[j].z, acc.z);
          acc.w = fmaf(w, v[j].w, acc.w);
        }
      }
    }
    if (act) *(float4 *)(sm.red[sl] + h * kD + c) = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < nsl; ++k) acc += sm.red[k][idx];
    a.out[((size_t)b * pv.hq + (size_t)kv * G) * kD + idx] = acc * sm.inv[idx / kD];
  }
}

// Register budget: three waves per SIMD for one M-tile of heads (G <= 4), two
// otherwise; the VALU reference takes what it needs.
template <int MT, int GH, bool MFMA, bool LUT>
__global__ void __launch_bounds__((64 * scan_waves<MT, MFMA>()))
__attribute__((amdgpu_waves_per_eu(MFMA ? (MT == 1 ? 3 : 2) : 1)))
decode_scan_kernel(DecArgs a) {
  constexpr int NW = scan_waves<MT, MFMA>();
  const PoolView &pv = a.pv;
  const int BH = pv.batch * pv.hkv;
  const int bh = blockIdx.x % BH, split = blockIdx.x / BH;
  const int b = bh / pv.hkv, kv = bh % pv.hkv;
  const int G = pv.hq / pv.hkv;
  const int wave = threadIdx.x >> 6;
  const int S = a.n_splits;
  float *parts = a.part + (size_t)bh * a.n_parts * G * kPartStride;
  __shared__ ScanUnion<MT, GH, NW, MFMA> sm;
  if constexpr (!MFMA) {
    // BF16 tile u runs on workgroup u % S, wave (u / S) % NW, before its pages
    const TileCtx tc = tile_ctx(pv, b);
    for (int u = split; u < a.n_chunks; u += S) {
      if (((u / S) % NW) == wave)
        bf16_tile_partial<GH>(a, tc, b, kv, u, sm.s.wave[wave].tile, parts + (size_t)(S + a.n_prefix + u) * G * kPartStride);
    }
  }
  float *dst = parts + (size_t)split * G * kPartStride;
  __shared__ int last_flag;
  if constexpr (MFMA && MT == 1) {
    // the split's partial leaves the rotated basis in the split itself; with
    // one split the output is already written
    __shared__ DynPages dp;
    run_scan_mfma<MT, GH, NW, true, LUT>(a, b, kv, split, dst, sm.s, &dp);
    if (a.n_prefix == 0) {
      if (S == 1 || !arrive_last(&a.counters[bh], S, &last_flag)) return;
      merge_plain<GH, 64 * NW>(a, b, kv, parts, S, sm.pm);
      return;
    }
    // shared prefix: the splits' partials (original basis, slots 0..S-1)
    // and the prefix chunks' (rotated basis, slots S..), inverse-rotated
    // once by the two-group merge
    if (S == 1) {
      stores_complete();
      __syncthreads();
    } else if (!arrive_last(&a.counters[bh], S, &last_flag)) {
      return;
    }
    merge_item<GH, 64 * NW>(a, b, kv, parts + (size_t)S * G * kPartStride, a.n_prefix, parts, S, sm.g);
    return;
  } else if constexpr (MFMA) {
    // several M-tiles (8 waves, heavier pages): the static page order
    // measured faster on the GQA-12 shared-prefix workload
    run_scan_mfma<MT, GH, NW, false, LUT>(a, b, kv, split, dst, sm.s, nullptr);
  }
  else run_scan_valu<MT, GH, NW>(a, b, kv, split, dst, sm.s);
  if (S == 1) {
    // the only workgroup of its (sequence, KV head): no counter round trip,
    // only its own partial stores completed before any thread reads them
    stores_complete();
    __syncthreads();
  } else if (!arrive_last(&a.counters[bh], S, &last_flag)) {
    return;
  }
  // the shared-prefix chunks' partials (rotated basis, written by the
  // prefix scan before this launch) merge as further history splits
  const int SH = S + a.n_prefix;
  merge_item<GH, 64 * NW>(a, b, kv, parts, SH, parts + (size_t)SH * G * kPartStride, a.n_chunks, sm.g);
}


// ===========================================================================
// shared-prefix scan
// ===========================================================================
// The leading prefix_pages history pages are the same physical pages for
// every sequence.  They are scanned once per KV head for up to kPfxWaves
// sequences at a time: a workgroup takes one chunk of those pages and one
// group of sequences, streams each page into LDS once, and every wave
// folds it into the state of its own sequence (all its query heads, the
// page math of the per-sequence scan).  Each wave then writes its
// sequence's (m, l, o) partial of the chunk, rotated basis, into the
// history-split slots n_splits + chunk; the per-sequence scan, launched
// after this one, merges them with its own splits.
constexpr int kPfxWaves = 8;          // sequences per workgroup, one per wave
constexpr int kPfxBufs = 4;           // page buffers of the workgroup's ring
constexpr int kPfxMaxChunk = 1024;    // pages per chunk (block-table entries in LDS)
static_assert(kMaxPrefixPages <= kPfxMaxChunk * (kMaxParts / 4), "the largest prefix fits the chunk limits");

// Query operands of one (sequence, KV head) in the workspace: the A
// operands of the logit MFMA, then {delta, Q_0, Q_1, 0} per head.
template <int MT, int GH>
constexpr size_t pq_floats() { return (size_t)MT * 2 * 64 * 4 + (size_t)GH * 4; }

// grid: B * Hkv; block: 256.
template <int MT, int GH>
__global__ void __launch_bounds__(256) prefix_prep_kernel(DecArgs a) {
  __shared__ QSmem<MT, GH> sm;
  const int bh = blockIdx.x;
  query_prep<MT, GH>(a, bh / a.pv.hkv, bh % a.pv.hkv, sm, nullptr, [] {});   // ends with a barrier
  float *dst = a.pq + (size_t)bh * pq_floats<MT, GH>();
  for (int e = threadIdx.x; e < MT * 2 * 64; e += blockDim.x) ((v4i *)dst)[e] = sm.aq[e];
  for (int e = threadIdx.x; e < GH * 4; e += blockDim.x) dst[MT * 2 * 64 * 4 + e] = (&sm.qc[0][0])[e];
}

template <int MT>
struct PfxSmem {
  uint4 pbuf[kPfxBufs][kPageBytes / 16];
  v4i wl[kPfxWaves][MT * 2 * 64];
  int bt[kPfxMaxChunk];   // block-table entries of the chunk (sequence 0)
  int avail;              // pages 0 .. avail - 1 are in LDS (raised by wave 0)
  int done[kPfxWaves];    // per wave: pages 0 .. done - 1 read into its registers
};

// Wait until at most n (<= 3) pages' copies are outstanding (5 loads each).
__device__ __forceinline__ void wait_pages3(int n) {
  if (n >= 3) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
  else wait_pages(n);
}

// grid: 8 * ceil(n_prefix * Hkv / 8) * ceil(B / kPfxWaves) blocks of
// kPfxWaves waves.  Block i -> XCD x = i % 8 (the hardware deals blocks to
// the eight XCDs in turn) and slot j = i / 8; (chunk, KV head) item
// 8 (j / nsg) + x, sequence group j % nsg.  The groups of one item are thus
// 8 blocks apart and run on the same XCD, whose L2 serves their reads of
// the item's pages after the first.
template <int MT, int GH, bool LUT>
__global__ void __launch_bounds__(64 * kPfxWaves) __attribute__((amdgpu_waves_per_eu(2)))
prefix_scan_kernel(DecArgs a) {
  const PoolView &pv = a.pv;
  const int nsg = (pv.batch + kPfxWaves - 1) / kPfxWaves;
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int item = 8 * (j / nsg) + x, sg = j % nsg;
  if (item >= a.n_prefix * pv.hkv) return;   // padding block (the whole block leaves)
  const int kv = item % pv.hkv, chunk = item / pv.hkv;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = pv.hq / pv.hkv;
  const int b = sg * kPfxWaves + wave;
  const bool active = b < pv.batch;
  const int pg0 = chunk * a.prefix_per_chunk;
  const int npg = max(0, min(a.prefix_pages, pg0 + a.prefix_per_chunk) - pg0);
  __shared__ PfxSmem<MT> sm;
  // block-table entries of the chunk (sequence 0's), and this wave's
  // sequence: its entries must be the same and its history must hold the
  // whole prefix
  const int32_t *bt0 = pv.block_table + pg0;
  for (int i = tid; i < npg; i += blockDim.x) sm.bt[i] = bt0[i];
  if (tid < kPfxWaves) sm.done[tid] = 0;
  if (tid == 0) sm.avail = 0;
  __syncthreads();
  if (active) {
    const int32_t *btb = pv.block_table + (size_t)b * pv.max_pages + pg0;
    bool diff = false;
    for (int i = lane; i < npg; i += 64) diff = diff || btb[i] != sm.bt[i];
    const bool any_diff = __builtin_amdgcn_ballot_w64(diff) != 0;
    const int n_hist = max(0, pv.seq_lens[b] - pv.sink - pv.recent);
    if (lane == 0 && pv.err) {
      if (any_diff) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
      if (chunk == 0 && n_hist < a.prefix_pages * kPageTokens) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    }
  }
  // this wave's query operands (a padding wave takes sequence 0's and
  // computes nothing)
  const int bq = active ? b : 0;
  const size_t bh = (size_t)bq * pv.hkv + kv;
  const float *pq = a.pq + bh * pq_floats<MT, GH>();
  const MetaSteps ms = meta_steps(a.rv, kv);
  QueryOps<MT> qo;
  load_query_ops<MT, GH, LUT>((const v4i *)pq, (const float (*)[4])(pq + MT * 2 * 64 * 4), G,
                              pv.sm_scale * kLog2e, ms, lane, qo);
  qo.lutk = LUT ? levels_of(a.rv, kv, false) : OSCAR_UNIFORM_LEVELS;
  qo.lutv = LUT ? levels_of(a.rv, kv, true) : OSCAR_UNIFORM_LEVELS;
  HistState<MT> st;
  hist_reset(st);
  v4i *wl = sm.wl[wave];
#pragma unroll
  for (int i = 0; i < MT * 2; ++i) wl[i * 64 + lane] = v4i{0, 0, 0, 0};
  // every load above has landed before the first copy is issued (wave 0
  // counts only its copies in vmcnt from here on)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const uint8_t *pbase = pv.pages + (size_t)kv * kPageBytes;
  const size_t pstride = (size_t)pv.hkv * kPageBytes;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)sm.pbuf[0];
  // page i -> buffer i % kPfxBufs; an entry out of range copies pool page 0
  // instead (in bounds, so that every page is one copy) and is skipped
  auto page_ok = [&](int i) {
    const int ph = sm.bt[i];
    return ph >= 0 && ph < pv.n_pages;
  };
  auto issue = [&](int i) {
    const int ph = page_ok(i) ? sm.bt[i] : 0;
    dma_page((uint64_t)(uintptr_t)(pbase + (size_t)ph * pstride), lds0 + (uint32_t)(i % kPfxBufs) * kPageBytes,
             16u * lane);
  };
  auto ld = [&](int *c) { return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
  // the fewest pages any wave has read
  auto min_done = [&] {
    int m = ld(&sm.done[0]);
#pragma unroll
    for (int w = 1; w < kPfxWaves; ++w) m = min(m, ld(&sm.done[w]));
    return m;
  };
  // The ring without workgroup barriers: wave 0 copies page j into buffer
  // j % kPfxBufs once every wave has read page j - kPfxBufs from it (every
  // done[w] > j - kPfxBufs), and raises avail to i + 1 once its copy of page
  // i has landed; a wave reads page i once avail > i and then sets its done
  // to i + 1.  Wave 0 blocks only for the page it needs next, i, whose
  // buffer waits for page i - kPfxBufs; every wave can read that page, as
  // it waits only for pages up to i - 1, all of which wave 0 has published.
  // So every wait ends, and the waves drift apart by up to the ring's depth
  // instead of meeting at every page.
  int issued = 0;
  bool bad = false;
  for (int i = 0; i < npg; ++i) {
    if (wave == 0) {
      // copy every page whose buffer is free, up to page i at least
      while (issued < npg && issued < i + kPfxBufs) {
        const int need = issued - kPfxBufs + 1;
        if (min_done() < need) {
          if (issued > i) break;   // not needed yet
          while (min_done() < need) __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        issue(issued);
        ++issued;
      }
      wait_pages3(issued - i - 1);   // copies issued after page i may stay outstanding
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_store(&sm.avail, i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      while (ld(&sm.avail) <= i) __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    PageRegs cur;
    load_page(cur, (const uint8_t *)sm.pbuf[i % kPfxBufs], n, q);
    wait_lds_reads();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_store(&sm.done[wave], i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const bool ok = page_ok(i);
    bad = bad || !ok;
    if (active && ok) int2_page<MT, true, LUT>(cur, kPageTokens, qo, st, wl);
  }
  if (bad && tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
  if (!active) return;
  // the wave's partial: value sums in metadata code units become o = sum w
  // (s8 b) code + sum w (z8 a - tau), per head
  float *dst = a.part + (bh * a.n_parts + a.n_splits + chunk) * G * kPartStride;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float l16 = row16_sum(st.lsum[mt]);
    const float z0 = row16_sum(st.z0[mt]), z1 = row16_sum(st.z1[mt]);
    const int hh = 4 * mt + q;
    if (hh < G) {
      const float zz0 = fmaf(z0, ms.va, -ms.vtau * l16), zz1 = fmaf(z1, ms.va, -ms.vtau * l16);
      float *d = dst + (size_t)hh * kPartStride;
      if (n == 0) {
        d[0] = st.mref[mt];
        d[1] = l16;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) d[kPartO + 16 * nt + n] = fmaf(st.facc[mt][nt], ms.vb, nt < 4 ? zz0 : zz1);
    }
  }
}


}  // namespace

namespace {
// scan workgroups the grid aims for: the caller's choice, else one per CU
int target_blocks(int blocks) { return blocks > 0 ? blocks : 256; }
int mt_of(int G) { return (G + 3) / 4; }
int gh_of(int G) { return 4 * mt_of(G); }
// variants 0 and 2: MFMA scan; 1: VALU scan
bool is_mfma(int variant) { return variant == 0; }
int nw_of(int G, int variant) { return !is_mfma(variant) ? 4 : (mt_of(G) == 1 ? 12 : 8); }
}  // namespace

DecodePlan make_decode_plan(int batch, int hkv, int hq, int max_pages, int sink, int recent, int variant,
                            int blocks, int prefix_pages) {
  DecodePlan p{};
  const int G = hq / hkv;
  const int MT = mt_of(G), GH = gh_of(G), NW = nw_of(G, variant);
  const int bh = batch * hkv;
  p.n_chunks = (sink + recent) / kTileTokens;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  // shared prefix: chunks of pages such that chunks x KV heads x sequence
  // groups is about the target grid, each chunk at most kPfxMaxChunk pages
  p.prefix_pages = prefix_pages;
  if (prefix_pages > 0) {
    const int nsg = (batch + kPfxWaves - 1) / kPfxWaves;
    int C = (target_blocks(blocks) + hkv * nsg - 1) / (hkv * nsg);
    C = C < 1 ? 1 : C;
    C = C > prefix_pages ? prefix_pages : C;
    C = C < (prefix_pages + kPfxMaxChunk - 1) / kPfxMaxChunk ? (prefix_pages + kPfxMaxChunk - 1) / kPfxMaxChunk : C;
    C = C > kMaxParts / 4 ? kMaxParts / 4 : C;
    p.prefix_per_chunk = (prefix_pages + C - 1) / C;
    p.n_prefix = (prefix_pages + p.prefix_per_chunk - 1) / p.prefix_per_chunk;   // no empty chunk
  }
  const int own_pages = max_pages - prefix_pages;   // pages the per-sequence scan covers at most
  int S = (target_blocks(blocks) + bh - 1) / bh;
  const int max_by_pages = own_pages > 0 ? (own_pages + NW - 1) / NW : 1;   // >= 1 page per wave
  S = S < 1 ? 1 : S;
  S = S > max_by_pages ? max_by_pages : S;
  S = S > kMaxSplits ? kMaxSplits : S;
  S = S > kMaxParts - p.n_chunks - p.n_prefix ? kMaxParts - p.n_chunks - p.n_prefix : S;
  p.n_splits = S;
  // one M-tile of heads on MFMA: one partial per split (BF16 tiles folded in)
  p.n_parts = (is_mfma(variant) && MT == 1) ? S + p.n_prefix : S + p.n_prefix + p.n_chunks;
  p.pages_per_split = own_pages > 0 ? (own_pages + S - 1) / S : 1;
  size_t off = 0;
  p.off_counters = off;
  off = al(off + (size_t)bh * sizeof(int));
  p.off_qconst = off;
  off = al(off + (is_mfma(variant) ? 0 : (size_t)bh * GH * 4 * sizeof(float)));
  p.off_qrot = off;
  off = al(off + (is_mfma(variant) ? 0 : (size_t)bh * GH * kD * sizeof(float)));
  p.off_part = off;
  off = al(off + (size_t)bh * p.n_parts * G * kPartStride * sizeof(float));
  p.off_pq = off;
  off = al(off + (p.n_prefix > 0 ? (size_t)bh * ((size_t)MT * 2 * 64 * 4 + (size_t)GH * 4) * sizeof(float) : 0));
  p.total = off;
  return p;
}

hipError_t launch_decode(const PoolView &pv, const RotView &rv, const uint16_t *q, float *out,
                         uint8_t *ws, int *counters, const DecodePlan &plan, int variant, hipStream_t s) {
  const int G = pv.hq / pv.hkv;
  const int BH = pv.batch * pv.hkv;
  DecArgs a{pv, rv, q, out, counters, (float *)(ws + plan.off_qconst),
            (float *)(ws + plan.off_qrot), (float *)(ws + plan.off_part),
            plan.n_splits, plan.n_chunks, plan.pages_per_split, plan.n_parts,
            plan.prefix_pages, plan.n_prefix, plan.prefix_per_chunk, (float *)(ws + plan.off_pq)};
  const bool mfma = is_mfma(variant);
  // the codebook scans when either tensor has a codebook (the other then
  // takes the uniform levels through the same lookup)
  const bool lut = rv.lev_K != nullptr || rv.lev_V != nullptr;
  hipError_t e;
  const dim3 sgrid(BH * plan.n_splits);
  // shared prefix (several M-tiles of heads, MFMA): the query operands, then
  // the prefix pages, both before the per-sequence scan that merges them
  const int nsg = (pv.batch + kPfxWaves - 1) / kPfxWaves;
  const dim3 pgrid(8 * ((plan.n_prefix * pv.hkv + 7) / 8) * nsg);
#define OSCAR_PREFIX(MT, GH, LUT)                                                                    \
  do {                                                                                               \
    hipLaunchKernelGGL((prefix_prep_kernel<MT, GH>), dim3(BH), dim3(256), 0, s, a);                  \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                             \
    hipLaunchKernelGGL((prefix_scan_kernel<MT, GH, LUT>), pgrid, dim3(64 * kPfxWaves), 0, s, a);     \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                             \
  } while (0)
#define OSCAR_LAUNCH(MT, GH)                                                                         \
  do {                                                                                               \
    if (mfma && plan.n_prefix > 0) {                                                                 \
      if (lut) OSCAR_PREFIX(MT, GH, true);                                                           \
      else OSCAR_PREFIX(MT, GH, false);                                                              \
    }                                                                                                \
    if (!mfma) {                                                                                     \
      hipLaunchKernelGGL((decode_pre_kernel<MT, GH>), dim3(BH), dim3(256), 0, s, a);                 \
      if ((e = hipGetLastError()) != hipSuccess) return e;                                           \
      hipLaunchKernelGGL((decode_scan_kernel<MT, GH, false, true>), sgrid,                           \
                         dim3(64 * scan_waves<MT, false>()), 0, s, a);                               \
    } else if (lut) {                                                                                \
      hipLaunchKernelGGL((decode_scan_kernel<MT, GH, true, true>), sgrid,                            \
                         dim3(64 * scan_waves<MT, true>()), 0, s, a);                                \
    } else {                                                                                         \
      hipLaunchKernelGGL((decode_scan_kernel<MT, GH, true, false>), sgrid,                           \
                         dim3(64 * scan_waves<MT, true>()), 0, s, a);                                \
    }                                                                                                \
  } while (0)
  if (G <= 4) OSCAR_LAUNCH(1, 4);
  else if (G <= 8) OSCAR_LAUNCH(2, 8);
  else if (G <= 12) OSCAR_LAUNCH(3, 12);
  else OSCAR_LAUNCH(4, 16);
#undef OSCAR_LAUNCH
#undef OSCAR_PREFIX
  return hipGetLastError();
}

// ===========================================================================
// Decode without a caller-provided workspace
// ===========================================================================
namespace {
// The buffer of oscar_decode_attention_noalloc, one per GPU for the life of
// the process.  [0, kNoAllocCounterBytes) holds the completion counters
// only: zero when the code object is loaded, cleared once more by the first
// call on each device, and returned to zero by every call; the rest holds
// the query operands and partials of the current call.
constexpr size_t kNoAllocCounterBytes = 64 * 1024;
static_assert(OSCAR_NOALLOC_SCRATCH_BYTES % 256 == 0 && OSCAR_NOALLOC_SCRATCH_BYTES > kNoAllocCounterBytes, "");
__device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch[kMaxDevices] = {};   // device address of `scratch` per device, once known

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t *p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}
}  // namespace

size_t noalloc_counter_bytes() { return kNoAllocCounterBytes; }

hipError_t noalloc_scratch(hipStream_t s, uint8_t **base) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    // the array's name is a host-side stand-in: only this address may be
    // passed to kernels or copies
    void *ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, s, (uint32_t *)ptr,
                       (int)(kNoAllocCounterBytes / 4));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    g_scratch[dev] = (uint8_t *)ptr;
  }
  *base = g_scratch[dev];
  return hipSuccess;
}

}  // namespace oscar
