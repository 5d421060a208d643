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
// Arithmetic order (fixed so that codes and metadata are reproducible bit
// for bit by any implementation that follows it):
//   S1 y_j = sum_k x_k U[k][j], float64, k ascending (bf16 x float32
//      products are exact in float64, so fma == multiply-then-add);
//   S2 radix-2 butterfly, stages h = 1..64, (a, b) -> (a + b, a - b), float64;
//   S3 multiply by the float64 nearest to 1/sqrt(128);
//   S4 output channel p takes butterfly output bitrev(p);
//   S5 round to float32; S6 clamp to [-tau, tau];
//   S7 per 64-channel group: s = (max - min) / 3 (float32 IEEE); with
//      a = (tau + tau) / 255 and b = (tau + tau) / 765: z8 = clamp(rint((min +
//      tau) / a), 0, 255), s8 = clamp(rint(s / b), 0, 255) (0 if tau is 0);
//      zero = z8 a - tau, scale = s8 b; code = the nearest codebook level
//      of u = (x - zero) / scale (level_code: on the uniform grid
//      clamp(rint(u), 0, 3)), all codes 0 if scale == 0.  Everything float32 (16
//      metadata bits per group: the density of the pages' 2.28 bits per
//      element at 128K; the encoding relative to tau is this library's);
//   S8 pack four codes per byte (page layout in oscar.h).
#include <type_traits>

#include "oscar_internal.h"
#include "oscar_wave.h"

#pragma clang fp contract(off)

namespace oscar {
namespace {

constexpr int kThreads = 128;     // single-token append: one thread per channel
constexpr int kPageThreads = 256; // bulk demotion: four waves of 16 page slots
constexpr double kInvSqrtD = 0x1.6a09e667f3bcdp-4;  // nearest double to 1/sqrt(128)
// Row stride (floats) of the bulk kernel's token rows in LDS: the matrix
// core's A operand reads 16 rows x 4 columns at once, and a stride of 4 mod
// 64 floats puts those 64 reads in 64 different banks.
constexpr int kXRow = 132;
typedef double v4d __attribute__((ext_vector_type(4)));

struct AppendArgs {
  PoolView pv;
  RotView rv;
  const uint16_t *k_new, *v_new;
  int n_new;
};

// S6..S8 for output channel p of one token (this lane; the wave holds the 64
// channels of one group): clamp, group metadata, code.  Returns the code;
// meta receives the group's 16-bit metadata s8 | z8 << 8 (same on every
// lane).  Zero and scale are 8-bit codes on grids over [-tau, tau] and
// [0, 2 tau / 3] (steps a = 2 tau / 255, b = 2 tau / 765): z8 = rint((min +
// tau) / a), s8 = rint(s / b), clamped to [0, 255] (0 when tau is 0); codes
// use the decoded zero z8 a - tau and scale s8 b, and the head's codebook
// thresholds (level_code; on the uniform grid rint(u) clamped to [0, 3]).
__device__ __forceinline__ uint32_t quantize_group(float v, float tau, const CodeThresholds &th, uint32_t &meta) {
  v = fminf(fmaxf(v, -tau), tau);
  const float mx = wave_max(v), mn = wave_min(v);
  const float s = __fdiv_rn(mx - mn, 3.0f);
  const float a = meta_zero_step(tau), b = meta_scale_step(tau);
  uint32_t z8 = 0, s8 = 0;
  if (a > 0.0f) z8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(mn + tau, a)), 0.0f), 255.0f);
  if (b > 0.0f) s8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(s, b)), 0.0f), 255.0f);
  const float zf = (float)z8 * a - tau;
  const float sf = (float)s8 * b;
  const uint32_t code = sf != 0.0f ? level_code(__fdiv_rn(v - zf, sf), th) : 0u;
  meta = s8 | (z8 << 8);
  return code;
}

// As quantize_group for output channel p; lane p % 64 == 0 stores the
// group's metadata to meta[p / 64] (the 4-byte entry of the token).
__device__ __forceinline__ uint32_t quantize_code(float v, float tau, const CodeThresholds &th, int p,
                                                  uint16_t *meta) {
  uint32_t m;
  const uint32_t code = quantize_group(v, tau, th, m);
  if ((p & 63) == 0) meta[p >> 6] = (uint16_t)m;
  return code;
}

// Bulk demotion, one 64-token history page of one (KV head, K|V) per
// workgroup.  grid: (pages, Hkv * 2, batch); block: 256 threads.  Wave w owns
// page slots 16 w .. 16 w + 15 (S1..S5 on the fp64 matrix core and in its
// lanes) and lane l output channels l and l + 64 of each (S6..S8).
// Demotes every position x with max(S0, p0 - W) <= x < p0 + n_new - W.
__global__ void __launch_bounds__(kPageThreads) __attribute__((amdgpu_waves_per_eu(2)))
append_demote_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  const int b = blockIdx.z;
  const int h = blockIdx.y >> 1;
  const int is_v = blockIdx.y & 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p0 = pv.seq_lens[b];
  if (p0 < 0) return;                                       // flagged by the store kernel
  const int L = p0 + a.n_new;
  const int xa = max(pv.sink, p0 - pv.recent);
  const int xb = L - pv.recent;
  if (xb <= xa) return;
  const int ha = xa - pv.sink, hb = xb - pv.sink;           // history index range
  const int c0 = (ha / kPageTokens + (int)blockIdx.x) * kPageTokens;   // first index of this page
  const int t0 = max(c0, ha), t1 = min(c0 + kPageTokens, hb);
  if (t1 <= t0) return;
  const int page_idx = c0 / kPageTokens;
  if (page_idx >= pv.max_pages) {
    if (tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    return;
  }
  const int phys = pv.block_table[(size_t)b * pv.max_pages + page_idx];
  if (phys < 0 || phys >= pv.n_pages) {
    if (tid == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
    return;
  }
  __shared__ __align__(16) float xs[kPageTokens][kXRow];    // bf16 sources as float32 (exact), token-major
  __shared__ __align__(16) float4 stat_s[kPageThreads / 64][16];   // per wave and slot: zero0, scale0, zero1, scale1
  __shared__ uint32_t smeta_s[kPageThreads / 64][16];     // per wave and slot: s8_0 | z8_0 << 8 | s8_1 << 16 | z8_1 << 24
  __shared__ __align__(16) uint8_t vst[kD][16];           // V code bytes of the page, channel-major

  // Gather: each wave its own 16 slots (zeros outside [t0, t1)); lane l
  // reads channels 2 l and 2 l + 1 of the token row.  The 16 loads are
  // issued together: a slot outside the range reads the row of t0 (valid)
  // and drops it.
  const uint16_t *ring = (is_v ? pv.recent_v : pv.recent_k) + ((size_t)b * pv.hkv + h) * pv.recent * kD;
  const uint16_t *fresh = (is_v ? a.v_new : a.k_new) + ((size_t)b * a.n_new * pv.hkv + h) * kD;
  const size_t fresh_stride = (size_t)pv.hkv * kD;   // between consecutive new tokens
  auto row_of = [&](int x, int rp) -> const uint16_t * {
    return x < p0 ? ring + (size_t)rp * kD : fresh + (size_t)(x - p0) * fresh_stride;
  };
  const int xw = c0 + 16 * w + pv.sink;   // position of the wave's first slot
  const uint16_t *row_t0 = row_of(t0 + pv.sink, (t0 + pv.sink) % pv.recent);
  uint32_t bits[16];
  {
    int rp = xw % pv.recent;   // ring slot of position xw + i
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hx = xw + i - pv.sink;
      const uint16_t *row = (hx >= t0 && hx < t1) ? row_of(xw + i, rp) : row_t0;
      bits[i] = ((const uint32_t *)row)[lane];
      rp = rp + 1 == pv.recent ? 0 : rp + 1;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hx = xw + i - pv.sink;
    float2 f = {0.0f, 0.0f};
    if (hx >= t0 && hx < t1) {
      f.x = bf16_to_f32((uint16_t)(bits[i] & 0xFFFFu));
      f.y = bf16_to_f32((uint16_t)(bits[i] >> 16));
    }
    *(float2 *)&xs[16 * w + i][2 * lane] = f;
  }
  __syncthreads();

  // S1: y_n = sum_k x_k U[k][n], float64, k ascending, on the fp64 matrix
  // core: each wave the 16 x 128 block Y = X U of its slots as eight 16 x 16
  // tiles, 32 steps of v_mfma_f64_16x16x4f64 over k.  One step adds the
  // products of k = 4 ks .. 4 ks + 3 in that order, rounding after each, so
  // the chain equals one fma chain over k ascending bit for bit (the
  // products of bf16 and float32 values are exact in float64; checked
  // against a plain fma chain on the device over wide exponent ranges).
  // Tile nt, column j holds output n = 8 j + nt: the eight B values of a
  // lane are adjacent floats of one U row (two 16-byte loads per step).
  // Operand lanes: A (16 x 4) lane l = X[slot l % 16][k = l / 16]; B (4 x 16)
  // lane l = U[k = l / 16][column l % 16]; D lane l, register r = slot
  // l / 16 + 4 r, column l % 16.
  const float *U = (is_v ? a.rv.U_V : a.rv.U_K) + (size_t)h * kD * kD;
  const int mi = lane & 15, kq = lane >> 4;
  const float *urow = U + (size_t)kq * kD + 8 * mi;   // row 4 ks + kq, columns 8 mi .. 8 mi + 7
  v4d acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = v4d{0.0, 0.0, 0.0, 0.0};
  float4 u0 = *(const float4 *)urow, u1 = *(const float4 *)(urow + 4);
#pragma unroll 4
  for (int ks = 0; ks < kD / 4; ++ks) {
    const int kn = ks + 1 < kD / 4 ? ks + 1 : ks;   // the last step reloads its own row (unused)
    const float4 n0 = *(const float4 *)(urow + (size_t)4 * kn * kD);
    const float4 n1 = *(const float4 *)(urow + (size_t)4 * kn * kD + 4);
    const double av = (double)xs[16 * w + mi][4 * ks + kq];
    const double bv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv[nt], acc[nt], 0, 0, 0);
    u0 = n0;
    u1 = n1;
  }

  // S2: butterfly stages h = 1, 2, 4 (element bits 0..2: the tiles of the
  // lane) and h = 8 .. 64 (bits 3..6: lanes j ^ (h / 8) of a 16-lane row),
  // in ascending order of h: pairs (a, b) at (e, e + h) -> (a + b, a - b).
#pragma unroll
  for (int hs = 1; hs <= 4; hs <<= 1) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      if (nt & hs) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double x0 = acc[nt][r], x1 = acc[nt + hs][r];
        acc[nt][r] = x0 + x1;
        acc[nt + hs][r] = x0 - x1;
      }
    }
  }
  auto stage = [&](auto M) {
    constexpr int m = decltype(M)::value;   // element bit 3 + log2(m) <-> lane bit log2(m)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double o = lane_xor_d<m>(acc[nt][r]);
        acc[nt][r] = (mi & m) ? o - acc[nt][r] : acc[nt][r] + o;
      }
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});

  // S3, S5: the float32 values of the wave's 16 slots, in butterfly order,
  // staged in its own rows of xs (free after S1).  Row stride 132 floats.
  const float tau = (is_v ? a.rv.tau_V : a.rv.tau_K)[h];
  const CodeThresholds th = code_thresholds(levels_of(a.rv, h, is_v));
  constexpr int kRow = 132;
  float *ys = &xs[16 * w][0];
  float4 *stat = stat_s[w];
  uint32_t *smeta = smeta_s[w];
  static_assert(kRow == kXRow, "staging reuses the wave's rows");
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float *row = ys + (kq + 4 * r) * kRow + 8 * mi;   // elements 8 mi .. 8 mi + 7 of slot kq + 4 r
    *(float4 *)row = make_float4((float)(acc[0][r] * kInvSqrtD), (float)(acc[1][r] * kInvSqrtD),
                                 (float)(acc[2][r] * kInvSqrtD), (float)(acc[3][r] * kInvSqrtD));
    *(float4 *)(row + 4) = make_float4((float)(acc[4][r] * kInvSqrtD), (float)(acc[5][r] * kInvSqrtD),
                                       (float)(acc[6][r] * kInvSqrtD), (float)(acc[7][r] * kInvSqrtD));
  }
  wave_lds_sync();
  // S6, S7 per slot and group, lane i < 16 taking slot 16 w + i.  Output
  // channel p takes element bitrev(p), so group g (channels 64 g .. 64 g + 63)
  // is the set of elements with e % 2 == g; min and max commute with the
  // order and with the clamp to [-tau, tau] (monotone), which is applied to
  // them.  Then the group metadata as in quantize_group.
  if (lane < 16) {
    const float4 *row = (const float4 *)(ys + lane * kRow);
    float mx0 = -INFINITY, mn0 = INFINITY, mx1 = -INFINITY, mn1 = INFINITY;
#pragma unroll 8
    for (int j = 0; j < kD / 4; ++j) {
      const float4 v = row[j];
      mx0 = fmaxf(mx0, fmaxf(v.x, v.z));
      mn0 = fminf(mn0, fminf(v.x, v.z));
      mx1 = fmaxf(mx1, fmaxf(v.y, v.w));
      mn1 = fminf(mn1, fminf(v.y, v.w));
    }
    float zf[2], sf[2];
    uint32_t meta = 0;
    const float mx[2] = {fminf(fmaxf(mx0, -tau), tau), fminf(fmaxf(mx1, -tau), tau)};
    const float mn[2] = {fminf(fmaxf(mn0, -tau), tau), fminf(fmaxf(mn1, -tau), tau)};
    const float za = meta_zero_step(tau), sb = meta_scale_step(tau);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float sg = __fdiv_rn(mx[g] - mn[g], 3.0f);
      uint32_t z8 = 0, s8 = 0;
      if (za > 0.0f) z8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(mn[g] + tau, za)), 0.0f), 255.0f);
      if (sb > 0.0f) s8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(sg, sb)), 0.0f), 255.0f);
      zf[g] = (float)z8 * za - tau;
      sf[g] = (float)s8 * sb;
      meta |= (s8 | (z8 << 8)) << (16 * g);
    }
    stat[lane] = make_float4(zf[0], sf[0], zf[1], sf[1]);
    smeta[lane] = meta;
  }
  wave_lds_sync();

  // S7 codes and S8 packing: lane l takes output channels l and l + 64
  const int e0 = bitrev7(lane), e1 = bitrev7(lane + 64);
  uint8_t *page = pv.pages + ((size_t)phys * pv.hkv + h) * kPageBytes;
  uint32_t vb[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};   // V: bytes 4 m + w of channels l, l + 64
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int slot = 16 * w + i;
    const bool valid = c0 + slot >= t0 && c0 + slot < t1;   // wave-uniform
    if (!valid) continue;
    const float4 st = stat[i];
    const float v0 = fminf(fmaxf(ys[i * kRow + e0], -tau), tau);
    const float v1 = fminf(fmaxf(ys[i * kRow + e1], -tau), tau);
    uint32_t code0 = 0, code1 = 0;
    if (st.y != 0.0f) code0 = level_code(__fdiv_rn(v0 - st.x, st.y), th);
    if (st.w != 0.0f) code1 = level_code(__fdiv_rn(v1 - st.z, st.w), th);
    if (lane == 0) *(uint32_t *)(page + (is_v ? kVMeta : kKMeta) + meta_entry(slot) * 4) = smeta[i];
    if (!is_v) {
      // K row: dword q holds channels 16 q .. 16 q + 15, two bits each
      uint32_t k0 = code0 << (2 * (lane & 15)), k1 = code1 << (2 * (lane & 15));
      k0 |= (uint32_t)lane_xor_i<1>((int)k0);
      k1 |= (uint32_t)lane_xor_i<1>((int)k1);
      k0 |= (uint32_t)lane_xor_i<2>((int)k0);
      k1 |= (uint32_t)lane_xor_i<2>((int)k1);
      k0 |= (uint32_t)lane_xor_i<4>((int)k0);
      k1 |= (uint32_t)lane_xor_i<4>((int)k1);
      k0 |= (uint32_t)lane_xor_i<8>((int)k0);
      k1 |= (uint32_t)lane_xor_i<8>((int)k1);
      if ((lane & 15) == 0) {
        uint32_t *row = (uint32_t *)(page + kKCodes + slot * 32);
        row[lane >> 4] = k0;
        row[4 + (lane >> 4)] = k1;
      }
    } else {
      // V: slot 16 w + i sits in byte 4 (i / 4) + w of each channel row, bits 2 (i % 4)
      vb[0][i >> 2] |= code0 << (2 * (i & 3));
      vb[1][i >> 2] |= code1 << (2 * (i & 3));
    }
  }
  if (!is_v) return;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    vst[lane][4 * m + w] = (uint8_t)vb[0][m];
    vst[lane + 64][4 * m + w] = (uint8_t)vb[1][m];
  }
  __syncthreads();
  if (tid < kD) {
    uint4 *dst = (uint4 *)(page + kVCodes + tid * 16);
    uint4 val = *(const uint4 *)vst[tid];
    if (t0 != c0 || t1 != c0 + kPageTokens) {
      // partial page: keep the bits of slots outside [t0 - c0, t1 - c0)
      uint32_t mk[4] = {0, 0, 0, 0};
      for (int s = t0 - c0; s < t1 - c0; ++s) {
        const int byte = 4 * ((s >> 2) & 3) + (s >> 4);
        mk[byte >> 2] |= 3u << (8 * (byte & 3) + 2 * (s & 3));
      }
      const uint4 old = *dst;
      val.x = (old.x & ~mk[0]) | (val.x & mk[0]);
      val.y = (old.y & ~mk[1]) | (val.y & mk[1]);
      val.z = (old.z & ~mk[2]) | (val.z & mk[2]);
      val.w = (old.w & ~mk[3]) | (val.w & mk[3]);
    }
    *dst = val;
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
  // Loads that do not depend on the sequence length are issued together
  // with it: the new token, the clip threshold and (S1) column j of U, all
  // 128 loads at once.  The length then decides the ring slot and the page.
  const uint16_t nb = (is_v ? a.v_new : a.k_new)[((size_t)b * pv.hkv + h) * kD + j];
  const float tau = (is_v ? a.rv.tau_V : a.rv.tau_K)[h];
  const CodeThresholds th = code_thresholds(levels_of(a.rv, h, is_v));
  const float *U = (is_v ? a.rv.U_V : a.rv.U_K) + (size_t)h * kD * kD + j;
  float u[kD];
#pragma unroll
  for (int k = 0; k < kD; ++k) u[k] = U[(size_t)k * kD];
  const int p0 = pv.seq_lens[b];
  __shared__ double xs[kD];
  __shared__ double ys[kD];
  if (p0 >= 0) {
    // the ring slot's old token and the page's block-table entry are
    // loaded together; the new token goes into the ring slot at the end
    const bool in_ring = p0 >= pv.sink;
    uint16_t *el = (is_v ? pv.recent_v : pv.recent_k) + (((size_t)b * pv.hkv + h) * pv.recent + p0 % pv.recent) * kD + j;
    const bool demote = in_ring && p0 - pv.recent >= pv.sink;   // the slot's token leaves the window
    const int page_idx = demote ? (p0 - pv.recent - pv.sink) / kPageTokens : 0;
    const bool in_table = demote && page_idx < pv.max_pages;
    int phys = in_table ? pv.block_table[(size_t)b * pv.max_pages + page_idx] : -1;
    const uint16_t old_raw = *el;   // in bounds for any p0: no branch, no early wait
    const uint16_t old = demote ? old_raw : 0;
    if (!in_ring) {
      const int ss = pv.sink_slot[b];
      if (ss >= 0 && ss < pv.n_sink_slots)
        (is_v ? pv.sink_v : pv.sink_k)[(((size_t)ss * pv.hkv + h) * pv.sink + p0) * kD + j] = nb;
      else if (blockIdx.x == 0 && j == 0 && pv.err)
        atomicOr(pv.err, OSCAR_DEVERR_SINKSLOT);
    }
    if (demote && !in_table && j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    if (in_table && (phys < 0 || phys >= pv.n_pages)) {
      if (j == 0 && pv.err) atomicOr(pv.err, OSCAR_DEVERR_PAGE);
      phys = -1;
    }
    if (phys >= 0) {   // block-uniform
      const int slot = (p0 - pv.recent - pv.sink) % kPageTokens;
      uint8_t *page = pv.pages + ((size_t)phys * pv.hkv + h) * kPageBytes;
      // V: the code byte this thread rewrites holds three other slots'
      // codes; its load goes out now, ahead of the projection
      uint8_t *vdst = page + kVCodes + j * 16 + vcode_byte(slot);
      const uint8_t vold = *vdst;   // in the page for K and V blocks alike: no branch
      xs[j] = (double)bf16_to_f32(old);
      __syncthreads();
      double y = 0.0;
#pragma unroll
      for (int k = 0; k < kD; ++k) y = fma(xs[k], (double)u[k], y);
      // S2: butterfly; stages 1..32 inside the wave, stage 64 through LDS
      auto stage1 = [&](auto M) {
        constexpr int hs = decltype(M)::value;
        const double o = lane_xor_d<hs>(y);
        y = (j & hs) ? o - y : y + o;
      };
      stage1(std::integral_constant<int, 1>{});
      stage1(std::integral_constant<int, 2>{});
      stage1(std::integral_constant<int, 4>{});
      stage1(std::integral_constant<int, 8>{});
      stage1(std::integral_constant<int, 16>{});
      stage1(std::integral_constant<int, 32>{});
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
      const float v = (float)(ys[bitrev7(p)] * kInvSqrtD);
      const uint32_t code =
          quantize_code(v, tau, th, p, (uint16_t *)(page + (is_v ? kVMeta : kKMeta) + meta_entry(slot) * 4));
      if (!is_v) {
        uint32_t c = code << (2 * (p & 3));
        c |= (uint32_t)lane_xor_i<1>((int)c);
        c |= (uint32_t)lane_xor_i<2>((int)c);
        if ((p & 3) == 0) page[kKCodes + slot * 32 + (p >> 2)] = (uint8_t)c;
      } else {
        // one 2-bit field of a byte shared with three other slots
        const uint32_t sh = 2 * (slot & 3);
        *vdst = (uint8_t)((vold & ~(3u << sh)) | (code << sh));
      }
    }
    if (in_ring) *el = nb;
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

// grid: (blocks, batch); block: 256.  Stores the new tokens that stay BF16
// (sink, or the final recent window): rows of 256 B, one per (token, KV
// head, K|V), sink tokens first; workgroup x takes rows [16 x, 16 x + 16).
// Runs after the demote kernel on the same stream, so every ring slot has
// been read before it is reused.  seq_lens is advanced by the commit kernel.
constexpr int kStoreRows = 16;
__global__ void __launch_bounds__(256) append_store_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  const int b = blockIdx.y;
  const int p0 = pv.seq_lens[b];
  if (p0 < 0) return;                                       // flagged by the commit kernel
  const int L = p0 + a.n_new;
  const int sink_slot = pv.sink_slot[b];
  const bool sink_ok = sink_slot >= 0 && sink_slot < pv.n_sink_slots;
  if (!sink_ok && p0 < pv.sink && blockIdx.x == 0 && threadIdx.x == 0 && pv.err)
    atomicOr(pv.err, OSCAR_DEVERR_SINKSLOT);
  const int n_sink_new = max(0, min(a.n_new, pv.sink - p0));
  const int i_ring0 = max(n_sink_new, L - pv.recent - p0);
  const int n_sink_st = sink_ok ? n_sink_new : 0;           // sink tokens stored
  const int n_tok = n_sink_st + (a.n_new - i_ring0);
  const int rows = n_tok * pv.hkv * 2;
  const int words = kD / 4;                                 // 8-byte words per row
  const int w = threadIdx.x & (words - 1);
  const int r1 = min(rows, ((int)blockIdx.x + 1) * kStoreRows);
  for (int r = (int)blockIdx.x * kStoreRows + (int)(threadIdx.x / words); r < r1; r += 256 / words) {
    const int is_v = r & 1, h = (r >> 1) % pv.hkv, ti = (r >> 1) / pv.hkv;
    const bool to_sink = ti < n_sink_st;
    const int i = to_sink ? ti : i_ring0 + (ti - n_sink_st);   // index among the new tokens
    const int pos = p0 + i;
    const uint64_t *src = (const uint64_t *)(is_v ? a.v_new : a.k_new);
    const uint64_t v = src[(((size_t)b * a.n_new + i) * pv.hkv + h) * words + w];
    if (to_sink) {
      uint64_t *sink = (uint64_t *)(is_v ? pv.sink_v : pv.sink_k);
      sink[(((size_t)sink_slot * pv.hkv + h) * pv.sink + pos) * words + w] = v;
    } else {
      uint64_t *ring = (uint64_t *)(is_v ? pv.recent_v : pv.recent_k);
      ring[(((size_t)b * pv.hkv + h) * pv.recent + (pos % pv.recent)) * words + w] = v;
    }
  }
}

// grid: 1; block: 256.  Advances seq_lens by n_new (after every kernel of
// the append has read the old length); a negative length is flagged.
__global__ void __launch_bounds__(256) append_commit_kernel(AppendArgs a) {
  const PoolView &pv = a.pv;
  for (int b = threadIdx.x; b < pv.batch; b += blockDim.x) {
    const int p0 = pv.seq_lens[b];
    if (p0 < 0) {
      if (pv.err) atomicOr(pv.err, OSCAR_DEVERR_LENGTH);
    } else {
      pv.seq_lens[b] = p0 + a.n_new;
    }
  }
}

}  // namespace

hipError_t launch_append(const PoolView &pv, const RotView &rv, const uint16_t *k_new,
                         const uint16_t *v_new, int n_new, hipStream_t s) {
  AppendArgs a{pv, rv, k_new, v_new, n_new};
  if (n_new == 1 && pv.app_cnt) {
    hipLaunchKernelGGL(append_one_kernel, dim3(pv.hkv * 2, pv.batch), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  // the demoted range is at most n_new history slots: it spans at most
  // n_new / 64 + 2 pages
  const int pages = n_new / kPageTokens + 2;
  hipLaunchKernelGGL(append_demote_kernel, dim3(pages, pv.hkv * 2, pv.batch), dim3(kPageThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // BF16 rows stored: at most min(n_new, sink + recent) tokens x Hkv x 2
  const long long store_rows = (long long)min(n_new, pv.sink + pv.recent) * pv.hkv * 2;
  const int store_blocks = (int)((store_rows + kStoreRows - 1) / kStoreRows);
  if (store_blocks > 0) {
    hipLaunchKernelGGL(append_store_kernel, dim3(store_blocks, pv.batch), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(append_commit_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
