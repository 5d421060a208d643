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
// core's B operand reads 4 columns x 16 rows at once, and a stride of 4 mod
// 64 floats puts those 64 reads in 64 different banks.
constexpr int kXRow = 132;
typedef double v4d __attribute__((ext_vector_type(4)));

// Exchanges x of the upper lanes with y of the lower lanes, where lower and
// upper are the two halves of each 32-lane group (M == 1: lane bit 4 clear /
// set) or of the wave (M == 2: lane bit 5): afterwards a lower lane holds
// (own x, partner's x) and an upper lane (partner's y, own y).
template <int M>
__device__ __forceinline__ void half_swap(uint32_t &x, uint32_t &y) {
  static_assert(M == 1 || M == 2, "half_swap: M");
  if constexpr (M == 1) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  }
}
template <int M>
__device__ __forceinline__ void half_swap(double &x, double &y) {
  const uint64_t bx = __builtin_bit_cast(uint64_t, x), by = __builtin_bit_cast(uint64_t, y);
  uint32_t xl = (uint32_t)bx, xh = (uint32_t)(bx >> 32), yl = (uint32_t)by, yh = (uint32_t)(by >> 32);
  half_swap<M>(xl, yl);
  half_swap<M>(xh, yh);
  x = __builtin_bit_cast(double, ((uint64_t)xh << 32) | xl);
  y = __builtin_bit_cast(double, ((uint64_t)yh << 32) | yl);
}
template <int M>
__device__ __forceinline__ void half_swap(float &x, float &y) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = __builtin_bit_cast(uint32_t, y);
  half_swap<M>(a, b);
  x = __builtin_bit_cast(float, a);
  y = __builtin_bit_cast(float, b);
}

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
// page slots 16 w .. 16 w + 15; from S2 on, the 128 elements of slot
// 16 w + (l % 16) sit in the four lanes l % 16 + 16 j, 32 in each.
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
  // core: each wave the 128 x 16 block Y^T = U^T X^T of its slots as eight
  // 16 x 16 tiles, 32 steps of v_mfma_f64_16x16x4f64 over k.  One step adds
  // the products of k = 4 ks .. 4 ks + 3 in that order, rounding after each,
  // so the chain equals one fma chain over k ascending bit for bit (the
  // products of bf16 and float32 values are exact in float64; checked
  // against a plain fma chain on the device over wide exponent ranges).
  // Tile nt, row i holds output n = 8 i + nt: the eight A values of a lane
  // are adjacent floats of one U row (two 16-byte loads per step).
  // Operand lanes: A (16 x 4) lane l = U[k = l / 16][n = 8 (l % 16) + nt];
  // B (4 x 16) lane l = X[slot l % 16][k = l / 16]; D lane l, register r =
  // row l / 16 + 4 r, slot l % 16.  So lane (mi = l % 16, kq = l / 16) ends
  // with n = 8 (kq + 4 r) + nt of slot mi in acc[nt][r]: n bits 0..2 = nt,
  // bits 3, 4 = lane bits 4, 5, bits 5, 6 = r.
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
    const double xv = (double)xs[16 * w + mi][4 * ks + kq];
    const double uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(uv[nt], xv, acc[nt], 0, 0, 0);
    u0 = n0;
    u1 = n1;
  }

  // S2: butterfly stages in ascending order of h, pairs (a, b) at (e, e + h)
  // -> (a + b, a - b).  h = 1, 2, 4: registers acc[nt] and acc[nt + h].
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
  // h = 8, 16 (element bits 3, 4: lane bits 4, 5).  The pair of registers
  // (acc[nt], acc[nt + m]) with nt & m == 0, m = 1 for h = 8 and 2 for h = 16,
  // holds elements that differ in bit 0 (resp. 1), whose stages are done.
  // half_swap gives every lane one (a, b) pair: the lower lane that of the
  // element with that bit clear, the upper lane the other; the sum goes to
  // acc[nt], the difference to acc[nt + m].  From then on register bit m of
  // nt stands for element bit 3 (resp. 4), and the lane bit for element bit 0
  // (resp. 1).
  auto cross = [&](auto M) {
    constexpr int m = decltype(M)::value;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      if (nt & m) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        double x0 = acc[nt][r], x1 = acc[nt + m][r];
        half_swap<m>(x0, x1);
        acc[nt][r] = x0 + x1;
        acc[nt + m][r] = x0 - x1;
      }
    }
  };
  cross(std::integral_constant<int, 1>{});
  cross(std::integral_constant<int, 2>{});
  // h = 32, 64 (element bits 5, 6): registers r and r + h / 32.
#pragma unroll
  for (int hr = 1; hr <= 2; hr <<= 1) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r & hr) continue;
        const double x0 = acc[nt][r], x1 = acc[nt][r + hr];
        acc[nt][r] = x0 + x1;
        acc[nt][r + hr] = x0 - x1;
      }
    }
  }
  // Now lane (mi, L4 = bit 4, L5 = bit 5) holds in acc[nt][r] element
  // n = L4 + 2 L5 + 4 nt2 + 8 nt0 + 16 nt1 + 32 r0 + 64 r1 of slot 16 w + mi
  // (ntj, rj: bit j of nt, r).  Output channel p takes element bitrev7(p),
  // so p = 64 L4 + 32 L5 + 16 nt2 + 8 nt0 + 4 nt1 + 2 r0 + r1: the lane's
  // 32 channels are 32 (2 L4 + L5) .. + 31, all in group g = L4.

  // S3, S5, S6 clamp: float32 values clamped to [-tau, tau].
  const float tau = (is_v ? a.rv.tau_V : a.rv.tau_K)[h];
  const CodeCuts cuts = code_cuts(code_thresholds(levels_of(a.rv, h, is_v)));
  float v[8][4];
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[nt][r] = fminf(fmaxf((float)(acc[nt][r] * kInvSqrtD), -tau), tau);
      mx = fmaxf(mx, v[nt][r]);
      mn = fminf(mn, v[nt][r]);
    }
  }
  // S6 group statistics over the slot's 64 channels of group L4: the lanes
  // l and l ^ 32.  First swap: a lower lane gets the partner's maximum, an
  // upper lane the partner's minimum; second swap hands each result over.
  {
    float x = mx, y = mn;
    half_swap<2>(x, y);
    const float t = (lane & 32) ? fminf(x, y) : fmaxf(x, y);
    float c = t, d = t;
    half_swap<2>(c, d);
    mx = c;
    mn = d;
  }
  // Group metadata as in quantize_group.
  const float za = meta_zero_step(tau), sb = meta_scale_step(tau);
  uint32_t z8 = 0, s8 = 0;
  {
    const float sg = __fdiv_rn(mx - mn, 3.0f);
    if (za > 0.0f) z8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(mn + tau, za)), 0.0f), 255.0f);
    if (sb > 0.0f) s8 = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(sg, sb)), 0.0f), 255.0f);
  }
  const float zf = (float)z8 * za - tau, sf = (float)s8 * sb;
  const int slot = 16 * w + mi;
  const bool valid = c0 + slot >= t0 && c0 + slot < t1;
  uint8_t *page = pv.pages + ((size_t)phys * pv.hkv + h) * kPageBytes;
  {
    // the token's 4-byte entry: s8_0 | z8_0 << 8 from lane bit 4 clear,
    // s8_1 | z8_1 << 8 from the lane 16 above
    uint32_t m0 = s8 | (z8 << 8), m1 = m0;
    half_swap<1>(m0, m1);
    if ((lane & 48) == 0 && valid)
      *(uint32_t *)(page + (is_v ? kVMeta : kKMeta) + meta_entry(slot) * 4) = m0 | (m1 << 16);
  }

  // S7 codes (level_code of fl(fl(v - zero) / scale), all 0 when the scale
  // is 0) through the cutoffs of code_cut; S8 packing.
  float cut[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) cut[j] = sf != 0.0f ? code_cut(cuts, j, sf) : INFINITY;
  uint32_t code[8][4];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float d = v[nt][r] - zf;
      code[nt][r] = (uint32_t)(d >= cut[0]) + (uint32_t)(d >= cut[1]) + (uint32_t)(d >= cut[2]);
    }
  }
  if (!is_v) {
    // K row: dword q holds channels 16 q .. 16 q + 15, two bits each; the
    // lane owns dwords 4 L4 + 2 L5 + nt2, whole.
    uint32_t kw[2] = {0, 0};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        kw[nt >> 2] |= code[nt][r] << (2 * (8 * (nt & 1) + 4 * ((nt >> 1) & 1) + 2 * (r & 1) + (r >> 1)));
    }
    if (valid) *(uint2 *)(page + kKCodes + slot * 32 + 4 * (4 * ((lane >> 4) & 1) + 2 * (lane >> 5))) = make_uint2(kw[0], kw[1]);
    return;
  }
  // V: slot 16 w + mi sits in byte 4 (mi / 4) + w of each channel row, bits
  // 2 (mi % 4).  Word j / 4 of the lane collects channel 32 (2 L4 + L5) + j
  // in byte j % 4; the four lanes mi ^ 1, mi ^ 2 merge theirs, then lane
  // mi % 4 == q stores words 2 q, 2 q + 1.
  uint32_t vw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * (nt >> 2) + 8 * (nt & 1) + 4 * ((nt >> 1) & 1) + 2 * (r & 1) + (r >> 1);
      vw[j >> 2] |= code[nt][r] << (8 * (j & 3) + 2 * (mi & 3));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    vw[j] |= (uint32_t)lane_xor_i<1>((int)vw[j]);
    vw[j] |= (uint32_t)lane_xor_i<2>((int)vw[j]);
  }
  {
    const int q = mi & 3;
    const uint32_t wa = q == 0 ? vw[0] : q == 1 ? vw[2] : q == 2 ? vw[4] : vw[6];
    const uint32_t wb = q == 0 ? vw[1] : q == 1 ? vw[3] : q == 2 ? vw[5] : vw[7];
    const int ch = 32 * (2 * ((lane >> 4) & 1) + (lane >> 5)) + 8 * q;   // channel of byte 0 of wa
    const int byte = 4 * (mi >> 2) + w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vst[ch + j][byte] = (uint8_t)(wa >> (8 * j));
      vst[ch + 4 + j][byte] = (uint8_t)(wb >> (8 * j));
    }
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
