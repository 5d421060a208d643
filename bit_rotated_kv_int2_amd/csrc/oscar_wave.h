// Wave-level building blocks shared by the decode kernels: DPP row
// reductions, byte gathers, and the BF16 64-token chunk attention used both
// by the BF16 sink/recent segment and by the all-BF16 baseline.
#pragma once

#include "oscar_internal.h"

namespace oscar {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// DPP controls (GFX9 encoding): quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, 8, 12.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor12 = 0x12C;

template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, dppi<CTRL>(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The value of lane (lane ^ M), M = 1, 2, ..., 32, by VALU lane movement
// instead of an LDS permute: DPP inside a 16-lane row for M < 16, the
// row-pair and half-wave swaps for M = 16, 32.  Where a movement delivers
// the partner's value in one of two results (row rotations by 4 and 12,
// the two outputs of a swap), the lane index is sent through the same
// movement to pick the result that came from lane ^ M.
template <int M>
__device__ __forceinline__ int lane_xor_i(int v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane_xor: M");
  if constexpr (M == 1) {
    return dppi<kDppQuadSwap1>(v);
  } else if constexpr (M == 2) {
    return dppi<kDppQuadSwap2>(v);
  } else if constexpr (M == 8) {
    return dppi<kDppRowRor8>(v);   // rotation by half a row: lane ^ 8 either way
  } else if constexpr (M == 4) {
    // both rotations by every lane before the choice: a DPP read from a
    // lane that a branch has switched off yields 0
    const int l = lane_id();
    const int a = dppi<kDppRowRor4>(v), b = dppi<kDppRowRor12>(v);
    return dppi<kDppRowRor4>(l) == (l ^ 4) ? a : b;
  } else {
    const int l = lane_id();
    if constexpr (M == 16) {
      const auto li = __builtin_amdgcn_permlane16_swap(l, l, false, false);
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (int)li[0] == (l ^ 16) ? (int)r[0] : (int)r[1];
    } else {
      const auto li = __builtin_amdgcn_permlane32_swap(l, l, false, false);
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (int)li[0] == (l ^ 32) ? (int)r[0] : (int)r[1];
    }
  }
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  return __builtin_bit_cast(float, lane_xor_i<M>(__builtin_bit_cast(int, v)));
}
template <int M>
__device__ __forceinline__ double lane_xor_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)lane_xor_i<M>((int)(uint32_t)b), hi = (uint32_t)lane_xor_i<M>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Reductions over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15); every
// lane of the row receives the result.  The maximum takes a plain DPP move
// and the NaN-propagating maximum (one v_maximum3_f32 per step; fmaxf would
// add a canonicalising max of the moved value).  Inputs are never NaN.
template <int CTRL>
__device__ __forceinline__ float movdppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_elementwise_maximum(v, movdppf<kDppQuadSwap1>(v));
  v = __builtin_elementwise_maximum(v, movdppf<kDppQuadSwap2>(v));
  v = __builtin_elementwise_maximum(v, movdppf<kDppRowRor4>(v));
  v = __builtin_elementwise_maximum(v, movdppf<kDppRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<kDppQuadSwap1>(v);
  v += dppf<kDppQuadSwap2>(v);
  v += dppf<kDppRowRor4>(v);
  v += dppf<kDppRowRor8>(v);
  return v;
}

// Stages 1, 2, ..., 32 of a 128-point Walsh-Hadamard butterfly whose
// elements l and l + 64 sit in lane l; stage 64 (x0 +- x1) is the caller's.
template <int M>
__device__ __forceinline__ void fwht_lane_stage(float &x0, float &x1, int lane) {
  const float o0 = lane_xor<M>(x0), o1 = lane_xor<M>(x1);
  x0 = (lane & M) ? o0 - x0 : x0 + o0;
  x1 = (lane & M) ? o1 - x1 : x1 + o1;
}
__device__ __forceinline__ void fwht_lane_stages(float &x0, float &x1, int lane) {
  fwht_lane_stage<1>(x0, x1, lane);
  fwht_lane_stage<2>(x0, x1, lane);
  fwht_lane_stage<4>(x0, x1, lane);
  fwht_lane_stage<8>(x0, x1, lane);
  fwht_lane_stage<16>(x0, x1, lane);
  fwht_lane_stage<32>(x0, x1, lane);
}

// Reductions over the whole wave; every lane receives the result.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_min(float v) {
  v = __builtin_elementwise_minimum(v, movdppf<kDppQuadSwap1>(v));
  v = __builtin_elementwise_minimum(v, movdppf<kDppQuadSwap2>(v));
  v = __builtin_elementwise_minimum(v, movdppf<kDppRowRor4>(v));
  v = __builtin_elementwise_minimum(v, movdppf<kDppRowRor8>(v));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fminf(fminf(a, b), fminf(c, d));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a + b) + (c + d);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dppi<kDppQuadSwap1>(v);
  v += dppi<kDppQuadSwap2>(v);
  v += dppi<kDppRowRor4>(v);
  v += dppi<kDppRowRor8>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// ---------------------------------------------------------------------------
// BF16 chunk attention for one wave.
//   K, V: 64 bf16 rows of 128 channels (row t = token t), `valid` leading rows
//   are real tokens.  Aq: the query operand of v_mfma_f32_16x16x32_bf16 with
//   rows = query heads (lane n = head, kgroup q: channels 32 q + 8 ks ..).
//   Running state (log2 units): m[i], l[i] for the head 4 q + i of the C
//   layout, and o[h][8] for channels 8 n .. 8 n + 7 and the token phase q
//   (summed over q at the end).  ps: this wave's [16][68] LDS scratch.
// ---------------------------------------------------------------------------
template <int GH>
__device__ __forceinline__ void bf16_chunk(const uint16_t *K, const uint16_t *V, int valid, int G,
                                           const v8bf (&Aq)[4], float sl2, float (&m)[4],
                                           float (&l)[4], float (&mrow)[GH], float (&o)[GH][8],
                                           float (*ps)[kPageTokens + 4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  float lg[4][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const uint16_t *kr = K + (size_t)(16 * tt + n) * kD + 32 * q;
    uint4 kk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kk[ks] = *(const uint4 *)(kr + 8 * ks);
    v4f C = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aq[ks], as_v8bf(kk[ks]), C, 0, 0, 0);
    const bool ok = (16 * tt + n) < valid;
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[tt][i] = ok ? C[i] * sl2 : -INFINITY;
  }
  float pm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = fmaxf(fmaxf(lg[0][i], lg[1][i]), fmaxf(lg[2][i], lg[3][i]));
    v = row16_max(v);
    const float mn = fmaxf(m[i], v);
    const float al = exp2_fast(m[i] - mn);
    float s = 0.f;
    float e[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      e[tt] = exp2_fast(lg[tt][i] - mn);
      s += e[tt];
    }
    s = row16_sum(s);
    l[i] = l[i] * al + s;
    m[i] = mn;
    pm[i] = mn;
    const int h = 4 * q + i;
    if (h < G) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) ps[h][16 * tt + n] = e[tt];
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    if (h >= G) continue;
    const int i = h & 3;
    const float v = (i == 0) ? pm[0] : (i == 1) ? pm[1] : (i == 2) ? pm[2] : pm[3];
    const float mh = __shfl(v, 16 * (h >> 2), 64);
    const float al = exp2_fast(mrow[h] - mh);
    mrow[h] = mh;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[h][c] *= al;
  }
  // Value rows: 16 tokens per lane (token phase q), issued 4 at a time so the
  // loads overlap.  Rows past `valid` re-read the last valid row (finite data)
  // and meet p = 0.
  const int tmax = valid - 1;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    uint4 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = min(q + 4 * (4 * blk + i), tmax);
      u[i] = *(const uint4 *)(V + (size_t)t * kD + 8 * n);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = q + 4 * (4 * blk + i);
      float vf[8];
      vf[0] = __uint_as_float(u[i].x << 16);
      vf[1] = __uint_as_float(u[i].x & 0xFFFF0000u);
      vf[2] = __uint_as_float(u[i].y << 16);
      vf[3] = __uint_as_float(u[i].y & 0xFFFF0000u);
      vf[4] = __uint_as_float(u[i].z << 16);
      vf[5] = __uint_as_float(u[i].z & 0xFFFF0000u);
      vf[6] = __uint_as_float(u[i].w << 16);
      vf[7] = __uint_as_float(u[i].w & 0xFFFF0000u);
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        if (h >= G) continue;
        const float p = ps[h][t];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[h][c] = fmaf(p, vf[c], o[h][c]);
      }
    }
  }
  wave_lds_sync();
}

// BF16 attention of one 16-token tile for one wave, from a fresh state, in
// two parts so that several tiles' loads can be in flight together.
//   K, V: 16 bf16 rows of 128 channels; the first `valid` (1..16) are real
//   tokens (rows past them are re-read from row valid - 1 and masked).
//   bf16_tile_load issues all eight 16-byte loads of a lane; bf16_tile_math
//   gives (log2 units) m[i], l[i] for head 4 q + i (row-uniform), o[h][8] =
//   sum over this lane's token phase (tokens q, q + 4, q + 8, q + 12) of p V
//   for channels 8 n .. 8 n + 7, relative to m.  ps: [GH][>= 16] LDS scratch
//   of the wave.
struct TileRegs {
  uint4 kk[4], vv[4];
};
__device__ __forceinline__ void bf16_tile_load(const uint16_t *K, const uint16_t *V, int valid, TileRegs &r) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const uint16_t *kr = K + (size_t)min(n, valid - 1) * kD + 32 * q;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) r.kk[ks] = *(const uint4 *)(kr + 8 * ks);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.vv[i] = *(const uint4 *)(V + (size_t)min(q + 4 * i, valid - 1) * kD + 8 * n);
}
template <int GH>
__device__ __forceinline__ void bf16_tile_math(const TileRegs &r, int valid, int G, const v8bf (&Aq)[4], float sl2,
                                               float (&m)[4], float (&l)[4], float (&o)[GH][8], float (*ps)[kD]) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  v4f C = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aq[ks], as_v8bf(r.kk[ks]), C, 0, 0, 0);
  const bool ok = n < valid;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lg = ok ? C[i] * sl2 : -INFINITY;
    m[i] = row16_max(lg);
    const float e = exp2_fast(lg - m[i]);   // valid >= 1: m is finite
    l[i] = row16_sum(e);
    const int h = 4 * q + i;
    if (h < G) ps[h][n] = e;
  }
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < GH; ++h) {
#pragma unroll
    for (int c = 0; c < 8; ++c) o[h][c] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vf[8];
    vf[0] = __uint_as_float(r.vv[i].x << 16);
    vf[1] = __uint_as_float(r.vv[i].x & 0xFFFF0000u);
    vf[2] = __uint_as_float(r.vv[i].y << 16);
    vf[3] = __uint_as_float(r.vv[i].y & 0xFFFF0000u);
    vf[4] = __uint_as_float(r.vv[i].z << 16);
    vf[5] = __uint_as_float(r.vv[i].z & 0xFFFF0000u);
    vf[6] = __uint_as_float(r.vv[i].w << 16);
    vf[7] = __uint_as_float(r.vv[i].w & 0xFFFF0000u);
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      // heads past G: continue keeps the loop fully unrolled (with break, twelve
      // heads kept o in scratch memory); sixteen heads fully unrolled fail to
      // compile with this toolchain, so they keep the early exit
      if (h >= G) {
        if constexpr (GH <= 12) continue;
        else break;
      }
      const float p = ps[h][q + 4 * i];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[h][c] = fmaf(p, vf[c], o[h][c]);
    }
  }
  wave_lds_sync();
}
template <int GH>
__device__ __forceinline__ void bf16_tile(const uint16_t *K, const uint16_t *V, int valid, int G,
                                          const v8bf (&Aq)[4], float sl2, float (&m)[4], float (&l)[4],
                                          float (&o)[GH][8], float (*ps)[kD]) {
  TileRegs r;
  bf16_tile_load(K, V, valid, r);
  bf16_tile_math<GH>(r, valid, G, Aq, sl2, m, l, o, ps);
}

// Load the bf16 query rows of the G heads of one KV head as the A operand.
__device__ __forceinline__ void load_bf16_query(const uint16_t *qbase, int G, v8bf (&Aq)[4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = {0, 0, 0, 0};
    if (n < G) u = *(const uint4 *)(qbase + (size_t)n * kD + 32 * q + 8 * ks);
    Aq[ks] = as_v8bf(u);
  }
}

// Sum the PV partials over the 4 token phases and combine the 4 waves of a
// block into one (m, l, o) partial per head (m in log2 units).
template <int GH>
__device__ __forceinline__ void bf16_block_combine(int G, const float (&m)[4], const float (&l)[4],
                                                   float (&o)[GH][8], float (*sm_m)[GH], float (*sm_l)[GH],
                                                   float (*sm_o)[GH][kD], float *dst_base) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    if (h >= G) continue;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[h][c];
      v += lane_xor<16>(v);
      v += lane_xor<32>(v);
      o[h][c] = v;
    }
  }
  if (q == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      if (h >= G) continue;
#pragma unroll
      for (int c = 0; c < 8; ++c) sm_o[wave][h][8 * n + c] = o[h][c];
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
  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, c = idx % kD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float ov = 0.f, lv = 0.f;
    if (M > -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (sm_m[w][h] == -INFINITY) continue;
        const float sc = exp2_fast(sm_m[w][h] - M);
        ov += sc * sm_o[w][h][c];
        lv += sc * sm_l[w][h];
      }
    }
    float *dst = dst_base + (size_t)h * kPartStride;
    if (c == 0) {
      st_coherent(dst, M);
      st_coherent(dst + 1, lv);
    }
    st_coherent(dst + kPartO + c, ov);
  }
}

}  // namespace oscar
