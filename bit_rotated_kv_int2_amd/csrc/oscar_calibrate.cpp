// Offline calibration of the per-head rotation and clip thresholds, host
// side, float64.
//
// Sources: [B] MarkTechPost (zh) "Together AI 开源 OSCAR…", section
// "OSCAR 有何不同做法" (key basis = eigenvectors of the empirical query
// covariance C_Q = (1/N) sum q^T q; value basis = eigenvectors of the
// score-weighted value covariance C_S = (1/N) V^T S^T S V; R = U H_Had P_br)
// and visual-guide step 04 (one-off offline calibration from a small sample
// producing per-layer rotations and clip thresholds); section
// "服务系统：混合精度缓存布局" (clip thresholds are calibration percentiles).
//
// Readings where the pages are silent: query heads sharing a KV head are
// pooled; S is the softmax of the scaled calibration scores, no mask;
// eigenvectors are ordered by descending eigenvalue and each column's
// largest-magnitude entry is made positive; tau is the linear-interpolation
// quantile of |x R| over every rotated calibration entry of the head.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "oscar_internal.h"

namespace oscar {
namespace {

int n_threads() {
  unsigned n = std::thread::hardware_concurrency();
  if (n == 0) n = 4;
  return (int)std::min(n, 16u);
}

template <class F>
void parallel_for(int64_t n, F f) {
  const int T = (int)std::min<int64_t>(n_threads(), std::max<int64_t>(1, n));
  std::vector<std::thread> th;
  for (int t = 0; t < T; ++t)
    th.emplace_back([&, t] {
      for (int64_t i = t; i < n; i += T) f(t, i);
    });
  for (auto &x : th) x.join();
}

// Cyclic Jacobi eigen-decomposition of a symmetric d x d matrix (row-major).
// On return A holds the eigenvalues on its diagonal and V the eigenvectors as
// columns.
void jacobi_eigen(int d, std::vector<double> &A, std::vector<double> &V) {
  V.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) V[(size_t)i * d + i] = 1.0;
  double total = 0.0;
  for (double x : A) total += x * x;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off += A[(size_t)p * d + q] * A[(size_t)p * d + q];
    if (off <= 1e-32 * total) break;
    for (int p = 0; p < d; ++p) {
      for (int q = p + 1; q < d; ++q) {
        const double apq = A[(size_t)p * d + q];
        if (apq == 0.0) continue;
        const double app = A[(size_t)p * d + p], aqq = A[(size_t)q * d + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < d; ++k) {   // columns p, q
          const double akp = A[(size_t)k * d + p], akq = A[(size_t)k * d + q];
          A[(size_t)k * d + p] = c * akp - s * akq;
          A[(size_t)k * d + q] = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {   // rows p, q
          const double apk = A[(size_t)p * d + k], aqk = A[(size_t)q * d + k];
          A[(size_t)p * d + k] = c * apk - s * aqk;
          A[(size_t)q * d + k] = s * apk + c * aqk;
        }
        A[(size_t)p * d + q] = A[(size_t)q * d + p] = 0.0;
        for (int k = 0; k < d; ++k) {
          const double vkp = V[(size_t)k * d + p], vkq = V[(size_t)k * d + q];
          V[(size_t)k * d + p] = c * vkp - s * vkq;
          V[(size_t)k * d + q] = s * vkp + c * vkq;
        }
      }
    }
  }
}

// Sorted, sign-fixed eigenbasis as float32 columns.  Returns false when a
// relative eigen-gap is below 1e-10 (basis not unique).
bool sorted_basis(int d, const std::vector<double> &C, float *U32) {
  std::vector<double> A(C), V;
  for (int i = 0; i < d; ++i)
    for (int j = i + 1; j < d; ++j) {
      const double m = 0.5 * (A[(size_t)i * d + j] + A[(size_t)j * d + i]);
      A[(size_t)i * d + j] = A[(size_t)j * d + i] = m;
    }
  jacobi_eigen(d, A, V);
  std::vector<int> idx(d);
  for (int i = 0; i < d; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int a, int b) { return A[(size_t)a * d + a] > A[(size_t)b * d + b]; });
  const double scale = std::max(std::fabs(A[(size_t)idx[0] * d + idx[0]]), 1e-300);
  for (int i = 0; i + 1 < d; ++i) {
    const double gap = std::fabs(A[(size_t)idx[i] * d + idx[i]] - A[(size_t)idx[i + 1] * d + idx[i + 1]]);
    if (gap / scale < 1e-10) return false;
  }
  for (int j = 0; j < d; ++j) {
    const int src = idx[j];
    int arg = 0;
    double best = -1.0;
    for (int k = 0; k < d; ++k) {
      const double v = std::fabs(V[(size_t)k * d + src]);
      if (v > best) {
        best = v;
        arg = k;
      }
    }
    const double sgn = V[(size_t)arg * d + src] < 0 ? -1.0 : 1.0;
    for (int k = 0; k < d; ++k) U32[(size_t)k * d + j] = (float)(sgn * V[(size_t)k * d + src]);
  }
  return true;
}

// Quantile with linear interpolation, following the order of float64
// operations of the common "linear" (type 7) definition.
double quantile_linear(std::vector<double> &v, double qv) {
  const int64_t n = (int64_t)v.size();
  const double vi = (double)n * qv + (1.0 + qv * (-1.0)) - 1.0;
  double lo_d = std::floor(vi);
  int64_t lo = (int64_t)lo_d;
  lo = std::max<int64_t>(0, std::min<int64_t>(n - 1, lo));
  const int64_t hi = std::min<int64_t>(n - 1, lo + 1);
  const double gamma = vi - lo_d;
  std::nth_element(v.begin(), v.begin() + lo, v.end());
  const double a = v[lo];
  double b = a;
  if (hi != lo) b = *std::min_element(v.begin() + lo + 1, v.end());
  const double diff = b - a;
  double r = (gamma >= 0.5) ? b - diff * (1.0 - gamma) : a + diff * gamma;
  if (a == b) r = a;
  return r;
}

// |x R| entries for every row of x [n][d] (float32 holding bf16 values),
// R = U32 H P; the permutation does not change the multiset.
void rotated_abs_serial(int d, const float *x, int64_t n, const float *U32, std::vector<double> &out) {
  out.resize((size_t)n * d);
  const double c = 1.0 / std::sqrt((double)d);
  std::vector<double> y(d);
  for (int64_t r = 0; r < n; ++r) {
    std::fill(y.begin(), y.end(), 0.0);
    const float *xr = x + (size_t)r * d;
    for (int k = 0; k < d; ++k) {
      const double xk = xr[k];
      const float *Uk = U32 + (size_t)k * d;
      for (int j = 0; j < d; ++j) y[j] += xk * (double)Uk[j];
    }
    for (int h = 1; h < d; h <<= 1)
      for (int i = 0; i < d; ++i)
        if (!(i & h)) {
          const double a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
    for (int j = 0; j < d; ++j) out[(size_t)r * d + j] = std::fabs(y[j] * c);
  }
}

}  // namespace

int calibrate_host(int d, int hkv, int hq, float sm_scale, const float *q_cal, int64_t n_q,
                   const float *k_cal, const float *v_cal, int64_t n_kv, double quantile_k,
                   double quantile_v, float *U_K, float *U_V, float *tau_K, float *tau_V,
                   char *err, size_t err_len) {
  const int G = hq / hkv;
  const int T = n_threads();
  std::vector<std::vector<double>> CQall(hkv), CSall(hkv);
  for (int kv = 0; kv < hkv; ++kv) {
    const float *K = k_cal + (size_t)kv * n_kv * d;
    const float *Vv = v_cal + (size_t)kv * n_kv * d;
    std::vector<std::vector<double>> cq(T, std::vector<double>((size_t)d * d, 0.0));
    std::vector<std::vector<double>> cs(T, std::vector<double>((size_t)d * d, 0.0));
    std::vector<double> Kd((size_t)n_kv * d), Vd((size_t)n_kv * d);
    for (size_t i = 0; i < Kd.size(); ++i) {
      Kd[i] = K[i];
      Vd[i] = Vv[i];
    }
    const int64_t rows = (int64_t)G * n_q;
    parallel_for(rows, [&](int t, int64_t r) {
      const int h = (int)(r / n_q);
      const int64_t i = r % n_q;
      const float *qr = q_cal + ((size_t)(kv * G + h) * n_q + i) * d;
      std::vector<double> qd(d), lg(n_kv), sv(d, 0.0);
      for (int c = 0; c < d; ++c) qd[c] = qr[c];
      double *CQ = cq[t].data();
      for (int a = 0; a < d; ++a) {
        const double qa = qd[a];
        for (int b = 0; b < d; ++b) CQ[(size_t)a * d + b] += qa * qd[b];
      }
      double mx = -INFINITY;
      for (int64_t j = 0; j < n_kv; ++j) {
        const double *kr = &Kd[(size_t)j * d];
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += qd[c] * kr[c];
        lg[j] = s * (double)sm_scale;
        mx = std::max(mx, lg[j]);
      }
      double den = 0.0;
      for (int64_t j = 0; j < n_kv; ++j) {
        lg[j] = std::exp(lg[j] - mx);
        den += lg[j];
      }
      for (int64_t j = 0; j < n_kv; ++j) {
        const double w = lg[j] / den;
        const double *vr = &Vd[(size_t)j * d];
        for (int c = 0; c < d; ++c) sv[c] += w * vr[c];
      }
      double *CS = cs[t].data();
      for (int a = 0; a < d; ++a) {
        const double sa = sv[a];
        for (int b = 0; b < d; ++b) CS[(size_t)a * d + b] += sa * sv[b];
      }
    });
    CQall[kv].assign((size_t)d * d, 0.0);
    CSall[kv].assign((size_t)d * d, 0.0);
    for (int t = 0; t < T; ++t)
      for (size_t i = 0; i < CQall[kv].size(); ++i) {
        CQall[kv][i] += cq[t][i];
        CSall[kv][i] += cs[t][i];
      }
    for (size_t i = 0; i < CQall[kv].size(); ++i) {
      CQall[kv][i] /= (double)rows;
      CSall[kv][i] /= (double)rows;
    }
  }
  // Eigenbases and thresholds of all heads in parallel (2 * hkv independent jobs).
  std::vector<int> bad(2 * hkv, 0);
  std::vector<std::vector<double>> vals(2 * hkv);
  parallel_for(2 * hkv, [&](int, int64_t job) {
    const int kv = (int)(job >> 1);
    const bool is_v = job & 1;
    float *U = (is_v ? U_V : U_K) + (size_t)kv * d * d;
    if (!sorted_basis(d, is_v ? CSall[kv] : CQall[kv], U)) {
      bad[job] = 1;
      return;
    }
    const float *X = (is_v ? v_cal : k_cal) + (size_t)kv * n_kv * d;
    rotated_abs_serial(d, X, n_kv, U, vals[job]);
    const double tq = quantile_linear(vals[job], is_v ? quantile_v : quantile_k);
    (is_v ? tau_V : tau_K)[kv] = (float)tq;
  });
  for (int job = 0; job < 2 * hkv; ++job)
    if (bad[job]) {
      snprintf(err, err_len, "kv head %d: %s spectrum is degenerate", job >> 1,
               (job & 1) ? "score-weighted value covariance" : "query covariance");
      return OSCAR_EINVAL;
    }
  return OSCAR_OK;
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook ([A] summary and outlook: a Lloyd-Max codebook for the
// 2-bit codes).  Every calibration token takes the write path up to its codes
// (the arithmetic order of the append kernels), the normalised values
// u = (x - zero) / scale of its groups with a non-zero scale are collected,
// and a 4-level Lloyd-Max quantiser of them, rounded to the 1/32 grid, gives
// the head's levels.
// ---------------------------------------------------------------------------
namespace {

constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;   // nearest double to 1/sqrt(128)

#pragma clang fp contract(off)
// u values of one token x [d] (float32 holding bf16), d = 128.
void token_normalised(int d, const float *x, const float *U, float tau, std::vector<float> &out) {
  double y[128];
  for (int j = 0; j < d; ++j) y[j] = 0.0;
  for (int k = 0; k < d; ++k) {   // S1: k ascending, one accumulator per output
    const double xk = (double)x[k];
    const float *ur = U + (size_t)k * d;
    for (int j = 0; j < d; ++j) y[j] += xk * (double)ur[j];
  }
  for (int h = 1; h < d; h <<= 1)   // S2: butterfly stages 1, 2, ..., 64
    for (int i = 0; i < d; ++i)
      if ((i & h) == 0) {
        const double a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  float xr[128];
  for (int pos = 0; pos < d; ++pos) {   // S3, S4, S5, S6
    const int src = bitrev7(pos);
    const float v = (float)(y[src] * kInvSqrt128);
    xr[pos] = std::fmin(std::fmax(v, -tau), tau);
  }
  const float za = (tau + tau) / 255.0f, sb = (tau + tau) / 765.0f;
  for (int g = 0; g < d / 64; ++g) {   // S7: group metadata, then u
    const float *xg = xr + 64 * g;
    float mx = xg[0], mn = xg[0];
    for (int c = 1; c < 64; ++c) {
      mx = std::fmax(mx, xg[c]);
      mn = std::fmin(mn, xg[c]);
    }
    const float sg = (mx - mn) / 3.0f;
    float z8 = 0.0f, s8 = 0.0f;
    if (za > 0.0f) z8 = std::fmin(std::fmax(std::nearbyint((mn + tau) / za), 0.0f), 255.0f);
    if (sb > 0.0f) s8 = std::fmin(std::fmax(std::nearbyint(sg / sb), 0.0f), 255.0f);
    const float zf = z8 * za - tau;
    const float sf = s8 * sb;
    if (sf == 0.0f) continue;
    for (int c = 0; c < 64; ++c) out.push_back((xg[c] - zf) / sf);
  }
}
#pragma clang fp contract(on)

// Lloyd-Max levels of the sorted samples x, from (0, 1, 2, 3).
void lloyd_max4(const std::vector<double> &x, double c[4]) {
  std::vector<double> csum(x.size() + 1, 0.0);
  for (size_t i = 0; i < x.size(); ++i) csum[i + 1] = csum[i] + x[i];
  for (int k = 0; k < 4; ++k) c[k] = (double)k;
  for (int it = 0; it < 1000; ++it) {
    size_t edges[5];
    edges[0] = 0;
    edges[4] = x.size();
    for (int k = 0; k < 3; ++k) {
      const double t = (c[k] + c[k + 1]) / 2;
      edges[k + 1] = (size_t)(std::lower_bound(x.begin(), x.end(), t) - x.begin());
    }
    double nc[4], moved = 0.0;
    for (int k = 0; k < 4; ++k) {
      nc[k] = c[k];
      if (edges[k + 1] > edges[k])
        nc[k] = (csum[edges[k + 1]] - csum[edges[k]]) / (double)(edges[k + 1] - edges[k]);
      moved = std::max(moved, std::fabs(nc[k] - c[k]));
    }
    for (int k = 0; k < 4; ++k) c[k] = nc[k];
    if (moved <= 1e-12) break;
  }
}

}  // namespace

int calibrate_codebook_host(int d, int hkv, const float *U, const float *tau, const float *x_cal, int64_t n,
                            uint32_t *levels, char *err, size_t err_len) {
  if (d != 128) {
    snprintf(err, err_len, "codebook calibration needs head_dim 128");
    return OSCAR_ENOTSUP;
  }
  for (int h = 0; h < hkv; ++h) {
    if (!(tau[h] >= 0.0f) || !std::isfinite(tau[h])) {
      snprintf(err, err_len, "tau of head %d is not a finite non-negative value", h);
      return OSCAR_EINVAL;
    }
  }
  parallel_for(hkv, [&](int, int64_t h) {
    const float *Uh = U + (size_t)h * d * d;
    const float *xh = x_cal + (size_t)h * n * d;
    std::vector<float> u;
    u.reserve((size_t)n * d);
    for (int64_t t = 0; t < n; ++t) token_normalised(d, xh + (size_t)t * d, Uh, tau[h], u);
    std::vector<double> x(u.begin(), u.end());
    std::sort(x.begin(), x.end());
    double c[4];
    lloyd_max4(x, c);
    int nk[4];
    for (int k = 0; k < 4; ++k) nk[k] = (int)std::min(96.0, std::max(0.0, std::nearbyint(c[k] * 32.0)));
    for (int k = 1; k < 4; ++k) nk[k] = std::max(nk[k], nk[k - 1] + 1);
    for (int k = 3; k >= 0; --k) {
      nk[k] = std::min(nk[k], 96 - (3 - k));
      if (k < 3) nk[k] = std::min(nk[k], nk[k + 1] - 1);
    }
    levels[h] = (uint32_t)nk[0] | ((uint32_t)nk[1] << 8) | ((uint32_t)nk[2] << 16) | ((uint32_t)nk[3] << 24);
  });
  return OSCAR_OK;
}

}  // namespace oscar
