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

}  // namespace oscar
