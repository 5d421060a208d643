// Host check of the code cutoffs (code_cuts / code_cut in oscar_internal.h):
// for every scale and threshold set tried, "a >= cut" must agree with the
// term of level_code on the correctly rounded quotient fl(a / s), for floats
// a at, around and between the cutoffs, and for ties at the rounding
// midpoints where those exist (subnormal thresholds).  Prints the number of
// disagreements and exits non-zero when there is one.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>

#include "oscar_internal.h"

using oscar::CodeCuts;
using oscar::CodeThresholds;

static uint32_t direct_code(float a, float s, const CodeThresholds &th) {
  const volatile float q = a / s;   // IEEE float division, round to nearest even
  return oscar::level_code(q, th);
}
static uint32_t cut_code(float a, const float cut[3]) {
  return (uint32_t)(a >= cut[0]) + (uint32_t)(a >= cut[1]) + (uint32_t)(a >= cut[2]);
}
static float step(float x, int n) {
  for (; n > 0; --n) x = nextafterf(x, INFINITY);
  for (; n < 0; ++n) x = nextafterf(x, -INFINITY);
  return x;
}

int main() {
  std::mt19937_64 rng(12345);
  std::uniform_real_distribution<float> U(0.0f, 1.0f);
  long long checked = 0, bad = 0;
  std::vector<CodeThresholds> ths;
  ths.push_back(oscar::code_thresholds(0xC0804000u));   // uniform grid 0, 1, 2, 3 (x 64)
  for (int i = 0; i < 200; ++i) {                       // random increasing codebooks
    uint32_t n[4];
    for (int j = 0; j < 4; ++j) n[j] = (uint32_t)(rng() % 256);
    for (int j = 1; j < 4; ++j)
      for (int k = j; k > 0 && n[k] < n[k - 1]; --k) std::swap(n[k], n[k - 1]);
    ths.push_back(oscar::code_thresholds(n[0] | (n[1] << 8) | (n[2] << 16) | (n[3] << 24)));
  }
  // thresholds at and near zero and in the subnormal range, where ties at
  // the midpoints are reachable
  const float dmin = std::numeric_limits<float>::denorm_min();
  ths.push_back(CodeThresholds{0.0f, dmin, 3 * dmin});
  ths.push_back(CodeThresholds{-dmin, 2 * dmin, 5 * dmin});
  ths.push_back(CodeThresholds{-0.0f, 0.0f, 1e-40f});
  auto check = [&](float a, float s, const CodeThresholds &th, const float cut[3]) {
    ++checked;
    if (direct_code(a, s, th) != cut_code(a, cut)) {
      if (bad < 10)
        std::printf("a=%a s=%a t=(%a %a %a): direct %u cut %u\n", a, s, th.t0, th.t1, th.t2,
                    direct_code(a, s, th), cut_code(a, cut));
      ++bad;
    }
  };
  for (size_t ti = 0; ti < ths.size(); ++ti) {
    const CodeThresholds &th = ths[ti];
    const CodeCuts cc = oscar::code_cuts(th);
    for (int si = 0; si < 600; ++si) {
      float s;
      if (si < 255) {                       // the scale grid s8 * (2 tau / 765) for a random tau
        const float tau = std::ldexp(0.5f + U(rng), (int)(rng() % 40) - 20);
        s = (float)(si + 1) * (2.0f * tau / 765.0f);
      } else if (si < 400) {                // powers of two and small integers (ties)
        s = std::ldexp((float)(1 + rng() % 7), (int)(rng() % 60) - 30);
      } else if (si < 450) {                // subnormal and tiny scales
        s = dmin * (float)(1 + rng() % 1000);
      } else {                              // arbitrary floats
        s = std::ldexp(0.5f + U(rng), (int)(rng() % 200) - 100);
      }
      float cut[3];
      for (int j = 0; j < 3; ++j) cut[j] = oscar::code_cut(cc, j, s);
      for (int j = 0; j < 3; ++j) {
        if (std::isinf(cut[j])) continue;
        for (int d = -3; d <= 3; ++d) check(step(cut[j], d), s, th, cut);
      }
      // ties: a = m s where representable
      for (int j = 0; j < 3; ++j) {
        const double b = cc.m[j] * (double)s;
        const float f = (float)b;
        if ((double)f == b) for (int d = -1; d <= 1; ++d) check(step(f, d), s, th, cut);
      }
      for (int k = 0; k < 64; ++k) {        // spread over the code range
        const float a = (float)((U(rng) * 4.0f - 0.5f) * s);
        check(a, s, th, cut);
        check(-a, s, th, cut);
      }
    }
  }
  std::printf("code cutoffs: %lld cases, %lld disagreements\n", checked, bad);
  return bad != 0;
}
