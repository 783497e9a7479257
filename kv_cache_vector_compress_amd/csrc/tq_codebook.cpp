// Lloyd-Max codebook for coordinates ~ N(0, 1/d), built on the host.
//
// The pages give the interface (nav.superapi.store "turboquant-pytorch",
// 核心 API: build_lloyd_max_codebook(dim, bits) -> (boundaries, centroids))
// and say the codebook is the MSE-optimal scalar quantiser of the rotated
// coordinates, whose law is N(0, 1/d) (算法细节 / 随机旋转).  Lloyd-Max
// optimality means: every boundary is the midpoint of its two centroids and
// every centroid is the mean of the density over its cell.  For a Gaussian
// the cell mean has the closed form
//     E[X | a < X <= b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a))   (X ~ N(0,1)),
// so the fixed point is solved here with Newton's method on that map, using
// erfc for tail probabilities.  The codebook of N(0, 1/d) is the standard
// one scaled by 1/sqrt(d).
#include <cmath>
#include <cstring>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr double kInvSqrt2Pi = 0.39894228040143267794;
constexpr double kInvSqrt2 = 0.70710678118654752440;

double phi(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }

// P(a < X <= b) for X ~ N(0,1), accurate in both tails.
double cell_prob(double a, double b) {
  if (a >= 0.0) return 0.5 * (std::erfc(a * kInvSqrt2) - std::erfc(b * kInvSqrt2));
  if (b <= 0.0) return 0.5 * (std::erfc(-b * kInvSqrt2) - std::erfc(-a * kInvSqrt2));
  return 1.0 - 0.5 * std::erfc(-a * kInvSqrt2) - 0.5 * std::erfc(b * kInvSqrt2);
}

// Solve the small dense system J x = r in place (Gaussian elimination, partial pivoting).
bool solve(int n, double* J, double* r) {
  for (int c = 0; c < n; ++c) {
    int p = c;
    for (int i = c + 1; i < n; ++i)
      if (std::fabs(J[i * n + c]) > std::fabs(J[p * n + c])) p = i;
    if (J[p * n + c] == 0.0) return false;
    if (p != c) {
      for (int k = 0; k < n; ++k) std::swap(J[p * n + k], J[c * n + k]);
      std::swap(r[p], r[c]);
    }
    for (int i = c + 1; i < n; ++i) {
      double f = J[i * n + c] / J[c * n + c];
      for (int k = c; k < n; ++k) J[i * n + k] -= f * J[c * n + k];
      r[i] -= f * r[c];
    }
  }
  for (int c = n - 1; c >= 0; --c) {
    double s = r[c];
    for (int k = c + 1; k < n; ++k) s -= J[c * n + k] * r[k];
    r[c] = s / J[c * n + c];
  }
  return true;
}

}  // namespace

// Standard-normal Lloyd-Max quantiser with L = 2^bits levels.
bool lloyd_max_standard(int bits, double* c, double* beta) {
  const int L = 1 << bits;
  double edges[17], mu[16], J[256], r[16];
  // start: means of L equal-probability cells, approximated by a uniform
  // spread over +-2.5 sigma (the iteration does not depend on the start)
  for (int i = 0; i < L; ++i) c[i] = -2.5 + 5.0 * (i + 0.5) / L;
  for (int it = 0; it < 200; ++it) {
    edges[0] = -INFINITY;
    edges[L] = INFINITY;
    for (int i = 1; i < L; ++i) edges[i] = 0.5 * (c[i - 1] + c[i]);
    double dmu_da[16], dmu_db[16];
    for (int i = 0; i < L; ++i) {
      double a = edges[i], b = edges[i + 1];
      double P = cell_prob(a, b);
      mu[i] = (phi(a) - phi(b)) / P;
      dmu_da[i] = std::isinf(a) ? 0.0 : phi(a) * (mu[i] - a) / P;
      dmu_db[i] = std::isinf(b) ? 0.0 : phi(b) * (b - mu[i]) / P;
    }
    // F(c) = mu(c) - c; Newton step on F with its analytic Jacobian
    std::memset(J, 0, sizeof(double) * L * L);
    for (int i = 0; i < L; ++i) {
      if (i > 0) { J[i * L + i - 1] += 0.5 * dmu_da[i]; J[i * L + i] += 0.5 * dmu_da[i]; }
      if (i < L - 1) { J[i * L + i] += 0.5 * dmu_db[i]; J[i * L + i + 1] += 0.5 * dmu_db[i]; }
      J[i * L + i] -= 1.0;
      r[i] = -(mu[i] - c[i]);
    }
    double step_max = 0.0;
    if (it < 5 || !solve(L, J, r)) {
      // plain Lloyd update for the first few iterations (robust start)
      for (int i = 0; i < L; ++i) { step_max = std::fmax(step_max, std::fabs(mu[i] - c[i])); c[i] = mu[i]; }
    } else {
      for (int i = 0; i < L; ++i) { step_max = std::fmax(step_max, std::fabs(r[i])); c[i] += r[i]; }
    }
    if (it >= 5 && step_max < 1e-15) break;
  }
  for (int i = 0; i < L / 2; ++i) {  // exact symmetry c_i = -c_{L-1-i}
    double m = 0.5 * (c[L - 1 - i] - c[i]);
    c[i] = -m;
    c[L - 1 - i] = m;
  }
  for (int i = 0; i < L - 1; ++i) beta[i] = 0.5 * (c[i] + c[i + 1]);
  if (L % 2 == 0) beta[L / 2 - 1] = 0.0;
  for (int i = 1; i < L; ++i)
    if (!(c[i] > c[i - 1]) || !std::isfinite(c[i])) return false;
  return true;
}

}  // namespace tq

extern "C" int tq_lloyd_max_codebook(int32_t head_dim, int32_t bits, double* centroids, double* boundaries) {
  if (head_dim < 1 || bits < 0 || bits > 4 || !centroids || (bits > 0 && !boundaries))
    return tq::fail(TQ_EINVAL, "tq_lloyd_max_codebook: need head_dim >= 1, bits in 0..4, non-null outputs");
  if (bits == 0) {  // one cell, the whole line: its centroid is the mean, 0
    centroids[0] = 0.0;
    return TQ_OK;
  }
  double c[16], b[16];
  if (!tq::lloyd_max_standard(bits, c, b)) return tq::fail(TQ_EINVAL, "tq_lloyd_max_codebook: no convergence");
  const double s = 1.0 / std::sqrt((double)head_dim);
  const int L = 1 << bits;
  for (int i = 0; i < L; ++i) centroids[i] = c[i] * s;
  for (int i = 0; i < L - 1; ++i) boundaries[i] = b[i] * s;
  return TQ_OK;
}
