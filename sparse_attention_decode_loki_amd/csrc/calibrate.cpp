// Offline PCA calibration of key vectors (host only).
//
// The Loki pages state that the projection is calibrated offline and that
// queries and keys are PCA-projected (pages titled "Loki: Low-rank Keys for
// Efficient Sparse Attention", summary page, summary line and "Approach").
// PCA here: eigenvectors of the centred sample covariance (divisor n - 1),
// eigenvalues in descending order, each eigenvector's sign fixed so that its
// largest-magnitude component (lowest index among equal magnitudes) is
// positive.  Eigen-decomposition by the cyclic Jacobi method (Golub & Van
// Loan, "Matrix Computations", section 8.5: two-by-two symmetric Schur
// rotations swept over all off-diagonal pairs until the off-diagonal mass
// vanishes), all in float64.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "loki.h"

namespace {

// Zero A(p,q) of the symmetric matrix A (row-major, n x n) by a plane
// rotation J with J(p,p) = J(q,q) = c, J(p,q) = s, J(q,p) = -s, replacing A by
// J^T A J and V by V J.
void rotate_pair(std::vector<double>& A, std::vector<double>& V, int n, int p, int q) {
  const double apq = A[p * n + q];
  if (apq == 0.0) return;
  const double tau = (A[q * n + q] - A[p * n + p]) / (2.0 * apq);
  const double t = (tau >= 0.0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
  const double c = 1.0 / std::sqrt(1.0 + t * t);
  const double s = t * c;
  for (int k = 0; k < n; ++k) {  // A J: columns p and q
    const double akp = A[k * n + p], akq = A[k * n + q];
    A[k * n + p] = c * akp - s * akq;
    A[k * n + q] = s * akp + c * akq;
  }
  for (int k = 0; k < n; ++k) {  // J^T (A J): rows p and q
    const double apk = A[p * n + k], aqk = A[q * n + k];
    A[p * n + k] = c * apk - s * aqk;
    A[q * n + k] = s * apk + c * aqk;
  }
  A[p * n + q] = 0.0;
  A[q * n + p] = 0.0;
  for (int k = 0; k < n; ++k) {
    const double vkp = V[k * n + p], vkq = V[k * n + q];
    V[k * n + p] = c * vkp - s * vkq;
    V[k * n + q] = s * vkp + c * vkq;
  }
}

double off_diagonal_sq(const std::vector<double>& A, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (i != j) s += A[i * n + j] * A[i * n + j];
  return s;
}

}  // namespace

extern "C" int loki_calibrate(const float* keys, int64_t n, int32_t D, float* P_out,
                              double* eigvals_out) {
  if (!keys || !P_out || n < 2 || D < 1) return LOKI_EINVAL;
  const int d = D;
  std::vector<double> mu(d, 0.0);
  for (int64_t i = 0; i < n; ++i)
    for (int m = 0; m < d; ++m) mu[m] += keys[i * d + m];
  for (int m = 0; m < d; ++m) mu[m] /= static_cast<double>(n);

  std::vector<double> C(static_cast<size_t>(d) * d, 0.0), x(d);
  for (int64_t i = 0; i < n; ++i) {
    for (int m = 0; m < d; ++m) x[m] = keys[i * d + m] - mu[m];
    for (int a = 0; a < d; ++a) {
      const double xa = x[a];
      double* row = &C[static_cast<size_t>(a) * d];
      for (int b = a; b < d; ++b) row[b] += xa * x[b];
    }
  }
  const double inv = 1.0 / static_cast<double>(n - 1);
  for (int a = 0; a < d; ++a)
    for (int b = a; b < d; ++b) {
      C[a * d + b] *= inv;
      C[b * d + a] = C[a * d + b];
    }

  double total = 0.0;
  for (double c : C) total += c * c;
  std::vector<double> V(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) V[i * d + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    if (off_diagonal_sq(C, d) <= 1e-32 * total) break;
    for (int p = 0; p < d - 1; ++p)
      for (int q = p + 1; q < d; ++q) rotate_pair(C, V, d, p, q);
  }

  std::vector<int> order(d);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return C[a * d + a] > C[b * d + b]; });
  for (int c = 0; c < d; ++c) {
    const int src = order[c];
    int imax = 0;
    for (int m = 1; m < d; ++m)
      if (std::fabs(V[m * d + src]) > std::fabs(V[imax * d + src])) imax = m;
    const double sgn = V[imax * d + src] < 0.0 ? -1.0 : 1.0;
    for (int m = 0; m < d; ++m) P_out[m * d + c] = static_cast<float>(sgn * V[m * d + src]);
    if (eigvals_out) eigvals_out[c] = C[src * d + src];
  }
  return LOKI_OK;
}
