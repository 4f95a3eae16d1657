// DRRQR channel selection, host code: which d_k' of the d_k key/query
// channels a pruned layer keeps.
//
// "On State Reduction in Linear Attention" (reading notes), paper Sec. 3.4 with
// its Algorithm 2 and App. B.2: on calibration samples M = [K_cal; Q_cal]
// (2N x n, one column per channel), a QR with column pivoting gives an
// initial permutation M P = Q [[A, B], [0, C]] (A: k x k); then, with
// U = A^{-1} B, omega_i = 1 / ||row i of A^{-1}||, gamma_j = ||column j of
// C|| and rho_ij = sqrt(U_ij^2 + (gamma_j / omega_i)^2), the selected column
// i and candidate j of the largest rho_ij > f trade places and the factor is
// re-triangularised, until every rho_ij <= f (strong rank-revealing QR).
// rho_ij is the factor by which that trade would grow |det A|, so each
// trade grows the volume spanned by the kept columns by more than f.
//
// This is calibration-time work on an n x n factor (n = d_k = 128), not a
// per-token kernel: it runs on the host, in fp64.  The tall M is first
// reduced to its n x n triangular factor R0 (one Householder QR); the
// pivoted QR and every swap then work on R0, since column-pivoted QR and
// the swap test depend on M only through M^T M = R0^T R0.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gdn_launch.hpp"

namespace gdn {

namespace {

// Column-major n-column matrix with `ld` rows: element (r, c) at c * ld + r.
struct ColMat {
  int rows, cols;
  std::vector<double> a;
  ColMat(int r, int c) : rows(r), cols(c), a((size_t)r * c, 0.0) {}
  double& at(int r, int c) { return a[(size_t)c * rows + r]; }
  double at(int r, int c) const { return a[(size_t)c * rows + r]; }
  double* col(int c) { return &a[(size_t)c * rows]; }
  void swap_cols(int i, int j) {
    if (i == j) return;
    for (int r = 0; r < rows; ++r) {
      const double t = at(r, i);
      at(r, i) = at(r, j);
      at(r, j) = t;
    }
  }
};

// Householder step on column c, rows c..rows-1: reduces X(c+1.., c) to zero
// and applies the reflection to columns c+1..cols-1.
void householder_step(ColMat& X, int c) {
  const int m = X.rows - c;
  double* x = X.col(c) + c;
  double nx = 0.0;
  for (int r = 0; r < m; ++r) nx += x[r] * x[r];
  nx = sqrt(nx);
  if (nx == 0.0) return;
  const double alpha = x[0] >= 0.0 ? -nx : nx;      // new diagonal element
  std::vector<double> v(x, x + m);
  v[0] -= alpha;
  double vv = 0.0;
  for (int r = 0; r < m; ++r) vv += v[r] * v[r];
  if (vv == 0.0) return;
  for (int j = c + 1; j < X.cols; ++j) {
    double* y = X.col(j) + c;
    double d = 0.0;
    for (int r = 0; r < m; ++r) d += v[r] * y[r];
    const double s = 2.0 * d / vv;
    for (int r = 0; r < m; ++r) y[r] -= s * v[r];
  }
  x[0] = alpha;
  for (int r = 1; r < m; ++r) x[r] = 0.0;
}

// The upper n x n triangle of X after Householder QR (optionally with
// column pivoting on the remaining column norms, recorded in perm).
ColMat triangular_factor(ColMat X, std::vector<int>* perm) {
  const int n = X.cols;
  for (int c = 0; c < n; ++c) {
    if (perm != nullptr) {
      int best = c;
      double bn = -1.0;
      for (int j = c; j < n; ++j) {
        double s = 0.0;
        for (int r = c; r < X.rows; ++r) s += X.at(r, j) * X.at(r, j);
        if (s > bn) {
          bn = s;
          best = j;
        }
      }
      X.swap_cols(c, best);
      const int t = (*perm)[c];
      (*perm)[c] = (*perm)[best];
      (*perm)[best] = t;
    }
    householder_step(X, c);
  }
  ColMat R(n, n);
  for (int j = 0; j < n; ++j)
    for (int r = 0; r <= j && r < X.rows; ++r) R.at(r, j) = X.at(r, j);
  return R;
}

}  // namespace

// Returns 0, or 1 when the pivoted factor shows rank(M) < k.
int drrqr_select(const double* M, int rows, int n, int k, double f, int max_swaps,
                 int* selected, int* swaps_out, double* rho_out) {
  // M row-major [rows][n] -> column-major copy
  ColMat X(rows, n);
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < n; ++c) X.at(r, c) = M[(size_t)r * n + c];
  ColMat R0 = triangular_factor(X, nullptr);
  std::vector<int> perm(n);
  for (int c = 0; c < n; ++c) perm[c] = c;
  ColMat R = triangular_factor(R0, &perm);
  if (!(fabs(R.at(k - 1, k - 1)) > 0.0)) return 1;   // rank(M) < k (or not finite)

  const int m = n - k;
  std::vector<double> Ainv((size_t)k * k), U((size_t)k * m), omega(k), gamma(m);
  int swaps = 0;
  double rmax = 0.0;
  for (;;) {
    // A^{-1} (upper triangular), column by column by back substitution
    for (int j = 0; j < k; ++j) {
      for (int i = k - 1; i >= 0; --i) {
        double s = (i == j) ? 1.0 : 0.0;
        for (int t = i + 1; t < k; ++t) s -= R.at(i, t) * Ainv[(size_t)t * k + j];
        Ainv[(size_t)i * k + j] = s / R.at(i, i);      // row-major: (i, j)
      }
    }
    for (int i = 0; i < k; ++i) {
      double s = 0.0;
      for (int j = 0; j < k; ++j) s += Ainv[(size_t)i * k + j] * Ainv[(size_t)i * k + j];
      omega[i] = 1.0 / sqrt(s);
      for (int j = 0; j < m; ++j) {
        double u = 0.0;
        for (int t = i; t < k; ++t) u += Ainv[(size_t)i * k + t] * R.at(t, k + j);
        U[(size_t)i * m + j] = u;
      }
    }
    for (int j = 0; j < m; ++j) {
      double s = 0.0;
      for (int r = k; r < n; ++r) s += R.at(r, k + j) * R.at(r, k + j);
      gamma[j] = sqrt(s);
    }
    int bi = 0, bj = 0;
    rmax = -1.0;
    for (int i = 0; i < k; ++i)
      for (int j = 0; j < m; ++j) {
        const double g = gamma[j] / omega[i];
        const double rho = sqrt(U[(size_t)i * m + j] * U[(size_t)i * m + j] + g * g);
        if (rho > rmax) {
          rmax = rho;
          bi = i;
          bj = j;
        }
      }
    if (!(rmax > f) || swaps >= max_swaps) break;
    R.swap_cols(bi, k + bj);
    const int t = perm[bi];
    perm[bi] = perm[k + bj];
    perm[k + bj] = t;
    R = triangular_factor(R, nullptr);
    ++swaps;
  }
  for (int i = 0; i < k; ++i) selected[i] = perm[i];
  if (swaps_out) *swaps_out = swaps;
  if (rho_out) *rho_out = rmax;
  return 0;
}

}  // namespace gdn
