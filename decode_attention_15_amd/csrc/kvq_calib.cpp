// Host side of the C ABI: the attention-aware calibration covariances and their eigenbasis, from which
// the OSCAR rotation R = U·H·P_br is composed ([OSCAR] summary page §3.2 offline steps 2-3, §3.4.2
// Factor 1: U diagonalizes the covariance, its columns ordered by decreasing eigenvalue).
//
// Everything here is fp64 on the host; none of it runs per decode step.
#include <math.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "kvq_internal.h"

using namespace kvq;

namespace {

bool all_finite(const float* x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return false;
  return true;
}

// Cyclic Jacobi eigenvalue iteration on the symmetric n x n row-major matrix A (overwritten; its diagonal
// ends as the eigenvalues).  V (row-major) accumulates the plane rotations, so that on return
// A_in = V diag(A) V^T.  Each rotation in the (p, q) plane is chosen to zero A[p][q]:
//   theta = (A_qq - A_pp) / (2 A_pq),  t = sign(theta) / (|theta| + sqrt(theta^2 + 1)),
//   c = 1 / sqrt(t^2 + 1),  s = t c,  A <- J^T A J, V <- V J with J_pp = J_qq = c, J_pq = s, J_qp = -s.
// Sweeps stop once the off-diagonal mass is below 1e-30 of the diagonal's (or exactly zero).
bool jacobi_eigen(std::vector<double>& A, std::vector<double>& V, int n) {
  V.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) V[(size_t)i * n + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, dia = 0.0;
    for (int p = 0; p < n; ++p) {
      dia += A[(size_t)p * n + p] * A[(size_t)p * n + p];
      for (int q = p + 1; q < n; ++q) off += A[(size_t)p * n + q] * A[(size_t)p * n + q];
    }
    if (off == 0.0 || off <= 1e-30 * dia) return true;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = A[(size_t)p * n + q];
        if (apq == 0.0) continue;
        const double theta = (A[(size_t)q * n + q] - A[(size_t)p * n + p]) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; ++k) {  // columns p, q: A J
          const double akp = A[(size_t)k * n + p], akq = A[(size_t)k * n + q];
          A[(size_t)k * n + p] = c * akp - s * akq;
          A[(size_t)k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {  // rows p, q: J^T (A J)
          const double apk = A[(size_t)p * n + k], aqk = A[(size_t)q * n + k];
          A[(size_t)p * n + k] = c * apk - s * aqk;
          A[(size_t)q * n + k] = s * apk + c * aqk;
        }
        A[(size_t)p * n + q] = A[(size_t)q * n + p] = 0.0;
        for (int k = 0; k < n; ++k) {  // V J
          const double vkp = V[(size_t)k * n + p], vkq = V[(size_t)k * n + q];
          V[(size_t)k * n + p] = c * vkp - s * vkq;
          V[(size_t)k * n + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  return false;
}

}  // namespace

extern "C" {

int kvq_query_covariance(const float* q_host, int64_t n_rows, double* C_out_host) {
  if (!q_host || !C_out_host || n_rows <= 0) return KVQ_EINVAL;
  if (!all_finite(q_host, (size_t)n_rows * D)) return KVQ_EINVAL;
  std::vector<double> C((size_t)D * D, 0.0);
  for (int64_t n = 0; n < n_rows; ++n) {
    const float* q = q_host + (size_t)n * D;
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) C[(size_t)i * D + j] += (double)q[i] * (double)q[j];
  }
  for (size_t e = 0; e < C.size(); ++e) C_out_host[e] = C[e] / (double)n_rows;
  return KVQ_OK;
}

int kvq_score_value_covariance(const float* v_host, int64_t n_keys, const float* s_host, int64_t n_rows,
                               double* C_out_host) {
  if (!v_host || !s_host || !C_out_host || n_keys <= 0 || n_rows <= 0) return KVQ_EINVAL;
  if (!all_finite(v_host, (size_t)n_keys * D) || !all_finite(s_host, (size_t)n_rows * n_keys)) return KVQ_EINVAL;
  std::vector<double> C((size_t)D * D, 0.0), sv(D);
  for (int64_t n = 0; n < n_rows; ++n) {
    std::fill(sv.begin(), sv.end(), 0.0);  // row n of S V, summed over keys in increasing order
    for (int64_t k = 0; k < n_keys; ++k) {
      const double w = s_host[(size_t)n * n_keys + k];
      const float* v = v_host + (size_t)k * D;
      for (int j = 0; j < D; ++j) sv[j] += w * (double)v[j];
    }
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) C[(size_t)i * D + j] += sv[i] * sv[j];
  }
  for (size_t e = 0; e < C.size(); ++e) C_out_host[e] = C[e] / (double)n_rows;
  return KVQ_OK;
}

int kvq_eigenbasis(const double* C_host, double* U_out_host, double* lambda_out_host) {
  if (!C_host || !U_out_host || !lambda_out_host) return KVQ_EINVAL;
  double scale = 0.0;
  for (int e = 0; e < D * D; ++e) {
    if (!isfinite(C_host[e])) return KVQ_EINVAL;
    scale = fmax(scale, fabs(C_host[e]));
  }
  for (int i = 0; i < D; ++i)
    for (int j = i + 1; j < D; ++j)
      if (fabs(C_host[i * D + j] - C_host[j * D + i]) > 1e-12 * scale) return KVQ_EINVAL;  // not symmetric
  std::vector<double> A(C_host, C_host + D * D), V;
  if (!jacobi_eigen(A, V, D)) return KVQ_ERANGE;
  // order by decreasing eigenvalue (ties by index), then fix each column's sign: entry of largest
  // magnitude (first such index) positive
  std::vector<int> order(D);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return A[(size_t)a * D + a] > A[(size_t)b * D + b]; });
  for (int k = 0; k < D; ++k) {
    const int c = order[k];
    lambda_out_host[k] = A[(size_t)c * D + c];
    int imax = 0;
    for (int i = 1; i < D; ++i)
      if (fabs(V[(size_t)i * D + c]) > fabs(V[(size_t)imax * D + c])) imax = i;
    const double sg = V[(size_t)imax * D + c] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < D; ++i) U_out_host[i * D + k] = sg * V[(size_t)i * D + c];
  }
  return KVQ_OK;
}

int kvq_build_oscar_rotation_from_covariance(const double* C_host, double* R_out_host) {
  if (!C_host || !R_out_host) return KVQ_EINVAL;
  std::vector<double> U((size_t)D * D), lam(D);
  const int st = kvq_eigenbasis(C_host, U.data(), lam.data());
  if (st != KVQ_OK) return st;
  return kvq_compose_oscar_rotation(U.data(), R_out_host);
}

}  // extern "C"
