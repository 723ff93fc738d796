// Least-squares fit of the Eq. 5 latency model (include/msa_latency.h).
//
// The five model terms of each sample form a row of the design matrix A
// (rows divided by the measured time for a relative fit).  Columns are scaled
// to unit 2-norm -- the terms differ by many orders of magnitude (1 against
// q2 * context) -- and the scaled system is solved by Householder QR, which
// avoids squaring the condition number as the normal equations would.  A
// diagonal element of R below 1e-10 of the largest means a coefficient is not
// determined by the samples.
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "msa.h"
#include "msa_latency.h"

namespace msa {
int set_error_msg(int code, const std::string& msg);
}

namespace {

constexpr int kTerms = 5;

void terms(double l1, double q1, double l2, double q2, double* t) {
  t[0] = 1.0;
  t[1] = q1 + q2;
  t[2] = l1 + l2;
  t[3] = q2 * (l1 + q1 + l2 + q2);
  t[4] = q1 * (l1 + q1);
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

}  // namespace

extern "C" {

int msa_latency_fit(const double* samples, int32_t n, int32_t relative, msa_latency_model* out) {
  using msa::set_error_msg;
  if (!samples || !out) return set_error_msg(MSA_ERR_INVALID_ARG, "samples or out is NULL");
  if (n < kTerms) return set_error_msg(MSA_ERR_INVALID_ARG, "need at least 5 samples");
  std::vector<double> A((size_t)n * kTerms), b(n);
  for (int32_t i = 0; i < n; ++i) {
    const double* s = samples + (size_t)i * 5;
    for (int j = 0; j < 4; ++j)
      if (!finite_nonneg(s[j])) return set_error_msg(MSA_ERR_INVALID_ARG, "sample " + std::to_string(i) +
                                                                              ": region sizes must be finite and >= 0");
    if (!std::isfinite(s[4]) || (relative && !(s[4] > 0.0)))
      return set_error_msg(MSA_ERR_INVALID_ARG, "sample " + std::to_string(i) + ": bad time");
    const double w = relative ? 1.0 / s[4] : 1.0;
    terms(s[0], s[1], s[2], s[3], &A[(size_t)i * kTerms]);
    for (int j = 0; j < kTerms; ++j) A[(size_t)i * kTerms + j] *= w;
    b[i] = s[4] * w;
  }
  // column scaling
  double scale[kTerms];
  for (int j = 0; j < kTerms; ++j) {
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += A[(size_t)i * kTerms + j] * A[(size_t)i * kTerms + j];
    if (!(ss > 0.0)) return set_error_msg(MSA_ERR_INVALID_ARG, "the samples do not determine all five coefficients");
    scale[j] = 1.0 / std::sqrt(ss);
    for (int32_t i = 0; i < n; ++i) A[(size_t)i * kTerms + j] *= scale[j];
  }
  std::vector<double> r(b);  // becomes Q^T b
  // Householder QR, column by column
  double diag[kTerms];
  for (int j = 0; j < kTerms; ++j) {
    double norm = 0.0;
    for (int32_t i = j; i < n; ++i) norm += A[(size_t)i * kTerms + j] * A[(size_t)i * kTerms + j];
    norm = std::sqrt(norm);
    const double ajj = A[(size_t)j * kTerms + j];
    const double alpha = ajj > 0 ? -norm : norm;
    diag[j] = alpha;
    // v = x - alpha e1, stored in place of column j (rows j..n-1)
    A[(size_t)j * kTerms + j] = ajj - alpha;
    double vnorm2 = 0.0;
    for (int32_t i = j; i < n; ++i) vnorm2 += A[(size_t)i * kTerms + j] * A[(size_t)i * kTerms + j];
    if (vnorm2 == 0.0) continue;  // column already reduced
    for (int c = j + 1; c < kTerms; ++c) {
      double dot = 0.0;
      for (int32_t i = j; i < n; ++i) dot += A[(size_t)i * kTerms + j] * A[(size_t)i * kTerms + c];
      const double f = 2.0 * dot / vnorm2;
      for (int32_t i = j; i < n; ++i) A[(size_t)i * kTerms + c] -= f * A[(size_t)i * kTerms + j];
    }
    double dot = 0.0;
    for (int32_t i = j; i < n; ++i) dot += A[(size_t)i * kTerms + j] * r[i];
    const double f = 2.0 * dot / vnorm2;
    for (int32_t i = j; i < n; ++i) r[i] -= f * A[(size_t)i * kTerms + j];
  }
  double dmax = 0.0;
  for (int j = 0; j < kTerms; ++j) dmax = std::fmax(dmax, std::fabs(diag[j]));
  for (int j = 0; j < kTerms; ++j)
    if (!(std::fabs(diag[j]) > 1e-10 * dmax))
      return set_error_msg(MSA_ERR_INVALID_ARG, "the samples do not determine all five coefficients");
  // back substitution: R x = (Q^T b)[0..4]; R's strict upper part is in A
  double x[kTerms];
  for (int j = kTerms - 1; j >= 0; --j) {
    double s = r[j];
    for (int c = j + 1; c < kTerms; ++c) s -= A[(size_t)j * kTerms + c] * x[c];
    x[j] = s / diag[j];
  }
  msa_latency_model m;
  std::memset(&m, 0, sizeof(m));
  for (int j = 0; j < kTerms; ++j) m.k[j] = x[j] * scale[j];
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    const double* s = samples + (size_t)i * 5;
    double t[kTerms];
    terms(s[0], s[1], s[2], s[3], t);
    double pred = 0.0;
    for (int j = 0; j < kTerms; ++j) pred += m.k[j] * t[j];
    const double res = relative ? (pred - s[4]) / s[4] : pred - s[4];
    ss += res * res;
  }
  m.rms = std::sqrt(ss / n);
  m.n = n;
  m.relative = relative ? 1 : 0;
  *out = m;
  return MSA_OK;
}

int msa_latency_eval(const msa_latency_model* model, double l1, double q1, double l2, double q2, double* t) {
  if (!model || !t) return msa::set_error_msg(MSA_ERR_INVALID_ARG, "model or t is NULL");
  double v[kTerms];
  terms(l1, q1, l2, q2, v);
  double s = 0.0;
  for (int j = 0; j < kTerms; ++j) s += model->k[j] * v[j];
  *t = s;
  return MSA_OK;
}

int msa_latency_delta_b(const msa_latency_model* model, double l1, double q1, double* dt) {
  if (!model || !dt) return msa::set_error_msg(MSA_ERR_INVALID_ARG, "model or dt is NULL");
  const double* k = model->k;
  *dt = k[4] * (l1 + 2.0 * q1) + (k[1] - k[2] + k[4]);
  return MSA_OK;
}

int msa_chunk_blocks(const msa_latency_model* model, double l1, double q1, double l2, int32_t remaining,
                     double budget, int32_t* chunk) {
  if (!model || !chunk) return msa::set_error_msg(MSA_ERR_INVALID_ARG, "model or chunk is NULL");
  if (remaining < 1) return msa::set_error_msg(MSA_ERR_INVALID_ARG, "remaining must be >= 1");
  if (!finite_nonneg(l1) || !finite_nonneg(q1) || !finite_nonneg(l2) || std::isnan(budget))
    return msa::set_error_msg(MSA_ERR_INVALID_ARG, "region sizes must be finite and >= 0, budget not NaN");
  // Scan from the largest candidate down: no monotonicity of the fitted model
  // is assumed (a fit may carry a negative coefficient).
  double t[kTerms];
  for (int32_t c = remaining; c >= 1; --c) {
    terms(l1, q1, l2, (double)c, t);
    double T = 0.0;
    for (int j = 0; j < kTerms; ++j) T += model->k[j] * t[j];
    if (T <= budget) {
      *chunk = c;
      return MSA_OK;
    }
  }
  *chunk = 1;
  return MSA_OK;
}

}  // extern "C"
