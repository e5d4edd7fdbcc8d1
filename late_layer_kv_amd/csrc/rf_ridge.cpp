// Closed-form ridge map on the host, float64 throughout (validation of maps).
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.2: centre X and Y by their means, A = Y^T X (X^T X + alpha I)^(-1),
// b = mu_Y - A mu_X, only A penalised, alpha = lambda tr(Xc^T Xc) / d_in.
// "Fitting": X^T X, X^T Y and the two means, summed over documents, lead to the
// same maps as one solve over all rows; a different lambda costs one more
// solve, not another pass over the data.  The solve is a Cholesky factorisation of the symmetric positive
// definite matrix Xc^T Xc + alpha I followed by two triangular solves per
// output column.
#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/rf.h"
#include "rf_error.h"
#include "rf_ridge_internal.h"

namespace {
rf_status rfail(rf_status st, const char* msg) {
  rf::set_last_error(msg);
  return st;
}
}  // namespace

struct rf_ridge_acc {
  int d_in = 0, d_out = 0;
  long long n = 0;
  std::vector<double> sx, sy, sxx, sxy;  // sxx [d_in][d_in], sxy [d_in][d_out]
};

void rf::ridge_acc_dims(const rf_ridge_acc* a, int* d_in, int* d_out) {
  *d_in = a->d_in;
  *d_out = a->d_out;
}

void rf::ridge_acc_add_sums(rf_ridge_acc* a, const double* sxx, const double* sxy, const double* sx,
                            const double* sy, int64_t n) {
  const int di = a->d_in, dout = a->d_out;
  for (int i = 0; i < di; ++i) {
    a->sx[i] += sx[i];
    for (int k = i; k < di; ++k) a->sxx[static_cast<size_t>(i) * di + k] += sxx[static_cast<size_t>(i) * di + k];
    for (int j = 0; j < dout; ++j) a->sxy[static_cast<size_t>(i) * dout + j] += sxy[static_cast<size_t>(i) * dout + j];
  }
  for (int j = 0; j < dout; ++j) a->sy[j] += sy[j];
  a->n += n;
}

extern "C" {

rf_status rf_ridge_acc_create(int32_t d_in, int32_t d_out, rf_ridge_acc** out) {
  if (!out) return rfail(RF_E_ARG, "out is null");
  *out = nullptr;
  if (d_in < 1 || d_out < 1) return rfail(RF_E_ARG, "d_in and d_out must be >= 1");
  rf_ridge_acc* a = new (std::nothrow) rf_ridge_acc();
  if (!a) return rfail(RF_E_ARG, "out of host memory");
  a->d_in = d_in;
  a->d_out = d_out;
  a->sx.assign(d_in, 0.0);
  a->sy.assign(d_out, 0.0);
  a->sxx.assign(static_cast<size_t>(d_in) * d_in, 0.0);
  a->sxy.assign(static_cast<size_t>(d_in) * d_out, 0.0);
  *out = a;
  return RF_OK;
}

void rf_ridge_acc_destroy(rf_ridge_acc* a) { delete a; }

rf_status rf_ridge_acc_add(rf_ridge_acc* a, const float* x, const float* y, int64_t n) {
  if (!a) return rfail(RF_E_ARG, "accumulator is null");
  if (n < 0) return rfail(RF_E_ARG, "n must be >= 0");
  if (n > 0 && (!x || !y)) return rfail(RF_E_ARG, "x or y is null");
  const int di = a->d_in, dout = a->d_out;
  std::vector<double> xr(di), yr(dout);
  for (int64_t r = 0; r < n; ++r) {
    const float* xp = x + r * di;
    const float* yp = y + r * dout;
    for (int i = 0; i < di; ++i) xr[i] = xp[i];
    for (int j = 0; j < dout; ++j) yr[j] = yp[j];
    for (int i = 0; i < di; ++i) {
      a->sx[i] += xr[i];
      const double xi = xr[i];
      double* srow = &a->sxx[static_cast<size_t>(i) * di];
      for (int k = i; k < di; ++k) srow[k] += xi * xr[k];  // upper triangle
      double* yrow = &a->sxy[static_cast<size_t>(i) * dout];
      for (int j = 0; j < dout; ++j) yrow[j] += xi * yr[j];
    }
    for (int j = 0; j < dout; ++j) a->sy[j] += yr[j];
  }
  a->n += n;
  return RF_OK;
}

rf_status rf_ridge_acc_sums(const rf_ridge_acc* a, double* sxx, double* sxy, double* sx, double* sy, int64_t* n) {
  if (!a) return rfail(RF_E_ARG, "accumulator is null");
  const int di = a->d_in, dout = a->d_out;
  if (sxx)
    for (int i = 0; i < di; ++i)
      for (int k = i; k < di; ++k) {
        const double v = a->sxx[static_cast<size_t>(i) * di + k];
        sxx[static_cast<size_t>(i) * di + k] = v;
        sxx[static_cast<size_t>(k) * di + i] = v;
      }
  if (sxy) std::copy(a->sxy.begin(), a->sxy.end(), sxy);
  if (sx) std::copy(a->sx.begin(), a->sx.end(), sx);
  if (sy) std::copy(a->sy.begin(), a->sy.end(), sy);
  if (n) *n = a->n;
  return RF_OK;
}

rf_status rf_ridge_solve(const rf_ridge_acc* a, double lambda, int32_t flags, float* A, float* b) {
  if (!a || !A || !b) return rfail(RF_E_ARG, "null argument");
  if (flags & ~RF_RIDGE_RAW) return rfail(RF_E_ARG, "unknown ridge flag");
  if (a->n < 1) return rfail(RF_E_ARG, "no rows accumulated");
  if (!(lambda >= 0.0)) return rfail(RF_E_ARG, "lambda must be >= 0");
  const int di = a->d_in, dout = a->d_out;
  const bool raw = flags & RF_RIDGE_RAW;
  const double n = static_cast<double>(a->n);
  std::vector<double> mx(di, 0.0), my(dout, 0.0);
  if (!raw) {
    for (int i = 0; i < di; ++i) mx[i] = a->sx[i] / n;
    for (int j = 0; j < dout; ++j) my[j] = a->sy[j] / n;
  }
  // C = Sxx - n mx mx^T (full symmetric), R = Sxy - n mx my^T
  std::vector<double> c(static_cast<size_t>(di) * di), rhs(static_cast<size_t>(di) * dout);
  for (int i = 0; i < di; ++i)
    for (int k = i; k < di; ++k) {
      const double v = a->sxx[static_cast<size_t>(i) * di + k] - n * mx[i] * mx[k];
      c[static_cast<size_t>(i) * di + k] = v;
      c[static_cast<size_t>(k) * di + i] = v;
    }
  for (int i = 0; i < di; ++i)
    for (int j = 0; j < dout; ++j)
      rhs[static_cast<size_t>(i) * dout + j] = a->sxy[static_cast<size_t>(i) * dout + j] - n * mx[i] * my[j];
  double alpha = lambda;
  if (!raw) {
    double tr = 0.0;
    for (int i = 0; i < di; ++i) tr += c[static_cast<size_t>(i) * di + i];
    alpha = lambda * tr / di;
  }
  for (int i = 0; i < di; ++i) c[static_cast<size_t>(i) * di + i] += alpha;
  // Cholesky C = L L^T, L stored in the lower triangle of c.
  for (int j = 0; j < di; ++j) {
    double d = c[static_cast<size_t>(j) * di + j];
    for (int k = 0; k < j; ++k) d -= c[static_cast<size_t>(j) * di + k] * c[static_cast<size_t>(j) * di + k];
    if (!(d > 0.0)) return rfail(RF_E_LINALG, "ridge system is not positive definite");
    const double ljj = std::sqrt(d);
    c[static_cast<size_t>(j) * di + j] = ljj;
    for (int i = j + 1; i < di; ++i) {
      double v = c[static_cast<size_t>(i) * di + j];
      for (int k = 0; k < j; ++k) v -= c[static_cast<size_t>(i) * di + k] * c[static_cast<size_t>(j) * di + k];
      c[static_cast<size_t>(i) * di + j] = v / ljj;
    }
  }
  // For every output column: L z = r, L^T w = z; W[:, j] = w, A[j][:] = w.
  std::vector<double> z(di);
  for (int j = 0; j < dout; ++j) {
    for (int i = 0; i < di; ++i) {
      double v = rhs[static_cast<size_t>(i) * dout + j];
      for (int k = 0; k < i; ++k) v -= c[static_cast<size_t>(i) * di + k] * z[k];
      z[i] = v / c[static_cast<size_t>(i) * di + i];
    }
    for (int i = di - 1; i >= 0; --i) {
      double v = z[i];
      for (int k = i + 1; k < di; ++k) v -= c[static_cast<size_t>(k) * di + i] * z[k];
      z[i] = v / c[static_cast<size_t>(i) * di + i];
    }
    double bj = my[j];
    for (int i = 0; i < di; ++i) {
      A[static_cast<size_t>(j) * di + i] = static_cast<float>(z[i]);
      bj -= z[i] * mx[i];
    }
    b[j] = raw ? 0.0f : static_cast<float>(bj);
  }
  return RF_OK;
}

rf_status rf_ridge_fit(const float* x, const float* y, int64_t n, int32_t d_in, int32_t d_out, double lambda,
                       int32_t flags, float* A, float* b) {
  rf_ridge_acc* acc = nullptr;
  rf_status st = rf_ridge_acc_create(d_in, d_out, &acc);
  if (st != RF_OK) return st;
  st = rf_ridge_acc_add(acc, x, y, n);
  if (st == RF_OK) st = rf_ridge_solve(acc, lambda, flags, A, b);
  rf_ridge_acc_destroy(acc);
  return st;
}

}  // extern "C"
