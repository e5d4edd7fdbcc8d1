// Ridge solve on the GPU from the device sums, fp64 throughout.
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.2 ("The ridge map", "Fitting"): with X and Y centred,
// A = Y^T X (X^T X + alpha I)^(-1), b = mu_Y - A mu_X and
// alpha = lambda * tr(Xc^T Xc) / d_in.  From the running sums:
//   C = Sxx - n mu_X mu_X^T + alpha I   (d_in x d_in, symmetric positive definite)
//   R = Sxy - n mu_X mu_Y^T             (d_in x d_out)
//   C W = R,  A = W^T,  b = mu_Y - W^T mu_X.
// (RF_RIDGE_RAW: no centring, alpha = lambda, b = 0.)
//
// C is factored C = L L^T by a right-looking blocked Cholesky with 64 x 64
// blocks, then L Z = R and L^T W = Z are solved block row by block row.  Per
// block step: the diagonal block is factored by one workgroup in LDS, the
// blocks below it are solved against it (one workgroup per block), and the
// trailing matrix takes a rank-64 update; the two triangular solves take the
// same shape, with the right-hand side's 64-column blocks in parallel.  The
// updates are 64 x 64 x 64 products on v_mfma_f64_16x16x4_f64 (lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 v + l / 16][l % 16]).
// Every sum runs in a fixed order: the result is bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "rf_solve.h"

namespace rf {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

constexpr int kB = 64;        // block size
constexpr int kLd = kB + 1;   // LDS row length in doubles (odd: rows fall in different banks)

struct SolveArgs {
  const double* sxx;  // [d_in][d_in], entries with column >= row
  const double* sxy;  // [d_in][d_out]
  const double* sx;   // [d_in]
  const double* sy;   // [d_out]
  double n;
  int d_in, d_out, raw;
  double lambda;
  double* c;          // [d_in][d_in], lower triangle used
  double* r;          // [d_in][d_out]
  double* mx;         // [d_in]
  double* my;         // [d_out]
  int* flag;          // set to 1 when a pivot is not positive
};

// mu = s / n (zero when raw), and the flag cleared.
__global__ void __launch_bounds__(256) means_kernel(const SolveArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *a.flag = 0;
  if (i < a.d_in) a.mx[i] = a.raw ? 0.0 : a.sx[i] / a.n;
  if (i < a.d_out) a.my[i] = a.raw ? 0.0 : a.sy[i] / a.n;
}

// C[i][k] for the block-lower part (block of k <= block of i), R[i][j].
__global__ void __launch_bounds__(256) form_kernel(const SolveArgs a) {
  const int i = blockIdx.y;
  for (int k = blockIdx.x * 256 + threadIdx.x; k < a.d_in + a.d_out; k += gridDim.x * 256) {
    if (k < a.d_in) {
      if (k / kB > i / kB) continue;
      const int lo = min(i, k), hi = max(i, k);
      a.c[static_cast<size_t>(i) * a.d_in + k] =
          a.sxx[static_cast<size_t>(lo) * a.d_in + hi] - a.n * a.mx[i] * a.mx[k];
    } else {
      const int j = k - a.d_in;
      a.r[static_cast<size_t>(i) * a.d_out + j] = a.sxy[static_cast<size_t>(i) * a.d_out + j] - a.n * a.mx[i] * a.my[j];
    }
  }
}

// alpha = lambda * tr(C) / d_in (lambda when raw), added to C's diagonal.
// One workgroup: strided partial sums, then a fixed tree.
__global__ void __launch_bounds__(256) ridge_diag_kernel(const SolveArgs a) {
  __shared__ double part[256];
  double t = 0.0;
  for (int i = threadIdx.x; i < a.d_in; i += 256) t += a.c[static_cast<size_t>(i) * a.d_in + i];
  part[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const double alpha = a.raw ? a.lambda : a.lambda * part[0] / a.d_in;
  for (int i = threadIdx.x; i < a.d_in; i += 256) a.c[static_cast<size_t>(i) * a.d_in + i] += alpha;
}

// Cholesky of diagonal block k in place (its lower triangle).
__global__ void __launch_bounds__(256) potrf_kernel(double* c, int d, int k, int* flag) {
  __shared__ double s[kB * kLd];
  double* blk = c + (static_cast<size_t>(k) * kB) * d + k * kB;
  for (int e = threadIdx.x; e < kB * kB; e += 256) {
    const int r = e / kB, q = e % kB;
    s[r * kLd + q] = blk[static_cast<size_t>(r) * d + q];
  }
  __syncthreads();
  for (int j = 0; j < kB; ++j) {
    // column j: its pivot (thread 0), then the entries below it
    if (threadIdx.x == 0) {
      double v = s[j * kLd + j];
      for (int p = 0; p < j; ++p) v -= s[j * kLd + p] * s[j * kLd + p];
      if (!(v > 0.0)) {
        *flag = 1;
        v = 1.0;  // keep going with finite values; the call reports the failure
      }
      s[j * kLd + j] = sqrt(v);
    }
    __syncthreads();
    const int i = j + 1 + static_cast<int>(threadIdx.x);
    if (i < kB) {
      double v = s[i * kLd + j];
      for (int p = 0; p < j; ++p) v -= s[i * kLd + p] * s[j * kLd + p];
      s[i * kLd + j] = v / s[j * kLd + j];
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < kB * kB; e += 256) {
    const int r = e / kB, q = e % kB;
    if (q <= r) blk[static_cast<size_t>(r) * d + q] = s[r * kLd + q];
  }
}

// Block (k + 1 + blockIdx.x, k) := B L_kk^-T: row r of B solves x L_kk^T = b
// by forward substitution (one thread per row).
__global__ void __launch_bounds__(64) trsm_panel_kernel(double* c, int d, int k) {
  __shared__ double l[kB * kLd];
  __shared__ double b[kB * kLd];
  const int i = k + 1 + blockIdx.x;
  const double* lk = c + (static_cast<size_t>(k) * kB) * d + k * kB;
  double* bk = c + (static_cast<size_t>(i) * kB) * d + k * kB;
  for (int e = threadIdx.x; e < kB * kB; e += 64) {
    const int r = e / kB, q = e % kB;
    l[r * kLd + q] = q <= r ? lk[static_cast<size_t>(r) * d + q] : 0.0;
    b[r * kLd + q] = bk[static_cast<size_t>(r) * d + q];
  }
  __syncthreads();
  const int r = threadIdx.x;
  for (int q = 0; q < kB; ++q) {
    double v = b[r * kLd + q];
    for (int p = 0; p < q; ++p) v -= b[r * kLd + p] * l[q * kLd + p];
    b[r * kLd + q] = v / l[q * kLd + q];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kB * kB; e += 64) {
    const int rr = e / kB, q = e % kB;
    bk[static_cast<size_t>(rr) * d + q] = b[rr * kLd + q];
  }
}

// Block row k of the right-hand side: forward (FWD: L_kk z = r) or backward
// (L_kk^T w = z) substitution, one thread per column.
template <bool FWD>
__global__ void __launch_bounds__(256) trsv_rows_kernel(const double* c, int d, double* rhs, int d_out, int k) {
  __shared__ double l[kB * kLd];
  const double* lk = c + (static_cast<size_t>(k) * kB) * d + k * kB;
  for (int e = threadIdx.x; e < kB * kB; e += 256) {
    const int r = e / kB, q = e % kB;
    l[r * kLd + q] = q <= r ? lk[static_cast<size_t>(r) * d + q] : 0.0;
  }
  __syncthreads();
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= d_out) return;
  double* x = rhs + (static_cast<size_t>(k) * kB) * d_out + col;
  double v[kB];
#pragma unroll
  for (int r = 0; r < kB; ++r) v[r] = x[static_cast<size_t>(r) * d_out];
  if (FWD) {
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      double t = v[r];
#pragma unroll
      for (int p = 0; p < r; ++p) t -= l[r * kLd + p] * v[p];
      v[r] = t / l[r * kLd + r];
    }
  } else {
#pragma unroll
    for (int r = kB - 1; r >= 0; --r) {
      double t = v[r];
#pragma unroll
      for (int p = r + 1; p < kB; ++p) t -= l[p * kLd + r] * v[p];
      v[r] = t / l[r * kLd + r];
    }
  }
#pragma unroll
  for (int r = 0; r < kB; ++r) x[static_cast<size_t>(r) * d_out] = v[r];
}

// D -= P Q on 64 x 64 blocks with fp64 MFMA; P and Q are staged in LDS as
// P[row][p] and Q[p][col] (each mode fills them from its own layout).
//   MODE 0 (Cholesky update, step k): C[i][j] -= C[i][k] C[j][k]^T, k < j <= i
//   MODE 1 (forward, step k):         R[i][cb] -= C[i][k] R[k][cb],  i > k
//   MODE 2 (backward, step k):        R[i][cb] -= C[k][i]^T R[k][cb], i < k
template <int MODE>
__global__ void __launch_bounds__(256) update_kernel(double* c, int d, double* rhs, int d_out, int k) {
  __shared__ double ps[kB * kLd];
  __shared__ double qs[kB * kLd];
  int i, j;
  double* dst;
  int ldd;
  const double *p_src, *q_src;
  int ldp, ldq;
  if (MODE == 0) {
    i = k + 1 + blockIdx.y;
    j = k + 1 + blockIdx.x;
    if (j > i) return;  // (whole workgroup)
    dst = c + (static_cast<size_t>(i) * kB) * d + j * kB;
    ldd = d;
    p_src = c + (static_cast<size_t>(i) * kB) * d + k * kB;
    q_src = c + (static_cast<size_t>(j) * kB) * d + k * kB;  // used transposed
    ldp = ldq = d;
  } else {
    i = MODE == 1 ? k + 1 + blockIdx.y : blockIdx.y;
    j = blockIdx.x;  // column block of the right-hand side
    dst = rhs + (static_cast<size_t>(i) * kB) * d_out + j * kB;
    ldd = d_out;
    p_src = MODE == 1 ? c + (static_cast<size_t>(i) * kB) * d + k * kB   // L_ik
                      : c + (static_cast<size_t>(k) * kB) * d + i * kB;  // L_ki, used transposed
    ldp = d;
    q_src = rhs + (static_cast<size_t>(k) * kB) * d_out + j * kB;
    ldq = d_out;
  }
  for (int e = threadIdx.x; e < kB * kB; e += 256) {
    const int r = e / kB, q = e % kB;
    const double pv = p_src[static_cast<size_t>(r) * ldp + q];
    const double qv = q_src[static_cast<size_t>(r) * ldq + q];
    if (MODE == 2) ps[q * kLd + r] = pv; else ps[r * kLd + q] = pv;
    if (MODE == 0) qs[q * kLd + r] = qv; else qs[r * kLd + q] = qv;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int l16 = lane & 15, lk = lane >> 4;
  d4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int p = 0; p < kB; p += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) av[a] = ps[(wr + 16 * a + l16) * kLd + p + lk];
#pragma unroll
    for (int b = 0; b < 2; ++b) bv[b] = qs[(p + lk) * kLd + wc + 16 * b + l16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wr + 16 * a + 4 * v + lk, col = wc + 16 * b + l16;
        dst[static_cast<size_t>(row) * ldd + col] -= acc[a][b][v];
      }
}

// A[j][i] = float(W[i][j]) through a 32 x 32 LDS tile; b[j] = my[j] - sum_i W[i][j] mx[i]
// in increasing i (b = 0 when raw, since then my = mx = 0).
__global__ void __launch_bounds__(256) transpose_out_kernel(const double* w, int d_in, int d_out, float* a) {
  __shared__ float t[32][33];
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) t[r][tx] = static_cast<float>(w[static_cast<size_t>(i0 + r) * d_out + j0 + tx]);
  __syncthreads();
  for (int r = ty; r < 32; r += 8) a[static_cast<size_t>(j0 + r) * d_in + i0 + tx] = t[tx][r];
}

__global__ void __launch_bounds__(256) offset_kernel(const double* w, const double* mx, const double* my, int d_in,
                                                     int d_out, float* b) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_out) return;
  double v = my[j];
  for (int i = 0; i < d_in; ++i) v -= w[static_cast<size_t>(i) * d_out + j] * mx[i];
  b[j] = static_cast<float>(v);
}

}  // namespace

size_t ridge_solve_workspace_bytes(int d_in, int d_out) {
  const size_t up = 256;
  auto r = [&](size_t v) { return (v + up - 1) / up * up; };
  return r(sizeof(double) * static_cast<size_t>(d_in) * d_in) + r(sizeof(double) * static_cast<size_t>(d_in) * d_out) +
         r(sizeof(double) * d_in) + r(sizeof(double) * d_out) + up;
}

hipError_t ridge_solve_enqueue(const RidgeSolveIn& in, double lambda, bool raw, float* a_out, float* b_out, void* ws,
                               int** flag_out, hipStream_t s) {
  const int di = in.d_in, dout = in.d_out;
  const size_t up = 256;
  auto r = [&](size_t v) { return (v + up - 1) / up * up; };
  char* p = static_cast<char*>(ws);
  SolveArgs a{};
  a.sxx = in.sxx;
  a.sxy = in.sxy;
  a.sx = in.sx;
  a.sy = in.sy;
  a.n = static_cast<double>(in.n);
  a.d_in = di;
  a.d_out = dout;
  a.raw = raw ? 1 : 0;
  a.lambda = lambda;
  a.c = reinterpret_cast<double*>(p);
  p += r(sizeof(double) * static_cast<size_t>(di) * di);
  a.r = reinterpret_cast<double*>(p);
  p += r(sizeof(double) * static_cast<size_t>(di) * dout);
  a.mx = reinterpret_cast<double*>(p);
  p += r(sizeof(double) * di);
  a.my = reinterpret_cast<double*>(p);
  p += r(sizeof(double) * dout);
  a.flag = reinterpret_cast<int*>(p);
  *flag_out = a.flag;

  hipLaunchKernelGGL(means_kernel, dim3((std::max(di, dout) + 255) / 256), dim3(256), 0, s, a);
  hipLaunchKernelGGL(form_kernel, dim3((di + dout + 255) / 256, di), dim3(256), 0, s, a);
  hipLaunchKernelGGL(ridge_diag_kernel, dim3(1), dim3(256), 0, s, a);
  const int T = di / kB, TC = dout / kB;
  for (int k = 0; k < T; ++k) {
    hipLaunchKernelGGL(potrf_kernel, dim3(1), dim3(256), 0, s, a.c, di, k, a.flag);
    if (k + 1 < T) {
      hipLaunchKernelGGL(trsm_panel_kernel, dim3(T - k - 1), dim3(64), 0, s, a.c, di, k);
      hipLaunchKernelGGL((update_kernel<0>), dim3(T - k - 1, T - k - 1), dim3(256), 0, s, a.c, di, a.r, dout, k);
    }
  }
  for (int k = 0; k < T; ++k) {
    hipLaunchKernelGGL((trsv_rows_kernel<true>), dim3((dout + 255) / 256), dim3(256), 0, s, a.c, di, a.r, dout, k);
    if (k + 1 < T)
      hipLaunchKernelGGL((update_kernel<1>), dim3(TC, T - k - 1), dim3(256), 0, s, a.c, di, a.r, dout, k);
  }
  for (int k = T - 1; k >= 0; --k) {
    hipLaunchKernelGGL((trsv_rows_kernel<false>), dim3((dout + 255) / 256), dim3(256), 0, s, a.c, di, a.r, dout, k);
    if (k > 0) hipLaunchKernelGGL((update_kernel<2>), dim3(TC, k), dim3(256), 0, s, a.c, di, a.r, dout, k);
  }
  hipLaunchKernelGGL(transpose_out_kernel, dim3(dout / 32, di / 32), dim3(256), 0, s, a.r, di, dout, a_out);
  hipLaunchKernelGGL(offset_kernel, dim3((dout + 255) / 256), dim3(256), 0, s, a.r, a.mx, a.my, di, dout, b_out);
  return hipGetLastError();
}

}  // namespace rf
