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
// block step: one workgroup factors the diagonal block in LDS and forms the
// inverse of its factor, Linv_k = L_kk^-1; the blocks below it become
// C_ik Linv_k^T and the trailing matrix takes a rank-64 update.  The two
// triangular solves take the same shape: Z_k = Linv_k R_k (or Linv_k^T Z_k)
// and rank-64 updates of the block rows still to come, with the right-hand
// side's 64-column blocks in parallel; the rows beyond a group of kSuper
// block rows take the group's updates in one pass, so each of their blocks
// is read and written once per group (8 rows per pass measured 2.4% faster
// than 4 and 1% faster than 16 at d = 5120).  Every product is a 64 x 64 x 64
// product on v_mfma_f64_16x16x4_f64 (lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 v + l / 16][l % 16]).  Every sum runs in a
// fixed order: the result is bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "rf_solve.h"

namespace rf {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

constexpr int kB = 64;        // block size
constexpr int kSuper = 8;     // block rows per pass of the triangular solves' updates
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

// Cholesky of diagonal block k in place (its lower triangle) and the inverse
// of its factor, Linv_k = L_kk^-1, in one right-looking sweep over the
// columns.  Thread t owns column l = t / 4 and rows i = t % 4 + 4 r (r < 16)
// of both the block (sv) and of Y, which starts as the identity; the four
// owners of a column are one lane quad.  At column j the quad of column j
// shares the pivot C_jj (a quad shuffle), scales the column by the pivot's
// reciprocal (column j of L) and publishes it; after the one barrier of the
// step every quad takes Y_jl, the entry of row j in its own column, from its
// own lane (j & 3) and scales it (row j of Linv: Y_j = e_j - sum_{p<j} L_jp
// Linv_p by then), and every thread updates its entries below row j:
// C_il -= L_ij L_lj and Y_il -= L_ij Linv_jl.  Column j of L travels through
// LDS in a double buffer, so the next column's quad may publish while others
// still read this one.
__device__ __forceinline__ void potrf_inv_block(double* c, int d, int k, int* flag, double* linv) {
  __shared__ double colj[2][kB];  // column j of L, by step parity
  __shared__ double rinv[2];      // 1 / L_jj, by step parity
  __shared__ double dg[kB];       // the pivots
  double* blk = c + (static_cast<size_t>(k) * kB) * d + k * kB;
  const int t = threadIdx.x;
  const int l = t >> 2, rg = t & 3;
  double sv[16], yv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = rg + 4 * r;
    sv[r] = i >= l ? blk[static_cast<size_t>(i) * d + l] : 0.0;
    yv[r] = i == l ? 1.0 : 0.0;
  }
  // j = 4 rj + src: the register index rj of row j is a constant of the
  // unrolled outer loop, and rows above it (r < rj) are skipped statically
#pragma unroll
  for (int rj = 0; rj < 16; ++rj) {
#pragma unroll 1
    for (int src = 0; src < 4; ++src) {
      const int j = 4 * rj + src, pb = src & 1;
      if (l == j) {
        double v = __shfl(sv[rj], src, 4);  // C_jj, from the quad's lane that holds row j
        if (!(v > 0.0)) {
          if (rg == 0) *flag = 1;
          v = 1.0;  // keep going with finite values; the call reports the failure
        }
        const double dj = sqrt(v);
        const double rp = 1.0 / dj;
        if (rg == 0) {
          dg[j] = dj;
          rinv[pb] = rp;
        }
#pragma unroll
        for (int r = rj; r < 16; ++r) {
          if (r > rj || rg > src) {  // i = rg + 4 r > j
            sv[r] *= rp;
            colj[pb][rg + 4 * r] = sv[r];
          }
        }
      }
      __syncthreads();
      const double rp = rinv[pb];
      const double yj = __shfl(yv[rj], src, 4) * rp;  // Linv_jl for this thread's column l
      if (rg == src) yv[rj] = yj;
      const double cl = l > j ? colj[pb][l] : 0.0;
#pragma unroll
      for (int r = rj; r < 16; ++r) {
        const int i = rg + 4 * r;
        if (r > rj || rg > src) {  // i > j
          const double ci = colj[pb][i];
          if (l > j && l <= i) sv[r] -= ci * cl;
          yv[r] -= ci * yj;
        }
      }
    }
  }
  __syncthreads();  // dg complete
  double* out = linv + static_cast<size_t>(k) * kB * kB;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = rg + 4 * r;
    if (i > l) blk[static_cast<size_t>(i) * d + l] = sv[r];
    else if (i == l) blk[static_cast<size_t>(i) * d + l] = dg[l];
    out[i * kB + l] = yv[r];
  }
}

__global__ void __launch_bounds__(256) potrf_inv_kernel(double* c, int d, int k, int* flag, double* linv) {
  potrf_inv_block(c, d, k, flag, linv);
}

// D -= sum_kk P_kk Q_kk (modes 0-2) or D = P Q (modes 3-5) on 64 x 64 blocks
// with fp64 MFMA.  Each P and Q is staged in LDS as P[row][p] and Q[p][col]
// (each mode fills them from its own layout) before D, which may be one of
// them, is written; the nk pieces of modes 1 and 2 accumulate in registers in
// increasing kk, so D is read and written once for all of them.
//   MODE 0 (Cholesky update, step k): C[i][j] -= C[i][k] C[j][k]^T,        k < j <= i
//   MODE 1 (forward, steps k..k+nk-1): R[i][cb] -= sum C[i][kk] R[kk][cb],  rows i = i0 + y
//   MODE 2 (backward, steps k..k+nk-1): R[i][cb] -= sum C[kk][i]^T R[kk][cb], rows i = i0 + y
//   MODE 3 (panel, step k):           C[i][k] = C[i][k] Linv_k^T,          i > k
//   MODE 4 (forward, step k):         R[k][cb] = Linv_k R[k][cb]
//   MODE 5 (backward, step k):        R[k][cb] = Linv_k^T R[k][cb]
// (bx, by) is the block's place in the launch grid; false: an empty block of
// MODE 0 (above the diagonal), nothing done.
template <int MODE>
__device__ __forceinline__ bool block_update(double* c, int d, double* rhs, int d_out, int k, int nk, int i0,
                                             const double* linv, int bx, int by, double* ps, double* qs) {
  constexpr bool kReplace = MODE >= 3;
  const int cb = bx;  // modes 1, 2, 4, 5: column block of the right-hand side
  int i = 0;
  double* dst;
  int ldd;
  if (MODE == 0) {
    i = k + 1 + by;
    if (k + 1 + bx > i) return false;  // (whole workgroup)
    dst = c + (static_cast<size_t>(i) * kB) * d + (k + 1 + bx) * kB;
    ldd = d;
  } else if (MODE == 3) {
    i = k + 1 + bx;
    dst = c + (static_cast<size_t>(i) * kB) * d + k * kB;
    ldd = d;
  } else if (MODE >= 4) {
    dst = rhs + (static_cast<size_t>(k) * kB) * d_out + cb * kB;
    ldd = d_out;
  } else {
    i = i0 + by;
    dst = rhs + (static_cast<size_t>(i) * kB) * d_out + cb * kB;
    ldd = d_out;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int l16 = lane & 15, lk = lane >> 4;
  d4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = d4{0.0, 0.0, 0.0, 0.0};
  const int pieces = (MODE == 1 || MODE == 2) ? nk : 1;
  // Piece kk's 64 x 64 blocks of P and Q go through registers: the loads of
  // piece kk + 1 are issued before the products of piece kk, so their latency
  // hides behind them; the order of the products is unchanged.
  double pv[kB * kB / 256], qv[kB * kB / 256];
  auto fetch = [&](int kk) {
    const int kc = k + kk;
    const double* li = linv + static_cast<size_t>(kc) * kB * kB;
    const double *p_src, *q_src;
    int ldp, ldq;
    if (MODE == 0) {
      p_src = c + (static_cast<size_t>(i) * kB) * d + kc * kB;
      q_src = c + (static_cast<size_t>(k + 1 + bx) * kB) * d + kc * kB;  // used transposed
      ldp = ldq = d;
    } else if (MODE == 3) {
      p_src = dst;
      ldp = d;
      q_src = li;  // used transposed
      ldq = kB;
    } else if (MODE >= 4) {
      p_src = li;  // MODE 5: used transposed
      ldp = kB;
      q_src = dst;
      ldq = d_out;
    } else {
      p_src = MODE == 1 ? c + (static_cast<size_t>(i) * kB) * d + kc * kB   // L_i,kc
                        : c + (static_cast<size_t>(kc) * kB) * d + i * kB;  // L_kc,i, used transposed
      ldp = d;
      q_src = rhs + (static_cast<size_t>(kc) * kB) * d_out + cb * kB;
      ldq = d_out;
    }
#pragma unroll
    for (int n = 0; n < kB * kB / 256; ++n) {
      const int e = static_cast<int>(threadIdx.x) + 256 * n;
      const int r = e / kB, q = e % kB;
      pv[n] = p_src[static_cast<size_t>(r) * ldp + q];
      qv[n] = q_src[static_cast<size_t>(r) * ldq + q];
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int n = 0; n < kB * kB / 256; ++n) {
      const int e = static_cast<int>(threadIdx.x) + 256 * n;
      const int r = e / kB, q = e % kB;
      if (MODE == 2 || MODE == 5) ps[q * kLd + r] = pv[n]; else ps[r * kLd + q] = pv[n];
      if (MODE == 0 || MODE == 3) qs[q * kLd + r] = qv[n]; else qs[r * kLd + q] = qv[n];
    }
  };
  fetch(0);
  put();
  __syncthreads();
  for (int kk = 0; kk < pieces; ++kk) {
    if (kk + 1 < pieces) fetch(kk + 1);
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
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (kk + 1 < pieces) {
      __syncthreads();  // every wave is done with piece kk
      put();
      __syncthreads();
    }
  }
  // D's old values are all read before any store, so the 16 reads are in
  // flight together (a read-modify-write per element would wait out each one:
  // the compiler cannot tell that the stores do not alias the later reads).
  double old[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wr + 16 * a + 4 * v + lk, col = wc + 16 * b + l16;
        old[a][b][v] = kReplace ? 0.0 : dst[static_cast<size_t>(row) * ldd + col];
      }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wr + 16 * a + 4 * v + lk, col = wc + 16 * b + l16;
        dst[static_cast<size_t>(row) * ldd + col] = kReplace ? acc[a][b][v] : old[a][b][v] - acc[a][b][v];
      }
  return true;
}

// One launch of block_update<MODE> over its grid.  Some workgroups then take
// the next step of the chain at once, because it depends on the launch only
// through the block they have just written (their stores are visible to the
// whole workgroup after the barrier), so no launch sits between the steps:
//   MODE 0: the workgroup of block (k+1, k+1) factors it (potrf_inv_block);
//   MODE 1 with fuse (rows k+1 .. of a group): the workgroups of row k+1 form
//           Z_{k+1} = Linv_{k+1} R_{k+1} for their column block (MODE 4);
//   MODE 2 with fuse (rows i0 .. k-1 of a group): the workgroups of row k-1
//           form Linv_{k-1}^T Z_{k-1} for their column block (MODE 5).
template <int MODE>
__global__ void __launch_bounds__(256) update_kernel(double* c, int d, double* rhs, int d_out, int k, int nk, int i0,
                                                     double* linv, int* flag, int fuse) {
  __shared__ double ps[kB * kLd];
  __shared__ double qs[kB * kLd];
  const int bx = blockIdx.x, by = blockIdx.y;
  if (!block_update<MODE>(c, d, rhs, d_out, k, nk, i0, linv, bx, by, ps, qs)) return;
  if (MODE == 0 && bx == 0 && by == 0) {
    __syncthreads();
    potrf_inv_block(c, d, k + 1, flag, linv);
  }
  if (MODE == 1 && fuse && by == 0) {
    __syncthreads();
    block_update<4>(c, d, rhs, d_out, k + 1, 1, 0, linv, bx, 0, ps, qs);
  }
  if (MODE == 2 && fuse && by == static_cast<int>(gridDim.y) - 1) {
    __syncthreads();
    block_update<5>(c, d, rhs, d_out, k - 1, 1, 0, linv, bx, 0, ps, qs);
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

// b[j] = my[j] - sum_i W[i][j] mx[i] (b = 0 when raw, since then my = mx = 0),
// in two fixed-order levels: partial sums over 128-row chunks of i, then the
// chunks in increasing order.
constexpr int kOffRows = 128;
__global__ void __launch_bounds__(256) offset_part_kernel(const double* w, const double* mx, int d_out, double* part) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_out) return;
  const int i0 = blockIdx.y * kOffRows;
  double v = 0.0;
  for (int i = i0; i < i0 + kOffRows; ++i) v += w[static_cast<size_t>(i) * d_out + j] * mx[i];
  part[static_cast<size_t>(blockIdx.y) * d_out + j] = v;
}

__global__ void __launch_bounds__(256) offset_kernel(const double* part, const double* my, int n_part, int d_out,
                                                     float* b) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d_out) return;
  double v = 0.0;
  for (int c = 0; c < n_part; ++c) v += part[static_cast<size_t>(c) * d_out + j];
  b[j] = static_cast<float>(my[j] - v);
}

}  // namespace

size_t ridge_solve_workspace_bytes(int d_in, int d_out) {
  const size_t up = 256;
  auto r = [&](size_t v) { return (v + up - 1) / up * up; };
  return r(sizeof(double) * static_cast<size_t>(d_in) * d_in) + r(sizeof(double) * static_cast<size_t>(d_in) * d_out) +
         r(sizeof(double) * d_in) + r(sizeof(double) * d_out) + r(sizeof(double) * static_cast<size_t>(d_in) * kB) +
         r(sizeof(double) * static_cast<size_t>(d_in / kOffRows) * d_out) + up;
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
  double* linv = reinterpret_cast<double*>(p);  // [d_in / 64][64][64]
  p += r(sizeof(double) * static_cast<size_t>(di) * kB);
  double* part = reinterpret_cast<double*>(p);  // [d_in / 128][d_out]
  p += r(sizeof(double) * static_cast<size_t>(di / kOffRows) * dout);
  a.flag = reinterpret_cast<int*>(p);
  *flag_out = a.flag;

  hipLaunchKernelGGL(means_kernel, dim3((std::max(di, dout) + 255) / 256), dim3(256), 0, s, a);
  hipLaunchKernelGGL(form_kernel, dim3((di + dout + 255) / 256, di), dim3(256), 0, s, a);
  hipLaunchKernelGGL(ridge_diag_kernel, dim3(1), dim3(256), 0, s, a);
  const int T = di / kB, TC = dout / kB;
  // block 0 is factored alone; the trailing update of step k factors block k+1
  hipLaunchKernelGGL(potrf_inv_kernel, dim3(1), dim3(256), 0, s, a.c, di, 0, a.flag, linv);
  for (int k = 0; k + 1 < T; ++k) {
    hipLaunchKernelGGL((update_kernel<3>), dim3(T - k - 1), dim3(256), 0, s, a.c, di, a.r, dout, k, 1, 0, linv,
                       a.flag, 0);
    hipLaunchKernelGGL((update_kernel<0>), dim3(T - k - 1, T - k - 1), dim3(256), 0, s, a.c, di, a.r, dout, k, 1, 0,
                       linv, a.flag, 0);
  }
  // L Z = R, kSuper block rows at a time: within the group, Z_k = Linv_k R_k
  // and a rank-64 update of the group's later rows; then one update of every
  // row below the group with all of its pieces.
  for (int k0 = 0; k0 < T; k0 += kSuper) {
    const int k1 = std::min(k0 + kSuper, T);
    hipLaunchKernelGGL((update_kernel<4>), dim3(TC), dim3(256), 0, s, a.c, di, a.r, dout, k0, 1, 0, linv, a.flag, 0);
    for (int k = k0; k + 1 < k1; ++k)  // also Z_{k+1} = Linv_{k+1} R_{k+1}
      hipLaunchKernelGGL((update_kernel<1>), dim3(TC, k1 - k - 1), dim3(256), 0, s, a.c, di, a.r, dout, k, 1, k + 1,
                         linv, a.flag, 1);
    if (k1 < T)
      hipLaunchKernelGGL((update_kernel<1>), dim3(TC, T - k1), dim3(256), 0, s, a.c, di, a.r, dout, k0, k1 - k0, k1,
                         linv, a.flag, 0);
  }
  // L^T W = Z the same way, from the last block row up.
  for (int k1 = T; k1 > 0; k1 -= kSuper) {
    const int k0 = std::max(k1 - kSuper, 0);
    hipLaunchKernelGGL((update_kernel<5>), dim3(TC), dim3(256), 0, s, a.c, di, a.r, dout, k1 - 1, 1, 0, linv, a.flag,
                       0);
    for (int k = k1 - 1; k > k0; --k)  // also row k-1's Linv_{k-1}^T product
      hipLaunchKernelGGL((update_kernel<2>), dim3(TC, k - k0), dim3(256), 0, s, a.c, di, a.r, dout, k, 1, k0, linv,
                         a.flag, 1);
    if (k0 > 0)
      hipLaunchKernelGGL((update_kernel<2>), dim3(TC, k0), dim3(256), 0, s, a.c, di, a.r, dout, k0, k1 - k0, 0, linv,
                         a.flag, 0);
  }
  hipLaunchKernelGGL(transpose_out_kernel, dim3(dout / 32, di / 32), dim3(256), 0, s, a.r, di, dout, a_out);
  hipLaunchKernelGGL(offset_part_kernel, dim3((dout + 255) / 256, di / kOffRows), dim3(256), 0, s, a.r, a.mx, dout,
                     part);
  hipLaunchKernelGGL(offset_kernel, dim3((dout + 255) / 256), dim3(256), 0, s, part, a.my, di / kOffRows, dout, b_out);
  return hipGetLastError();
}

}  // namespace rf
