// Device capture of the ridge fit's running sums.
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.2 ("Fitting"): the maps come from running sums of X^T X, X^T Y and
// the means over calibration text, then one closed-form solve per layer.  The
// activations are captured on the GPU during exact prefill, so the sums are
// formed there too.  bf16 values and their products are exact in fp64, so the
// fp64 matrix instructions used here give the host accumulator's sums up to
// the order of fp64 additions; the solve stays on the host (rf_ridge_solve).
//
// Contraction over rows, per 128 x 128 output tile, one workgroup of 4 waves
// (2 x 2, each 64 x 64 as 4 x 4 blocks of v_mfma_f64_16x16x4_f64):
//   S[i][j] += sum_r X[r][i0 + i] * Z[r][j0 + j],  Z = X (tiles with i0 <= j0) or Y.
// Rows stream through LDS 32 at a time (bf16, rows padded to 144 values so the
// four 4-row groups a fragment read touches fall in different banks), double
// buffered with register prefetch of the next 32 rows.  Lane l of an MFMA
// supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// D[4 v + l / 16][l % 16], v = 0..3.  Each tile belongs to one workgroup per
// launch, which adds its fp64 partial to the running sum once at the end.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "../../include/rf.h"
#include "rf_error.h"
#include "rf_ridge_internal.h"
#include "rf_solve.h"

namespace rf {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));

constexpr int kCT = 128;          // output tile
constexpr int kCR = 32;           // rows per stage
constexpr int kPad = 144;         // LDS row length in bf16 values
constexpr int kPart = kCR * kPad; // one operand's stage, in bf16 values

struct CaptureParams {
  const uint16_t* x;
  int64_t ld_x;
  const uint16_t* y;
  int64_t ld_y;
  int64_t n;
  int d_in, d_out;
  int t_in, t_out;   // tiles along d_in and d_out
  int tiles_xx;      // t_in (t_in + 1) / 2 upper tiles of X^T X
  double* sxx;       // [d_in][d_in]
  double* sxy;       // [d_in][d_out]
};

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(b) << 16));
}

// 16 bytes (8 bf16) of row r, columns c0 .. c0+7 of a row-major matrix, or zeros past the last row.
__device__ __forceinline__ uint4 load8(const uint16_t* base, int64_t ld, int64_t r, int64_t n, int c0) {
  if (r >= n) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(base + r * ld + c0);
}

__global__ void __launch_bounds__(256) capture_kernel(const CaptureParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kPart];  // [buffer][operand][row * kPad + col]
  int b = blockIdx.x;
  int ti, tj;
  const uint16_t* zb;
  int64_t ldz;
  double* out;
  int ldo;
  if (b < p.tiles_xx) {
    ti = 0;
    while (b >= p.t_in - ti) {
      b -= p.t_in - ti;
      ++ti;
    }
    tj = ti + b;
    zb = p.x;
    ldz = p.ld_x;
    out = p.sxx;
    ldo = p.d_in;
  } else {
    b -= p.tiles_xx;
    ti = b / p.t_out;
    tj = b - ti * p.t_out;
    zb = p.y;
    ldz = p.ld_y;
    out = p.sxy;
    ldo = p.d_out;
  }
  const int i0 = ti * kCT, j0 = tj * kCT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  // staging: 2 operands x 32 rows x 16 chunks of 8 values = 1024 chunks, 4 per thread
  uint4 pre[4];
  auto fetch = [&](int64_t r0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = t + u * 256;
      const int op = c >> 9, row = (c >> 4) & 31, col = (c & 15) * 8;
      pre[u] = op == 0 ? load8(p.x, p.ld_x, r0 + row, p.n, i0 + col) : load8(zb, ldz, r0 + row, p.n, j0 + col);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = t + u * 256;
      const int op = c >> 9, row = (c >> 4) & 31, col = (c & 15) * 8;
      *reinterpret_cast<uint4*>(&lds[buf][op][row * kPad + col]) = pre[u];
    }
  };

  d4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = d4{0.0, 0.0, 0.0, 0.0};

  const int stages = static_cast<int>((p.n + kCR - 1) / kCR);
  if (stages > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  const int col_a = wi * 64 + (lane & 15), col_b = wj * 64 + (lane & 15);
  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < stages) fetch(static_cast<int64_t>(s + 1) * kCR);
    const uint16_t* xa = lds[buf][0];
    const uint16_t* zb_l = lds[buf][1];
#pragma unroll 2
    for (int ks = 0; ks < kCR / 4; ++ks) {
      const int row = ks * 4 + (lane >> 4);
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = bf16_to_f64(xa[row * kPad + col_a + 16 * a]);
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = bf16_to_f64(zb_l[row * kPad + col_b + 16 * c]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[c], acc[a][c], 0, 0, 0);
    }
    if (s + 1 < stages) stash(buf ^ 1);
    __syncthreads();
  }

  // D[4 v + lane / 16][lane % 16] of block (a, c) -> S[i0 + wi*64 + 16a + 4v + lane/16][j0 + wj*64 + 16c + lane%16]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + wi * 64 + 16 * a + 4 * v + (lane >> 4);
        const int j = j0 + wj * 64 + 16 * c + (lane & 15);
        out[static_cast<size_t>(i) * ldo + j] += acc[a][c][v];
      }
}

// Column sums in a fixed order: partial[k][c] over rows k*per .. (k+1)*per - 1,
// then out[c] += sum over k in order.
__global__ void __launch_bounds__(256) colsum_partial_kernel(const uint16_t* m, int64_t ld, int64_t n, int d,
                                                             int64_t per, double* partial) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int k = blockIdx.y;
  if (c >= d) return;
  const int64_t r0 = k * per, r1 = r0 + per < n ? r0 + per : n;
  double s = 0.0;
  for (int64_t r = r0; r < r1; ++r) s += bf16_to_f64(m[r * ld + c]);
  partial[static_cast<size_t>(k) * d + c] = s;
}

__global__ void __launch_bounds__(256) colsum_reduce_kernel(const double* partial, int chunks, int d, double* out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  double s = 0.0;
  for (int k = 0; k < chunks; ++k) s += partial[static_cast<size_t>(k) * d + c];
  out[c] += s;
}

__global__ void __launch_bounds__(256) zero_f64_kernel(double* p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

constexpr int kChunks = 64;  // row chunks of the column sums

rf_status cfail(rf_status st, const char* msg) {
  set_last_error(msg);
  return st;
}

}  // namespace
}  // namespace rf

struct rf_ridge_dev {
  int d_in = 0, d_out = 0;
  long long n = 0;
  double* buf = nullptr;  // sxx, sxy, sx, sy, partial (one allocation)
  double *sxx = nullptr, *sxy = nullptr, *sx = nullptr, *sy = nullptr, *partial = nullptr;
  size_t elems = 0;       // doubles of sxx + sxy + sx + sy
};

namespace {

rf_status launch_zero(rf_ridge_dev* a, hipStream_t s) {
  const size_t blocks = (a->elems + 255) / 256;
  hipLaunchKernelGGL(rf::zero_f64_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a->buf, a->elems);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    rf::set_last_error(hipGetErrorString(e));
    return RF_E_HIP;
  }
  return RF_OK;
}

}  // namespace

extern "C" {

rf_status rf_ridge_dev_create(int32_t d_in, int32_t d_out, rf_ridge_dev** out) {
  if (!out) return rf::cfail(RF_E_ARG, "out is null");
  *out = nullptr;
  if (d_in < 1 || d_out < 1 || d_in % rf::kCT || d_out % rf::kCT)
    return rf::cfail(RF_E_SHAPE, "d_in and d_out must be positive multiples of 128");
  rf_ridge_dev* a = new rf_ridge_dev();
  a->d_in = d_in;
  a->d_out = d_out;
  const size_t nxx = static_cast<size_t>(d_in) * d_in, nxy = static_cast<size_t>(d_in) * d_out;
  a->elems = nxx + nxy + d_in + d_out;
  const size_t total = a->elems + static_cast<size_t>(rf::kChunks) * std::max(d_in, d_out);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&a->buf), total * sizeof(double));
  if (e != hipSuccess) {
    delete a;
    rf::set_last_error(hipGetErrorString(e));
    return RF_E_HIP;
  }
  a->sxx = a->buf;
  a->sxy = a->sxx + nxx;
  a->sx = a->sxy + nxy;
  a->sy = a->sx + d_in;
  a->partial = a->sy + d_out;
  rf_status st = launch_zero(a, nullptr);
  if (st == RF_OK && (e = hipStreamSynchronize(nullptr)) != hipSuccess) {
    rf::set_last_error(hipGetErrorString(e));
    st = RF_E_HIP;
  }
  if (st != RF_OK) {
    rf_ridge_dev_destroy(a);
    return st;
  }
  *out = a;
  return RF_OK;
}

void rf_ridge_dev_destroy(rf_ridge_dev* a) {
  if (!a) return;
  if (a->buf) (void)hipFree(a->buf);
  delete a;
}

rf_status rf_ridge_dev_add(rf_ridge_dev* a, const uint16_t* x, int64_t ld_x, const uint16_t* y, int64_t ld_y,
                           int64_t n, void* stream) {
  if (!a) return rf::cfail(RF_E_ARG, "accumulator is null");
  if (n < 0) return rf::cfail(RF_E_ARG, "n must be >= 0");
  if (n == 0) return RF_OK;
  if (!x || !y) return rf::cfail(RF_E_ARG, "x or y is null");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15)
    return rf::cfail(RF_E_ARG, "x and y must be 16-byte aligned");
  if (ld_x < a->d_in || ld_x % 8 || ld_y < a->d_out || ld_y % 8)
    return rf::cfail(RF_E_ARG, "ld_x >= d_in and ld_y >= d_out, both multiples of 8");
  hipStream_t s = static_cast<hipStream_t>(stream);
  rf::CaptureParams p{};
  p.x = x;
  p.ld_x = ld_x;
  p.y = y;
  p.ld_y = ld_y;
  p.n = n;
  p.d_in = a->d_in;
  p.d_out = a->d_out;
  p.t_in = a->d_in / rf::kCT;
  p.t_out = a->d_out / rf::kCT;
  p.tiles_xx = p.t_in * (p.t_in + 1) / 2;
  p.sxx = a->sxx;
  p.sxy = a->sxy;
  hipLaunchKernelGGL(rf::capture_kernel, dim3(p.tiles_xx + p.t_in * p.t_out), dim3(256), 0, s, p);
  const int64_t per = (n + rf::kChunks - 1) / rf::kChunks;
  const int chunks = static_cast<int>((n + per - 1) / per);
  hipLaunchKernelGGL(rf::colsum_partial_kernel, dim3((a->d_in + 255) / 256, chunks), dim3(256), 0, s, x, ld_x, n,
                     a->d_in, per, a->partial);
  hipLaunchKernelGGL(rf::colsum_reduce_kernel, dim3((a->d_in + 255) / 256), dim3(256), 0, s, a->partial, chunks,
                     a->d_in, a->sx);
  hipLaunchKernelGGL(rf::colsum_partial_kernel, dim3((a->d_out + 255) / 256, chunks), dim3(256), 0, s, y, ld_y, n,
                     a->d_out, per, a->partial);
  hipLaunchKernelGGL(rf::colsum_reduce_kernel, dim3((a->d_out + 255) / 256), dim3(256), 0, s, a->partial, chunks,
                     a->d_out, a->sy);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    rf::set_last_error(hipGetErrorString(e));
    return RF_E_HIP;
  }
  a->n += n;
  return RF_OK;
}

size_t rf_ridge_dev_solve_workspace_bytes(const rf_ridge_dev* a) {
  return a ? rf::ridge_solve_workspace_bytes(a->d_in, a->d_out) : 0;
}

rf_status rf_ridge_dev_solve(const rf_ridge_dev* a, double lambda, int32_t flags, float* A, float* b, void* ws,
                             size_t ws_bytes, void* stream) {
  if (!a || !A || !b) return rf::cfail(RF_E_ARG, "null argument");
  if (flags & ~RF_RIDGE_RAW) return rf::cfail(RF_E_ARG, "unknown ridge flag");
  if (a->n < 1) return rf::cfail(RF_E_ARG, "no rows accumulated");
  if (!(lambda >= 0.0)) return rf::cfail(RF_E_ARG, "lambda must be >= 0");
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(b)) & 3)
    return rf::cfail(RF_E_ARG, "a and b must be 4-byte aligned");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < rf::ridge_solve_workspace_bytes(a->d_in, a->d_out))
    return rf::cfail(RF_E_WORKSPACE, "workspace too small or not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  rf::RidgeSolveIn in{a->sxx, a->sxy, a->sx, a->sy, a->n, a->d_in, a->d_out};
  int* flag = nullptr;
  hipError_t e = rf::ridge_solve_enqueue(in, lambda, flags & RF_RIDGE_RAW, A, b, ws, &flag, s);
  int h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    rf::set_last_error(hipGetErrorString(e));
    return RF_E_HIP;
  }
  if (h) return rf::cfail(RF_E_LINALG, "ridge system is not positive definite");
  return RF_OK;
}

rf_status rf_ridge_dev_merge(rf_ridge_dev* a, rf_ridge_acc* acc, void* stream) {
  if (!a || !acc) return rf::cfail(RF_E_ARG, "null argument");
  int di = 0, dout = 0;
  rf::ridge_acc_dims(acc, &di, &dout);
  if (di != a->d_in || dout != a->d_out) return rf::cfail(RF_E_SHAPE, "accumulators differ in d_in or d_out");
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<double> h(a->elems);
  hipError_t e = hipMemcpyAsync(h.data(), a->buf, a->elems * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    rf::set_last_error(hipGetErrorString(e));
    return RF_E_HIP;
  }
  const size_t nxx = static_cast<size_t>(di) * di, nxy = static_cast<size_t>(di) * dout;
  rf::ridge_acc_add_sums(acc, h.data(), h.data() + nxx, h.data() + nxx + nxy, h.data() + nxx + nxy + di, a->n);
  a->n = 0;
  return launch_zero(a, s);
}

}  // extern "C"
