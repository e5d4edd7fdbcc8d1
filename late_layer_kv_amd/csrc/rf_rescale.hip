// Measurement of the value rescale.
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.3 ("Value rescale"): per request, late layer and key-value head,
// the mean over the request's first c tail rows of each row's exact value
// norm divided by its predicted value norm.  The value vectors come from the K/V kernel
// (value half only, stored densely by calibration row); these two kernels
// reduce them, each in a fixed summation order, so the result does not depend
// on the launch shape.
#include <hip/hip_runtime.h>

#include "rf_internal.h"

namespace rf {
namespace {

__device__ __forceinline__ float sumsq_bf16x8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16);
    const float hi = __uint_as_float(w[i] & 0xffff0000u);
    s += lo * lo + hi * hi;
  }
  return s;
}

// One thread per (calibration row, head) of one layer.
__global__ void __launch_bounds__(256) head_ratio_kernel(const RatioParams p) {
  const int g = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.n * p.n_kv) return;
  const int m = idx / p.n_kv, h = idx - m * p.n_kv;
  const size_t off = static_cast<size_t>(m) * p.n_kv * p.head_dim + static_cast<size_t>(h) * p.head_dim;
  const uint4* e = reinterpret_cast<const uint4*>(p.ve[g] + off);
  const uint4* q = reinterpret_cast<const uint4*>(p.vp[g] + off);
  float se = 0.0f, sp = 0.0f;
  for (int i = 0; i < p.head_dim / 8; ++i) {
    se += sumsq_bf16x8(e[i]);
    sp += sumsq_bf16x8(q[i]);
  }
  p.ratio[g][idx] = sp > 0.0f ? sqrtf(se) / sqrtf(sp) : -1.0f;
}

// One wave per (layer, group, head): the mean of the group's ratios.  Lane t
// adds rows t, t + 64, t + 128, ... in order; the 64 lane sums and counts then
// combine in a fixed butterfly (a row loop per output took 150 us at 512
// calibration rows).
__global__ void __launch_bounds__(256) scale_mean_kernel(const float* ratio, const int32_t* group, int n, int n_kv,
                                                         int n_groups, int n_late, float* scale) {
  const int idx = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (idx >= n_late * n_groups * n_kv) return;  // (whole wave)
  const int h = idx % n_kv;
  const int grp = (idx / n_kv) % n_groups;
  const int l = idx / (n_kv * n_groups);
  const float* r = ratio + static_cast<size_t>(l) * n * n_kv + h;
  float sum = 0.0f;
  int cnt = 0;
  for (int m = lane; m < n; m += 64) {
    const float v = r[static_cast<size_t>(m) * n_kv];
    if (group[m] == grp && v >= 0.0f) {
      sum += v;
      ++cnt;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sum += __shfl_xor(sum, o);
    cnt += __shfl_xor(cnt, o);
  }
  if (lane == 0) scale[idx] = cnt ? sum / static_cast<float>(cnt) : 1.0f;
}

__global__ void __launch_bounds__(256) zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_head_ratio(const RatioParams& p, int n_layers, hipStream_t s) {
  const int blocks = (p.n * p.n_kv + 255) / 256;
  hipLaunchKernelGGL(head_ratio_kernel, dim3(blocks > 0 ? blocks : 1, n_layers), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scale_mean(const float* ratio, const int32_t* group, int n, int n_kv, int n_groups, int n_late,
                             float* scale, hipStream_t s) {
  const int total = n_late * n_groups * n_kv;  // one wave each, four per workgroup
  hipLaunchKernelGGL(scale_mean_kernel, dim3((total + 3) / 4), dim3(256), 0, s, ratio, group, n, n_kv, n_groups,
                     n_late, scale);
  return hipGetLastError();
}

}  // namespace rf
