// Expansion of int8 maps into bf16 for the map contraction.
//
// "RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill",
// section 2.2 ("Size and cost") and section 4.2: a map is stored as int8 codes
// with one bf16 scale for each 128-weight block of a row.  The contraction runs on
// bf16 matrix instructions, so each launch group's maps are first expanded,
// w = bf16(q * s) rounded to nearest even.  q * s is exact in fp32 (8-bit code
// times 8-bit significand), so the only rounding is the final one.
//
// The kernel is bound by HBM: per weight it reads 1 byte of code and 1/64
// byte of scale and writes 2 bytes.  One thread expands 16 consecutive codes
// of one row (a 16-byte load, two 16-byte stores); consecutive threads walk a
// row, so every wavefront touches 1 KB of codes and 2 KB of output in order.
#include <hip/hip_runtime.h>

#include "rf_internal.h"

namespace rf {
namespace {

typedef __bf16 bf16x2q __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2q v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Four signed codes packed in a dword, each times s, as two bf16 pairs.
__device__ __forceinline__ void expand4(uint32_t c, float s, uint32_t& o0, uint32_t& o1) {
  const float f0 = static_cast<float>(static_cast<int32_t>(c << 24) >> 24);
  const float f1 = static_cast<float>(static_cast<int32_t>(c << 16) >> 24);
  const float f2 = static_cast<float>(static_cast<int32_t>(c << 8) >> 24);
  const float f3 = static_cast<float>(static_cast<int32_t>(c) >> 24);
  o0 = pack2(f0 * s, f1 * s);
  o1 = pack2(f2 * s, f3 * s);
}

__global__ void __launch_bounds__(256) dequant_kernel(const DequantParams p) {
  const int g = blockIdx.y;
  const int per_row = p.d_in >> 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(p.d_out) * per_row) return;
  const int o = static_cast<int>(idx / per_row);
  const int k16 = static_cast<int>(idx - static_cast<int64_t>(o) * per_row) << 4;
  const uint16_t sb = p.s[g][static_cast<int64_t>(o) * (p.d_in / kQ8Block) + k16 / kQ8Block];
  const float s = __uint_as_float(static_cast<uint32_t>(sb) << 16);
  const int64_t off = static_cast<int64_t>(o) * p.d_in + k16;
  const uint4 c = *reinterpret_cast<const uint4*>(p.q[g] + off);
  uint4 lo, hi;
  expand4(c.x, s, lo.x, lo.y);
  expand4(c.y, s, lo.z, lo.w);
  expand4(c.z, s, hi.x, hi.y);
  expand4(c.w, s, hi.z, hi.w);
  uint4* dst = reinterpret_cast<uint4*>(p.w[g] + off);
  dst[0] = lo;
  dst[1] = hi;
}

}  // namespace

hipError_t launch_dequant(const DequantParams& p, int n_layers, hipStream_t s) {
  const int64_t per_layer = static_cast<int64_t>(p.d_out) * (p.d_in >> 4);
  const int blocks = static_cast<int>((per_layer + 255) / 256);
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks, n_layers), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace rf
