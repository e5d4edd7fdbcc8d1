// The fill-row set on the GPU ("RidgeFill: Training-Free Late-Layer Cache
// Fill for Faster Prefill", section 2.1: the rows the fill writes are all rows
// of the batch minus the exact set, the tail of every request plus any chosen
// prefix rows).
//
// The exact rows mark a byte mask; the unmarked rows are then compacted in
// ascending order by a count / scan / write sequence over blocks of 4,096
// rows, so that the work spreads over many workgroups (one workgroup per
// block) instead of one workgroup walking the whole batch:
//   clear : mask[r] = 0 for r < n_rows, 1 for the padding up to a whole block
//   mark  : mask[e] = 1 for every exact row e (duplicates and any order fine)
//   count : cnt[b] = unmarked rows of block b
//   scan  : off[b] = cnt[0] + ... + cnt[b-1] (one workgroup, fixed order), n_fill
//   write : the unmarked rows of block b, ascending, at fill_rows[off[b] ...]
// Every step is deterministic and the output is the same for any order of the
// exact rows.  A thread owns 16 consecutive rows, read as one 16-byte load of
// the mask; mask bytes are 0 or 1, so the marked rows of a 4-byte word are its
// popcount.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rf_internal.h"

namespace rf {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowsPerThread = 16;
constexpr int kRowsPerBlock = kRowThreads * kRowsPerThread;  // 4,096 rows per workgroup
constexpr int kScanThreads = 1024;

constexpr size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of the fill-row set for n_rows rows: the mask padded to whole
// blocks, then the per-block counts and offsets.
constexpr size_t ws_bytes_for(int n_rows) {
  return round_up(round_up(static_cast<size_t>(n_rows > 0 ? n_rows : 1), kRowsPerBlock), 256) +
         2 * round_up(round_up(static_cast<size_t>(n_rows > 0 ? n_rows : 1), kRowsPerBlock) / kRowsPerBlock * 4, 256);
}

// Exclusive prefix sum of v over the workgroup (kWaves waves of 64); `total`
// receives the workgroup's sum.  wave_sums holds kWaves ints of LDS.
template <int kWaves>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = wave_sums[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();  // wave_sums may be reused by the caller
  return before + x - v;
}

// Unmarked rows among the 16 mask bytes in m.
__device__ __forceinline__ int unmarked16(uint4 m) {
  return kRowsPerThread - (__popc(m.x) + __popc(m.y) + __popc(m.z) + __popc(m.w));
}

// One 16-byte store per thread; n_pad is a multiple of kRowsPerBlock.
__global__ void __launch_bounds__(kRowThreads) rows_clear_kernel(uint8_t* mask, int n_rows, int n_pad) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x) * 16;
  if (i >= n_pad) return;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[q] |= (i + 4 * q + j < n_rows) ? 0u : (1u << (8 * j));
  }
  *reinterpret_cast<uint4*>(mask + i) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(kRowThreads) rows_mark_kernel(const int32_t* exact, int n_exact, uint8_t* mask,
                                                                int n_rows) {
  const int i = blockIdx.x * kRowThreads + threadIdx.x;
  if (i >= n_exact) return;
  const int r = exact[i];
  if (r >= 0 && r < n_rows) mask[r] = 1;
}

__global__ void __launch_bounds__(kRowThreads) rows_count_kernel(const uint8_t* mask, int32_t* cnt) {
  __shared__ int wave_sums[kRowThreads / 64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x * kRowsPerThread;
  const int c = unmarked16(*reinterpret_cast<const uint4*>(mask + r0));
  int total;
  block_exclusive_scan<kRowThreads / 64>(c, wave_sums, total);
  if (threadIdx.x == 0) cnt[blockIdx.x] = total;
}

// One workgroup: off[b] = sum of cnt[0 .. b), in chunks of 1024 with a carry.
__global__ void __launch_bounds__(kScanThreads) rows_scan_kernel(const int32_t* cnt, int n_blocks, int32_t* off,
                                                                 int32_t* n_fill) {
  __shared__ int wave_sums[kScanThreads / 64];
  int carry = 0;
  for (int base = 0; base < n_blocks; base += kScanThreads) {
    const int b = base + static_cast<int>(threadIdx.x);
    const int v = b < n_blocks ? cnt[b] : 0;
    int total;
    const int e = block_exclusive_scan<kScanThreads / 64>(v, wave_sums, total);
    if (b < n_blocks) off[b] = carry + e;
    carry += total;
  }
  if (threadIdx.x == 0) *n_fill = carry;
}

__global__ void __launch_bounds__(kRowThreads) rows_write_kernel(const uint8_t* mask, const int32_t* off,
                                                                 int32_t* fill_rows) {
  __shared__ int wave_sums[kRowThreads / 64];
  const int r0 = blockIdx.x * kRowsPerBlock + threadIdx.x * kRowsPerThread;
  const uint4 m = *reinterpret_cast<const uint4*>(mask + r0);
  int total;
  int o = off[blockIdx.x] + block_exclusive_scan<kRowThreads / 64>(unmarked16(m), wave_sums, total);
  const uint32_t words[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j)
    if (((words[j >> 2] >> (8 * (j & 3))) & 0xffu) == 0) fill_rows[o++] = r0 + j;
}

}  // namespace

size_t fill_rows_ws_bytes(int n_rows) { return ws_bytes_for(n_rows); }

// Workspace carve: mask [pad] bytes, cnt [blocks] int32, off [blocks] int32.
hipError_t launch_fill_rows(const int32_t* exact, int n_exact, int n_rows, void* ws, int32_t* fill_rows,
                            int32_t* n_fill, hipStream_t s) {
  const int pad = static_cast<int>(round_up(static_cast<size_t>(n_rows > 0 ? n_rows : 1), kRowsPerBlock));
  const int blocks = pad / kRowsPerBlock;
  uint8_t* mask = static_cast<uint8_t*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(mask + round_up(pad, 256));
  int32_t* off = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(cnt) + round_up(static_cast<size_t>(blocks) * 4, 256));
  const int clear_threads = pad / 16;
  hipLaunchKernelGGL(rows_clear_kernel, dim3((clear_threads + kRowThreads - 1) / kRowThreads), dim3(kRowThreads), 0,
                     s, mask, n_rows, pad);
  if (n_exact > 0)
    hipLaunchKernelGGL(rows_mark_kernel, dim3((n_exact + kRowThreads - 1) / kRowThreads), dim3(kRowThreads), 0, s,
                       exact, n_exact, mask, n_rows);
  hipLaunchKernelGGL(rows_count_kernel, dim3(blocks), dim3(kRowThreads), 0, s, mask, cnt);
  hipLaunchKernelGGL(rows_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, cnt, blocks, off, n_fill);
  hipLaunchKernelGGL(rows_write_kernel, dim3(blocks), dim3(kRowThreads), 0, s, mask, off, fill_rows);
  return hipGetLastError();
}

}  // namespace rf

// ---- The fill-row set without allocation ----------------------------------
// For callers that cannot allocate device memory, the scratch of the
// fill-row set (mask, block counts, block offsets) can live in this
// library-owned array instead of a workspace: room for kNoAllocMaxRows rows,
// about 1 MiB, held on every GPU the library runs on until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// only stands in for the device symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept per device.  All calls on one GPU share the array: the
// clear kernel resets the mask on every call, and calls that overlap on one
// GPU (unordered streams) race.
static __device__ __align__(256) uint8_t scratch[rf::ws_bytes_for(rf::kNoAllocMaxRows)];

namespace rf {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

hipError_t launch_fill_rows_noalloc(const int32_t* exact, int n_exact, int n_rows, int32_t* fill_rows,
                                    int32_t* n_fill, hipStream_t s) {
  if (n_rows > kNoAllocMaxRows) return hipErrorInvalidValue;  // the caller reports the limit first
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_dev[dev] = p;
    }
    ws = g_scratch_dev[dev];
  }
  return launch_fill_rows(exact, n_exact, n_rows, ws, fill_rows, n_fill, s);
}

}  // namespace rf
