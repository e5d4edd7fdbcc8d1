// Internal interface of the GPU ridge solve (rf_solve.hip), used by the
// device-sum API in rf_capture.hip.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rf {

// Device running sums of one layer (the layout rf_ridge_dev keeps).
struct RidgeSolveIn {
  const double* sxx;  // [d_in][d_in], entries with column >= row
  const double* sxy;  // [d_in][d_out]
  const double* sx;   // [d_in]
  const double* sy;   // [d_out]
  long long n;
  int d_in, d_out;    // multiples of 64
};

size_t ridge_solve_workspace_bytes(int d_in, int d_out);
// Enqueues the whole solve on s: a [d_out][d_in] and b [d_out] (device fp32).
// *flag_out points at a device int in ws that is nonzero after the stream
// reaches it if the system was not positive definite.
hipError_t ridge_solve_enqueue(const RidgeSolveIn& in, double lambda, bool raw, float* a, float* b, void* ws,
                               int** flag_out, hipStream_t s);

}  // namespace rf
