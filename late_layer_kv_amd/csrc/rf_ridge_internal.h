// Internal interface between the host ridge accumulator (rf_ridge.cpp) and the
// device capture of its sums (rf_capture.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/rf.h"

namespace rf {
// Dimensions of a host accumulator.
void ridge_acc_dims(const rf_ridge_acc* a, int* d_in, int* d_out);
// Adds raw sums to a host accumulator: sxx [d_in][d_in] (only entries with
// column >= row are read), sxy [d_in][d_out], sx [d_in], sy [d_out], n rows.
void ridge_acc_add_sums(rf_ridge_acc* a, const double* sxx, const double* sxy, const double* sx, const double* sy,
                        int64_t n);
}  // namespace rf
