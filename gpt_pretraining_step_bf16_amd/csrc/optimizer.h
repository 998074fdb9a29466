// Launchers of the optimizer kernels beyond the plain Muon step: AdamW and
// NorMuon (defined in elementwise.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

// AdamW on two tensors of n elements at w + off0 and w + off1 (moments packed
// as [2][n]); bc1 / bc2 are the bias corrections 1 - beta^t.
hipError_t launch_adamw(float* w, uint16_t* wb, const float* g, float* m, float* v, long off0, long off1,
                        long n, float lr, float b1, float b2, float eps, float wd, float bc1, float bc2,
                        hipStream_t s);

// NorMuon on a Muon group's Newton-Schulz output x32 ([count, x_rows, x_cols]):
// updates the per-row second moment state ([count, x_rows]) and writes the
// per-row scale rs ([count, x_rows]); terms is scratch of 2 * count * x_rows.
hipError_t launch_normuon(const MuonGroup& g, const float* x32, float* state, float beta2, float* rs,
                          float* terms, hipStream_t s);
// launch_muon_update with row r of X multiplied by row_scale[j * x_rows + r].
hipError_t launch_muon_update_scaled(const MuonGroup& g, const float* x32, float* params,
                                     uint16_t* params_bf16, float lr, const float* row_scale, hipStream_t s);
