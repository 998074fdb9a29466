// Launchers of the elementwise optimizer kernels that are not part of the
// Muon path (defined in elementwise.hip).
#pragma once

#include <hip/hip_runtime.h>

// AdamW on two tensors of n elements at w + off0 and w + off1 (moments packed
// as [2][n]); bc1 / bc2 are the bias corrections 1 - beta^t.
hipError_t launch_adamw(float* w, uint16_t* wb, const float* g, float* m, float* v, long off0, long off1,
                        long n, float lr, float b1, float b2, float eps, float wd, float bc1, float bc2,
                        hipStream_t s);
