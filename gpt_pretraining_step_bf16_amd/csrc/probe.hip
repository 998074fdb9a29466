// Measurement probe (not part of the step): a dense bf16 MFMA issue-rate
// kernel. Its duration gives the matrix-core rate the chip sustains at the
// clock it holds under full MFMA load, a second denominator beside the
// published peak for the utilisation figures.
#include "../../include/gpt.h"
#include "common.h"

namespace {

// Each wave runs 4 independent accumulator chains of v_mfma_f32_32x32x16_bf16
// on register operands (no memory traffic in the loop), enough to keep the
// SIMD's matrix pipe issuing back to back.
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  const float x = 1e-3f * (float)(lane + 1);
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(x * (float)(k + 1));
    b[k] = (__bf16)(x - 1e-4f * (float)k);
  }
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int i = 0; i < iters; ++i) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, acc3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc0[k] + acc1[k] + acc2[k] + acc3[k];
  // Keeps the chains live; the sink holds one value per workgroup.
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

gpt_status gpt_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink, double* flops, void* stream) {
  if (blocks < 1 || iters < 1 || !sink || !flops) return GPT_EINVAL;
  // 4 waves per workgroup, 4 MFMAs of 32 x 32 x 16 (2 * 16384 flops) per iteration per wave.
  *flops = (double)blocks * 4.0 * (double)iters * 4.0 * 2.0 * 32.0 * 32.0 * 16.0;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_EHIP;
}

}  // extern "C"
