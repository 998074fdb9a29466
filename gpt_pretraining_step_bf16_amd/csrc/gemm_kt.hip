// GEMM instantiations with one K-strided operand: the input gradients
// (activation gradient times a weight read along its out dimension).
#include "gemm_kernel.h"

hipError_t launch_gemm_kt(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (g.sym != 0) return hipErrorInvalidValue;
  if (g.a_kmajor) {
    switch (g.epi) {
      case EPI_DRELU2_BF16: GEMM_LAUNCH(true, false, EPI_DRELU2_BF16); break;
      case EPI_F32: GEMM_LAUNCH(true, false, EPI_F32); break;
      case EPI_BF16: GEMM_LAUNCH(true, false, EPI_BF16); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (g.epi) {
      case EPI_F32: GEMM_LAUNCH(false, true, EPI_F32); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}
