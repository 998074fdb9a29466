// GEMM instantiations, both operands K-contiguous: forward projections.
#include "gemm_kernel.h"

hipError_t launch_gemm_kk_fwd(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (g.sym != 0) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_BF16: GEMM_LAUNCH(true, true, EPI_BF16); break;
    case EPI_RELU_BF16: GEMM_LAUNCH(true, true, EPI_RELU_BF16); break;
    case EPI_RELU2_BF16: GEMM_LAUNCH(true, true, EPI_RELU2_BF16); break;
    case EPI_RESID_BF16: GEMM_LAUNCH(true, true, EPI_RESID_BF16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
