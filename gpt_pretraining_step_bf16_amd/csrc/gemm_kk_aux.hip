// GEMM instantiations, both operands K-contiguous: fp32 outputs and the
// Newton-Schulz polynomial / update epilogues.
#include "gemm_kernel.h"

hipError_t launch_gemm_kk_aux(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (g.sym != 0 && ((g.epi != EPI_NS_POLY && g.epi != EPI_H_NS_POLY) || g.M != g.N)) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_F32: GEMM_LAUNCH(true, true, EPI_F32); break;
    case EPI_F32_ACC: GEMM_LAUNCH(true, true, EPI_F32_ACC); break;
    case EPI_NS_POLY: GEMM_LAUNCH(true, true, EPI_NS_POLY); break;
    case EPI_NS_UPDATE: GEMM_LAUNCH(true, true, EPI_NS_UPDATE); break;
    case EPI_H_NS_POLY: GEMM_LAUNCH(true, true, EPI_H_NS_POLY); break;
    case EPI_H_NS_UPDATE: GEMM_LAUNCH(true, true, EPI_H_NS_UPDATE); break;
    case EPI_H_NS_LAST: GEMM_LAUNCH(true, true, EPI_H_NS_LAST); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
