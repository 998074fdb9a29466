// GEMM instantiations with both operands K-strided: weight gradients (K runs
// over tokens) and the Newton-Schulz Gram matrix (bf16 and fp16 operands).
#include "gemm_kernel.h"

hipError_t launch_gemm_tt(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (g.sym != 0 && ((g.epi != EPI_HILO && g.epi != EPI_H_GRAM) || g.M != g.N)) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_SPLITK: GEMM_LAUNCH(false, false, EPI_SPLITK); break;
    case EPI_F32_ACC: GEMM_LAUNCH(false, false, EPI_F32_ACC); break;
    case EPI_HILO: GEMM_LAUNCH(false, false, EPI_HILO); break;
    case EPI_H_GRAM: GEMM_LAUNCH(false, false, EPI_H_GRAM); break;
    case EPI_F32: GEMM_LAUNCH(false, false, EPI_F32); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
