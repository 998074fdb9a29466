// GEMM instantiations, both operands K-contiguous: forward projections.
#include "gemm_kernel.h"

hipError_t launch_gemm_kk_fwd(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if (g.sym != 0) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_BF16: GEMM_LAUNCH(true, true, EPI_BF16); break;
    case EPI_RELU_BF16: GEMM_LAUNCH(true, true, EPI_RELU_BF16); break;
    case EPI_RELU2_BF16: GEMM_LAUNCH(true, true, EPI_RELU2_BF16); break;
    case EPI_RESID_BF16: GEMM_LAUNCH(true, true, EPI_RESID_BF16); break;
    case EPI_QKN_BF16:
      // Ping-pong kernel only (its epilogue pairs waves w, w ^ 1 over a head);
      // heads of 128 columns need whole 256-column tiles up to qk_heads.
      if (!gemm_pp_ok(g) || g.qk_rstd == nullptr || g.qk_cs == nullptr || g.qk_T <= 0 || g.qk_heads < 0 ||
          g.batch != 1 || g.splits != 1 || g.alpha != 1.f)
        return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_impl::gemm_pp_kernel<true, true, EPI_QKN_BF16>), dim3(gemm_pp_grid(grid)),
                         dim3(gemm_impl::PP_THR), 0, s, g);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
