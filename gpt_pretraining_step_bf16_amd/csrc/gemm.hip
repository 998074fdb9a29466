// GEMM host side: argument defaults, dispatch of launch_gemm to the kernel
// instantiation of the operand layout and epilogue (gemm_*.hip), and the
// deterministic split-K reduction.
#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace {

__global__ void splitk_reduce_kernel(const float* __restrict__ part, long s_split, int splits,
                                     float* __restrict__ out, long n4, int accumulate) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    float4 s = accumulate ? reinterpret_cast<const float4*>(out)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; ++k) {
      const float4 v = reinterpret_cast<const float4*>(part + k * s_split)[i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

}  // namespace

void gemm_args_init(GemmArgs& g) {
  g = GemmArgs{};
  g.alpha = 1.f;
  g.beta = 0.f;
  g.batch = 1;
  g.splits = 1;
  g.k_chunk = 0;
}

hipError_t launch_gemm(const GemmArgs& g0, hipStream_t s) {
  GemmArgs g = g0;
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (g.splits < 1) g.splits = 1;
  if (g.k_chunk <= 0) g.k_chunk = g.K;
  if (g.splits == 1) g.k_chunk = g.K > 0 ? g.K : 1;
  const int tside = (g.M + 255) / 256;
  const int tiles = g.sym ? tside * (tside + 1) / 2 : tside * ((g.N + 255) / 256);
  const dim3 grid(tiles, g.batch * g.splits);
  if (g.a_kmajor && g.b_kmajor) {
    if (g.epi == EPI_BF16 || g.epi == EPI_RELU_BF16 || g.epi == EPI_RELU2_BF16 || g.epi == EPI_RESID_BF16 ||
        g.epi == EPI_QKN_BF16)
      return launch_gemm_kk_fwd(g, grid, s);
    return launch_gemm_kk_aux(g, grid, s);
  }
  if (g.a_kmajor != g.b_kmajor) return launch_gemm_kt(g, grid, s);
  return launch_gemm_tt(g, grid, s);
}

hipError_t launch_splitk_reduce(const float* part, long s_split, int splits, float* out, long n,
                                int accumulate, hipStream_t s) {
  const long n4 = n / 4;
  int blocks = (int)std::min<long>((n4 + 255) / 256, 8192);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, s_split, splits, out,
                     n4, accumulate);
  return hipGetLastError();
}
