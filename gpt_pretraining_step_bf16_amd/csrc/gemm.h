// Host-side interface of the MFMA GEMM (gemm.hip, gemm_*.hip): bf16 operands,
// or fp16 ones for the EPI_H_* epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------------------
// MFMA GEMM:  C[b](m, n) <- epilogue( sum_k A[b](m, k) * B[b](n, k) )
// ---------------------------------------------------------------------------
enum GemmEpilogue {
  EPI_F32 = 0,          // C f32 = alpha*acc
  EPI_F32_ACC = 1,      // C f32 = beta*C + alpha*acc
  EPI_BF16 = 2,         // C bf16 = alpha*acc
  EPI_RELU_BF16 = 3,    // C bf16 = max(acc, 0)
  EPI_RESID_BF16 = 4,   // C bf16 = C + acc (in place)
  EPI_DRELU2_BF16 = 5,  // C bf16 = acc * 2 * sqrt(D) (D = relu(u)^2 bf16, same shape as C, ldd)
  EPI_SPLITK = 6,       // C f32 [split] = acc (partials, reduced later)
  EPI_HILO = 7,         // v = alpha*acc -> C bf16 hi(v), C2 bf16 lo(v)
  EPI_NS_POLY = 8,      // v = alpha*acc + beta*(D + D2) (D, D2 bf16 hi/lo) -> C hi, C2 lo
  EPI_NS_UPDATE = 9,    // v = alpha*acc + beta*D (D f32) -> C3 f32 v (unless C3 is null), C f16 v
  EPI_RELU2_BF16 = 10,  // C bf16 = max(acc, 0)^2
  // fp16 operands (v_mfma_f32_32x32x16_f16), fp32 accumulation:
  EPI_H_GRAM = 11,      // C f16 = alpha*acc
  EPI_H_NS_POLY = 12,   // v = alpha*acc + beta*D (D f16) -> C f16 v
  EPI_H_NS_UPDATE = 13, // v = alpha*acc + beta*D (D f16) -> C f16 v
  EPI_H_NS_LAST = 14,   // v = alpha*acc + beta*D (D f16) -> C3 f32 v (D layout)
  // QKV projection: C bf16 = acc, with heads (128 columns) below qk_heads
  // RMS-normalised and rotated (RoPE) per row, their norm scales to qk_rstd.
  EPI_QKN_BF16 = 15,
};

struct GemmArgs {
  const uint16_t* a;     // operand bases (bf16 or fp16 bits)
  const uint16_t* b;
  int M, N, K;
  long lda, ldb;         // leading dimensions (elements)
  long sa, sb;           // batch strides (elements)
  int a_kmajor, b_kmajor;
  int sym;               // 1: C is symmetric (M == N; HILO, NS_POLY, H_GRAM, H_NS_POLY): only tiles
                         //    tm <= tn are computed, off-diagonal ones also stored transposed
  void* c;
  long ldc, sc;
  void* c2;
  void* c3;
  const void* d;
  const void* d2;
  long ldd, sd;
  float alpha, beta;
  int batch;
  int splits;            // split-K factor (EPI_SPLITK only)
  int k_chunk;           // K per split, multiple of 64
  long s_split;          // element stride between split partials
  int epi;
  // EPI_QKN_BF16: rstd out [M, qk_heads]; (cos, sin) table [qk_T][64] pairs;
  // row m is position m % qk_T.
  float* qk_rstd;
  const float* qk_cs;
  int qk_T;
  int qk_heads;
};

void gemm_args_init(GemmArgs& g);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
// out[i] = (accumulate ? out[i] : 0) + sum_s part[s*s_split + i], i < n (n % 4 == 0)
hipError_t launch_splitk_reduce(const float* part, long s_split, int splits, float* out, long n,
                                int accumulate, hipStream_t s);


// Per-layout GEMM instantiation launchers (gemm_*.hip); grid is the
// persistent grid chosen by launch_gemm.
hipError_t launch_gemm_kk_fwd(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_kk_aux(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_kt(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_tt(const GemmArgs& g, dim3 grid, hipStream_t s);
