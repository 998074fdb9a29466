// Host-side launch interfaces of the gfx950 kernels (all asynchronous on a stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM:  C[b](m, n) <- epilogue( sum_k A[b](m, k) * B[b](n, k) )
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
  EPI_NS_UPDATE = 9,    // v = alpha*acc + beta*D (D f32) -> C3 f32 v, C hi, C2 lo
  EPI_RELU2_BF16 = 10,  // C bf16 = max(acc, 0)^2
};

struct GemmArgs {
  const uint16_t* a[3];  // per K-segment operand bases (bf16 bits); nseg segments are summed
  const uint16_t* b[3];
  int nseg;
  int M, N, K;
  long lda, ldb;         // leading dimensions (elements)
  long sa, sb;           // batch strides (elements)
  int a_kmajor, b_kmajor;
  int sym;               // 1: C is symmetric (M == N; HILO / NS_POLY only): only tiles
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
};

void gemm_args_init(GemmArgs& g);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
// out[i] = (accumulate ? out[i] : 0) + sum_s part[s*s_split + i], i < n (n % 4 == 0)
hipError_t launch_splitk_reduce(const float* part, long s_split, int splits, float* out, long n,
                                int accumulate, hipStream_t s);

// ---------------------------------------------------------------------------
// Attention (causal, head size 128) over a packed qkv [B*T, 3*H*128] bf16 buffer
// ---------------------------------------------------------------------------
// lse2: log2-domain softmax normaliser of the scaled scores, [B, H, T].
hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse2, int B, int T, int H,
                                hipStream_t s);
// delta: [B, H, T] scratch (rowsum(dO * O)).
hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse2,
                                const uint16_t* dO, uint16_t* dqkv, float* delta, int B, int T,
                                int H, hipStream_t s);

// ---------------------------------------------------------------------------
// Elementwise / row kernels
// ---------------------------------------------------------------------------
hipError_t launch_fill_u32(void* p, uint32_t value, long n_words, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s);
hipError_t launch_rope_table(float* cs, int T, hipStream_t s);  // cs [T][64][2] (cos, sin)
hipError_t launch_embed_fwd(const int32_t* tok, const uint16_t* wte, float* x, int* err, long N,
                            int d, int V, hipStream_t s);
hipError_t launch_embed_bwd(const int32_t* tok, const float* dx, float* dwte, long N, int d, int V,
                            hipStream_t s);
hipError_t launch_rmsnorm_fwd(const float* x, uint16_t* xn, float* rstd, long N, int d,
                              hipStream_t s);
// dx (+)= rstd * (dxn - xn * mean(dxn * xn)); also writes dx_bf16.
hipError_t launch_rmsnorm_bwd(const float* dxn, const uint16_t* xn, const float* rstd, float* dx,
                              uint16_t* dx_bf16, long N, int d, int accumulate, hipStream_t s);
hipError_t launch_qknorm_rope_fwd(uint16_t* qkv, float* rstd_qk, const float* cs, long N, int T,
                                  int H, hipStream_t s);
hipError_t launch_qknorm_rope_bwd(uint16_t* dqkv, const uint16_t* qkv, const float* rstd_qk,
                                  const float* cs, long N, int T, int H, hipStream_t s);
hipError_t launch_count_targets(const int32_t* tgt, long N, int V, int* counter, int* err,
                                hipStream_t s);
// Row-wise softmax cross-entropy over bf16 logits [rows, V] in place -> dz bf16,
// loss_rows [rows] f32. inv_count read from device (1 / #valid targets).
hipError_t launch_ce_softmax(uint16_t* logits, const int32_t* tgt, float* loss_rows, long rows,
                             int V, const int* n_valid, hipStream_t s);
hipError_t launch_loss_reduce(const float* loss_rows, long N, const int* n_valid, float* loss,
                              hipStream_t s);

// ---------------------------------------------------------------------------
// Muon
// ---------------------------------------------------------------------------
struct MuonGroup {
  long base;        // element offset of the group's first matrix in the flat buffers
  long layer_stride;
  int per_layer;    // matrices of this group in one layer
  long mat_stride;  // element offset between consecutive matrices within a layer
  int count;        // matrices in the group
  int rows, cols;   // element count per matrix is rows * cols
  int transposed_mask;  // bit i set: matrix i-of-layer is stored [x_cols, x_rows] (wide)
  long x_rows, x_cols;  // NS orientation X [x_rows, x_cols], x_rows >= x_cols, multiples of 32
};
hipError_t launch_muon_momentum(const MuonGroup& g, const float* grads, float* mom, float mu,
                                float* partials, int blocks_per_mat, hipStream_t s);
hipError_t launch_muon_pack(const MuonGroup& g, const float* mom, const float* partials,
                            int blocks_per_mat, float* x32, uint16_t* xh, uint16_t* xl,
                            hipStream_t s);
hipError_t launch_muon_update(const MuonGroup& g, const float* x32, float* params,
                              uint16_t* params_bf16, float lr, hipStream_t s);
// Frobenius-normalise count fp32 matrices of n elements in place and split into hi/lo.
hipError_t launch_ns_prepare(float* x32, uint16_t* xh, uint16_t* xl, int count, long n,
                             float* partials, int blocks_per_mat, hipStream_t s);
hipError_t launch_split_hilo(const float* x32, uint16_t* xh, uint16_t* xl, long n, hipStream_t s);

// Per-layout GEMM instantiation launchers (gemm_*.hip); grid is the
// persistent grid chosen by launch_gemm.
hipError_t launch_gemm_kk_fwd(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_kk_aux(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_kt(const GemmArgs& g, dim3 grid, hipStream_t s);
hipError_t launch_gemm_tt(const GemmArgs& g, dim3 grid, hipStream_t s);
