// Host-side launch interfaces of the gfx950 kernels (all asynchronous on a stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

hipError_t launch_fill_u32(void* p, uint32_t value, long n_words, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s);
hipError_t launch_rope_table(float* cs, int T, hipStream_t s);  // cs [T][64][2] (cos, sin)
hipError_t launch_embed_fwd(const int32_t* tok, const uint16_t* wte, float* x, int* err, long N,
                            int d, int V, hipStream_t s);
// Scratch of the ordered row scatter-add (embedding and value-embedding table
// gradients), for N positions of rows W wide: part >= scatter_part_bytes,
// run_ids >= scatter_ids_bytes, nruns >= scatter_groups * 4 bytes.
struct ScatterWs {
  float* part;
  int32_t* run_ids;
  int32_t* nruns;
};
constexpr int kScatterMaxGroups = 2048;  // N <= 2048 * 256 positions per call
inline long scatter_groups(long N) { return (N + 255) / 256; }
inline size_t scatter_part_bytes(long N, long W) { return (size_t)scatter_groups(N) * 256 * W * 4; }
inline size_t scatter_ids_bytes(long N) { return (size_t)scatter_groups(N) * 256 * 4; }
// dwte (+)= per-token sums of the dx rows, in a fixed order; rows of absent
// tokens are written as 0 (left unchanged with accumulate).
hipError_t launch_embed_bwd(const int32_t* tok, const float* dx, float* dwte, long N, int d, int V, int accumulate,
                            const ScatterWs& ws, hipStream_t s);
// The value-embedding table gradient: dtable (+)= per-token sums of the rows
// 3 sigmoid(logits[i][h]) dv[i][h*128 .. h*128+127] (dv bf16, row stride ld).
hipError_t launch_ve_table_bwd(const uint16_t* dv, long ld, const float* logits, int Hkv, const int32_t* tok,
                               long N, int V, float* dtable, int accumulate, const ScatterWs& ws, hipStream_t s);
hipError_t launch_rmsnorm_fwd(const float* x, uint16_t* xn, float* rstd, long N, int d,
                              hipStream_t s);
// dx (+)= rstd * (dxn - xn * mean(dxn * xn)); also writes dx_bf16.
hipError_t launch_rmsnorm_bwd(const float* dxn, const uint16_t* xn, const float* rstd, float* dx,
                              uint16_t* dx_bf16, long N, int d, int accumulate, hipStream_t s);
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
                            int blocks_per_mat, float* x32, uint16_t* xb, hipStream_t s);
hipError_t launch_muon_update(const MuonGroup& g, const float* x32, float* params,
                              uint16_t* params_bf16, float lr, hipStream_t s);
// Frobenius-normalise count fp32 matrices of n elements in place and write their bf16 copy.
hipError_t launch_ns_prepare(float* x32, uint16_t* xb, int count, long n, float* partials,
                             int blocks_per_mat, hipStream_t s);

// ---------------------------------------------------------------------------
// Residual scalars and backout (all arrays fp32 [n], n % 4 == 0; scalars are
// device pointers to bf16 weights)
// ---------------------------------------------------------------------------
int resid_partials_count();  // float2 partials the two reductions below need
// x_prev <- x; x <- a x + b x0
hipError_t launch_resid_mix_fwd(float* x, const float* x0, float* x_prev, const uint16_t* pa, const uint16_t* pb,
                                long n, hipStream_t s);
// y <- y + scale * c * x (c = *pc, or 1 if pc is null)
hipError_t launch_axpy_f32(float* y, const float* x, const uint16_t* pc, float scale, long n, hipStream_t s);
// With g = dx: *ga (+)= g . x_prev, *gb (+)= g . x0, dx0 += b g, dx <- a g, dxb <- bf16(a g)
hipError_t launch_resid_mix_bwd(float* dx, uint16_t* dxb, const float* x_prev, const float* x0, float* dx0,
                                const uint16_t* pa, const uint16_t* pb, long n, float2* partials, float* ga,
                                float* gb, int accumulate, hipStream_t s);
// *gc (+)= -(dx . xbo); dback <- dx
hipError_t launch_backout_bwd(const float* dx, const float* xbo, float* dback, long n, float2* partials,
                              float* gc, int accumulate, hipStream_t s);
// dx += -c dback, dxb <- bf16(dx)
hipError_t launch_backout_add(float* dx, uint16_t* dxb, const float* dback, const uint16_t* pc, long n,
                              hipStream_t s);
// AdamW on n contiguous elements (no alignment assumed)
hipError_t launch_adamw_small(float* w, uint16_t* wb, const float* g, float* m, float* v, long n, float lr,
                              float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t s);

// ---------------------------------------------------------------------------
// Smear (x fp32 [N, d], rows b * T + t; gate weights and lambda are bf16)
// ---------------------------------------------------------------------------
int smear_partials_floats();
// x <- smear(xe); a <- gate logits [N]
hipError_t launch_smear_fwd(const float* xe, float* x, float* a, const uint16_t* pw, const uint16_t* plam, long N,
                            int T, int d, hipStream_t s);
// dxo <- gradient of xe from dy; *gw [24], *glam (+)= the gate's gradients
hipError_t launch_smear_bwd(const float* dy, const float* xe, const float* a, float* dxo, const uint16_t* pw,
                            const uint16_t* plam, long N, int T, int d, float* partials, float* gw, float* glam,
                            int accumulate, hipStream_t s);

// ---------------------------------------------------------------------------
// Value embeddings (table bf16 [V, Hkv*128], gate bf16 [Hkv, 32], Hkv <= 16)
// ---------------------------------------------------------------------------
int ve_partials_floats(int Hkv);
// v of qkv += 3 sigmoid(gate . xn[0:32]) * table[token]; logits [N, Hkv]
hipError_t launch_ve_fwd(uint16_t* qkv, const uint16_t* xn, const int32_t* tok, const uint16_t* table,
                         const uint16_t* gate, float* logits, long N, int d, int Hkv, int V, hipStream_t s);
// dtable (+)= (ordered scatter, ws), dgate (+)= (ordered sums), dxn[:, 0:32] += the gate's
// input gradient; dlogit [N, Hkv] and partials are scratch
hipError_t launch_ve_bwd(const uint16_t* dqkv, const uint16_t* xn, const int32_t* tok, const uint16_t* table,
                         const uint16_t* gate, const float* logits, float* dtable, float* dlogit, float* partials,
                         float* dgate, float* dxn, long N, int d, int Hkv, int V, int accumulate,
                         const ScatterWs& ws, hipStream_t s);
// AdamW on n (multiple of 4) contiguous elements, moments at m, v
hipError_t launch_adamw_range(float* w, uint16_t* wb, const float* g, float* m, float* v, long n, float lr,
                              float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t s);
