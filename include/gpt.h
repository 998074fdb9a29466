/*
 * gpt.h -- C ABI of the MI355X (gfx950) pretraining step of the
 * depth-parameterised GPT: one forward + backward pass over a microbatch and
 * one Muon update of the block matrices.
 *
 * Sources (cited by page title and section):
 *   [CT50] dev.to, "Como treinar seu próprio ChatGPT por 50 dólares".
 *   [HADA] GeekNews (hada.io) summary of the nanochat launch README.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Plain C types only. Device buffers are raw device pointers; `stream` is a
 *   hipStream_t passed as void* (NULL = the null stream).
 * - The caller allocates and owns every device buffer (parameters, bf16
 *   shadow, gradients, momentum, tokens, loss, workspaces). The library never
 *   allocates device memory and keeps no device state between calls; a
 *   gpt_model is a host-side plan (shapes and the flat parameter layout).
 * - Matrices are row-major [out, in] as in a bias-free Linear layer
 *   ([CT50] "3. Gerenciamento de Precisão": weights are kept in full precision
 *   and cast to the activation type on use). Flat buffers hold the tensors in
 *   canonical order: wte; per layer wq, wk, wv, wo, wfc, wproj; lm_head.
 * - bf16 buffers hold raw bfloat16 bits (uint16_t), round-to-nearest-even.
 * - All compute calls are asynchronous on `stream`; results are valid after
 *   the stream is synchronised. One model handle serves one stream at a time.
 * - Host-side validation happens before any launch and returns a status; on a
 *   non-OK status nothing was launched. Errors found on the device (a token
 *   or target outside the vocabulary) set a flag in the first word of the
 *   gpt_fwd_bwd workspace; each gpt_fwd_bwd call clears it first, and
 *   gpt_check() reports it. Nothing crosses the ABI as a C++ exception.
 */
#ifndef GPT_STEP_GPT_H
#define GPT_STEP_GPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gpt_model gpt_model;

typedef enum {
  GPT_OK = 0,
  GPT_EINVAL = -1,     /* bad argument: null pointer, depth/vocab/seq/batch out of range */
  GPT_ESHAPE = -2,     /* shape not supported (e.g. seq > the plan's max_seq) */
  GPT_EHIP = -3,       /* a HIP runtime call failed */
  GPT_ETOKEN = -4,     /* a token id or target outside [0, vocab) (target -1 = ignore) */
  GPT_EWORKSPACE = -5, /* workspace missing or smaller than the *_workspace_bytes() value */
  GPT_EDATA = -6       /* input data unusable: an empty document, or the document stream ran out */
} gpt_status;

enum { GPT_KIND_EMB = 0, GPT_KIND_MATRIX = 1, GPT_KIND_LM_HEAD = 2, GPT_KIND_SCALAR = 3, GPT_KIND_GATE = 4 };

typedef struct {
  char name[32];   /* "wte", "h<l>.wq" ... "h<l>.wproj", "lm_head" */
  int64_t offset;  /* element offset into every flat buffer (params, bf16, grads, momentum) */
  int32_t rows;    /* out features (vocab for wte / lm_head) */
  int32_t cols;    /* in features */
  int32_t kind;    /* GPT_KIND_* */
  int32_t layer;   /* block index, -1 for wte and lm_head */
} gpt_tensor;

/*
 * Plan a model from the depth knob ([CT50] "Filosofia: Um Único Seletor Para
 * Controlar Tudo": width, heads and the rest follow from --depth). The rule is
 * not printed on the page; this library uses width d = 64*depth rounded up to
 * a multiple of 128, heads H = d/128 of size 128, MLP hidden 4d.
 *   depth   1..64
 *   vocab   64..262144, multiple of 64 (the pages' tokenizer has 32768)
 *   max_seq 1..16384, the longest sequence later calls may pass
 * On success *out receives a handle to release with gpt_destroy().
 */
gpt_status gpt_create(int32_t depth, int32_t vocab, int32_t max_seq, gpt_model** out);

/*
 * gpt_create with grouped-query attention ([CT50] "1. Modelo GPT" lists
 * attention with fewer KV heads): kv_heads key/value heads of 128, dividing
 * the H query heads; query head h attends with key/value head h / (H / kv_heads).
 * wk and wv become [kv_heads*128, d]. kv_heads = 0 means H (plain multi-head).
 * Returns GPT_EINVAL when kv_heads does not divide H.
 */
gpt_status gpt_create_gqa(int32_t depth, int32_t vocab, int32_t max_seq, int32_t kv_heads, gpt_model** out);
void gpt_destroy(gpt_model* m);

/* Key/value heads of the model (H unless created with fewer). */
int32_t gpt_kv_heads(const gpt_model* m);

/*
 * A model with the optional architecture features of [CT50] "1. Modelo GPT"
 * ("Truques de Eficiência" items 1 and 3; the page prints one line for each):
 *   kv_heads       as for gpt_create_gqa (0: every head)
 *   resid_scalars  1: tensors resid_lambdas [1, depth] and x0_lambdas
 *                  [1, depth]; block i reads resid_lambdas[i] * x +
 *                  x0_lambdas[i] * x0 as its input stream, x0 being the
 *                  embedding output
 *   backout_layer  -1, or k in [0, depth): tensor backout_lambda [1, 1];
 *                  backout_lambda times the stream entering block k (after its
 *                  mix) is subtracted before the final norm
 *   smear          1: tensors smear_gate [1, 24] and smear_lambda [1, 1]
 *                  ("Truques de Eficiência" item 2); the embedding output
 *                  becomes x_t + smear_lambda * sigmoid(smear_gate . x_t[0:24])
 *                  * x_(t-1), x_(-1) = 0 at a sequence's first token (this is
 *                  the x0 of the residual scalars)
 *   ve_layers      bit l set: layer l has a value embedding ("Embeddings de
 *                  Valor (ResFormer)"): tensors h{l}.ve [vocab, kv_heads*128]
 *                  (kind GPT_KIND_EMB) and h{l}.ve_gate [kv_heads, 32] (kind
 *                  GPT_KIND_GATE); v of each key/value head h gets
 *                  3 * sigmoid(ve_gate[h] . xn[0:32]) times the token's row,
 *                  xn being the block's normalised input. kv_heads <= 16.
 *                  These follow lm_head, before the scalar tensors.
 * Scalar tensors (kind GPT_KIND_SCALAR) follow lm_head in the flat layout and
 * belong to the AdamW group; gpt_fwd_bwd reads them from params_bf16 like
 * every weight and writes their gradients. Returns GPT_EINVAL for values out
 * of range.
 */
typedef struct {
  int32_t depth, vocab, max_seq;
  int32_t kv_heads;
  int32_t resid_scalars;
  int32_t backout_layer;
  int32_t smear;
  int64_t ve_layers;
} gpt_config;
gpt_status gpt_create_config(const gpt_config* cfg, gpt_model** out);
/* The backout layer, or -1. */
int32_t gpt_backout_layer(const gpt_model* m);

/* dims[6] <- {depth, width, heads, mlp_hidden, vocab, max_seq}. */
gpt_status gpt_dims(const gpt_model* m, int32_t dims[6]);

/*
 * Attention window of every layer ([CT50] "1. Modelo GPT" lists window
 * attention that alternates short and long context, e.g. "SSSL", and
 * "5. Flash Attention Unificado" passes a window_size to the attention call;
 * the page gives no sizes). windows is a HOST array of n == depth entries:
 * layer l's queries i see keys i - windows[l] .. i; -1 is the full causal
 * context (the default after gpt_create). NULL resets every layer to -1.
 * Returns GPT_ESHAPE if n != depth, GPT_EINVAL for an entry below -1.
 * Later gpt_fwd_bwd calls on this model use the windows.
 */
gpt_status gpt_set_attention_windows(gpt_model* m, const int32_t* windows, int32_t n);
/* windows[0 .. n-1] <- the model's windows (n == depth). */
gpt_status gpt_get_attention_windows(const gpt_model* m, int32_t* windows, int32_t n);

/* Total element count of the flat parameter layout (also of grads / momentum). */
int64_t gpt_num_params(const gpt_model* m);
int32_t gpt_num_tensors(const gpt_model* m);
/* Describe tensor i (0 <= i < gpt_num_tensors) of the canonical order. */
gpt_status gpt_tensor_info(const gpt_model* m, int32_t i, gpt_tensor* out);

/* Bytes of device workspace gpt_fwd_bwd needs for `batch` sequences of length `seq`. */
size_t gpt_workspace_bytes(const gpt_model* m, int32_t batch, int32_t seq);

/*
 * One forward and backward pass over a microbatch ([CT50] "1. Modelo GPT":
 * untied token embedding, pre-norm blocks with RoPE, QK normalisation, causal
 * attention and a ReLU^2 MLP, then the untied head and softmax cross-entropy).
 *   params_bf16  device, [gpt_num_params] bf16 shadow of the fp32 parameters
 *   tokens       device, int32 [batch, seq], ids in [0, vocab)
 *   targets      device, int32 [batch, seq], ids in [0, vocab) or -1 (ignored)
 *   loss         device, 1 float: mean cross-entropy over non-ignored targets
 *   grads        device, fp32 [gpt_num_params], same layout as the parameters
 *   accumulate   0: grads are overwritten; 1: grads are added to (gradient
 *                accumulation over microbatches, as the single-GPU mode in
 *                [HADA] "Requisitos do ambiente de computação" does)
 *   workspace    device, >= gpt_workspace_bytes(m, batch, seq) bytes,
 *                256-byte aligned; holds activations and the sticky error flag
 * batch * seq is at most 524288 tokens (GPT_ESHAPE otherwise).
 * Ids outside the vocabulary set GPT_ETOKEN in the workspace flag; such tokens
 * embed as zeros and such targets are ignored, so the call still completes.
 * Every sum runs in a fixed order (no floating-point atomics), so repeated
 * calls on the same inputs give the same bits; the embedding and
 * value-embedding rows of ids absent from the batch get exact zeros.
 * The weight gradients' split-K reductions run on the model's second stream
 * (as in muon_step; not while launch timing is on); `stream` waits on it
 * before the call returns, so work queued on `stream` afterwards sees every
 * gradient.
 */
gpt_status gpt_fwd_bwd(gpt_model* m, const uint16_t* params_bf16, const int32_t* tokens,
                       const int32_t* targets, int32_t batch, int32_t seq, float* loss,
                       float* grads, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of device workspace muon_step and normuon_step need (each matrix
 * group has its own Newton-Schulz buffers: the groups run concurrently). */
size_t muon_workspace_bytes(const gpt_model* m);

/*
 * One Muon update of every block matrix ([CT50] "2. Otimizador Muon": 2-D
 * matrices take momentum orthogonalised by a Newton-Schulz iteration
 * A = X^T X, B = b A + c A A, X = a X + X B over a table of (a, b, c)).
 * wte and lm_head belong to the page's AdamW group and are left unchanged.
 *   params       device fp32 [gpt_num_params], updated in place
 *   params_bf16  device bf16 shadow, refreshed for the updated matrices
 *   grads        device fp32 gradients
 *   momentum     device fp32 [gpt_num_params], M <- momentum_coef * M + G
 *   ns_coeffs    HOST pointer to ns_steps rows of (a, b, c) floats, or NULL
 *                for the built-in five-row table (gpt_ns_default_coeffs)
 *   ns_steps     1..8 (1..5 with the built-in table; GPT_EINVAL otherwise)
 * Per matrix: X0 = M / (||M||_F + 1e-7), oriented so rows >= cols, ns_steps
 * iterations, W <- W - lr * sqrt(max(1, rows/cols)) * X. The iteration runs
 * with fp32 accumulation; the MFMA operands are bf16 in the first iteration
 * and fp16 in the others (one MFMA product per matrix product), X is kept in
 * fp16 between iterations and the last one writes it in fp32, which keeps the
 * result within about 2e-3 (Gaussian inputs at the block shapes) to 8e-3
 * (small Gaussian matrices) relative L2 of the fp64 iteration.
 * The matrix groups (attention, MLP) run side by side: the first on `stream`,
 * the others on a second stream of the model's (default priority, made on
 * the first call for the device current then) after an event recorded on
 * `stream`; `stream` then waits on an event recorded after them, so work
 * queued on `stream` afterwards sees the whole update. With launch timing
 * on (gpt_profile_enable) the groups run one after the other on `stream`.
 */
gpt_status muon_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                     float* momentum, float lr, float momentum_coef, const float* ns_coeffs,
                     int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The built-in Newton-Schulz table that muon_step and normuon_step use when
 * ns_coeffs is NULL. Rows 1-2: the two (a, b, c) triples the Polar Express
 * list of [CT50] "2. Otimizador Muon" prints before it breaks off. Rows 3-5:
 * the list continued by its own construction (each row the odd quintic
 * a s + b s^3 + c s^5 with the least maximum of |1 - p(s)| over the interval
 * of singular values the earlier rows leave, from [1e-3, 1]).
 *   out       HOST buffer of 3 * max_rows floats (may be NULL), filled row by row
 *   max_rows  rows to copy at most
 * Returns the number of rows of the table (5). Host only; no GPU call.
 */
int32_t gpt_ns_default_coeffs(float* out, int32_t max_rows);

/*
 * Elements of the NorMuon second-moment state: one fp32 per element of the
 * longer side of each block matrix (per row of wq, wo and wfc, per column of
 * wproj; per row of wk and wv, or per column when they have fewer rows than
 * columns under grouped-query attention). Layout: the d x d matrices in the
 * order layer 0 wq, wk, wv, wo, layer 1 wq, ... (d each), then layer 0 wfc,
 * wproj, layer 1 wfc, ... (4d each). With kv_heads < H the first block is
 * layer 0 wq, wo, layer 1 wq, wo, ... (d each), then layer 0 wk, wv, ... (d
 * each), then the MLP pairs.
 */
int64_t normuon_state_elems(const gpt_model* m);

/*
 * muon_step with NorMuon variance reduction ([CT50] "2. Otimizador Muon", the
 * NorMuon paragraph after the iteration). After the iteration, per matrix,
 * with O the orthogonalised update in the stored orientation:
 *   v_mean_i     = mean of O^2 over the shorter side, one per neuron i
 *   state_i     <- beta2 * state_i + (1 - beta2) * v_mean_i
 *   step_i       = 1 / sqrt(max(state_i, 1e-10))
 *   v_norm       = sqrt(sum v_mean_i),  v_norm_new = sqrt(sum v_mean_i step_i^2)
 *   O_i         <- O_i * step_i * v_norm / max(v_norm_new, 1e-10)
 * then W <- W - lr * sqrt(max(1, rows/cols)) * O as in muon_step (the
 * rescaled O keeps its Frobenius norm). The page prints only part of this
 * rule; the averaged dimension, the moving average and v_norm_new are the
 * readings stated here.
 *   second_moment  device fp32 [normuon_state_elems(m)], zero before the
 *                  first step, updated in place
 *   beta2          in [0, 1)
 * Other arguments as for muon_step (same workspace size). Returns GPT_EINVAL
 * for a null second_moment or beta2 outside [0, 1), before any launch.
 */
gpt_status normuon_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                        float* momentum, float* second_moment, float lr, float momentum_coef, float beta2,
                        const float* ns_coeffs, int32_t ns_steps, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Elements of each AdamW moment buffer: wte, then every tensor from lm_head on
 * (lm_head, value embeddings and gates, scalars), in layout order. */
int64_t adamw_state_elems(const gpt_model* m);

/*
 * One AdamW step of wte, lm_head, the value embeddings and their gates, and the
 * scalar tensors ([CT50] "2. Otimizador Muon": embeddings, lm_head and scalars
 * are optimised by AdamW; the page gives no hyperparameters, so all of them
 * are arguments). Per element, with t = step:
 *   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
 *   w <- w - lr * weight_decay * w - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * (decoupled decay scaled by lr, from the weights before the step).
 *   params, params_bf16, grads  as for muon_step; only the AdamW group changes,
 *                               and its bf16 shadow is refreshed
 *   exp_avg, exp_avg_sq         device fp32 [adamw_state_elems(m)]: the moments
 *                               of wte, then of every tensor from lm_head on,
 *                               in layout order; zero before step 1
 *   step                        1-based step count (bias correction)
 * Returns GPT_EINVAL for null pointers, step < 1, betas outside [0, 1),
 * eps < 0 or non-finite lr / weight_decay, before any launch.
 */
gpt_status adamw_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                      float* exp_avg, float* exp_avg_sq, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int32_t step, void* stream);

/* params_bf16 <- round-to-nearest-even bf16 of params, every tensor. */
gpt_status gpt_refresh_bf16(const gpt_model* m, const float* params, uint16_t* params_bf16,
                            void* stream);

/* Synchronise `stream`, then return the device error flag of a gpt_fwd_bwd
 * workspace (GPT_OK or GPT_ETOKEN) from its most recent call, and clear it. */
gpt_status gpt_check(const gpt_model* m, void* workspace, void* stream);

const char* gpt_status_str(gpt_status s);

/*
 * Launch timing (measurement of [CT50] "Métricas para Monitorar": train/mfu
 * and train/tok_per_sec need per-kernel time). When enabled, gpt_fwd_bwd and
 * muon_step record a pair of HIP events on `stream` around every matrix
 * product and attention launch (the events are host runtime objects the
 * model creates once and reuses; no device memory). gpt_profile_read waits
 * for the recorded events and sums, for one category, the elapsed time in
 * milliseconds, the algorithmic FLOPs and the launch count since the last
 * enable/reset. Categories: 0 projection / head / weight-gradient GEMMs,
 * 1 attention forward, 2 attention backward (causal FLOPs, recompute not
 * counted), 3 Newton-Schulz GEMMs (symmetric products count the
 * upper-triangle tiles they compute).
 */
gpt_status gpt_profile_enable(gpt_model* m, int32_t enable);
gpt_status gpt_profile_reset(gpt_model* m);
gpt_status gpt_profile_read(gpt_model* m, int32_t category, double* ms, double* flops,
                            int64_t* launches);

/*
 * Step-level entry points. Each runs one step of the path above on caller
 * buffers with the same kernels gpt_fwd_bwd / muon_step launch; the test
 * suite uses them to compare single steps with the oracle.
 */

/* C[b] (op)= sum_k A[b](m,k) * B[b](n,k) in bf16 x bf16 -> fp32.
 *   a_kmajor: 1 -> A element (m,k) at A[m*lda + k]; 0 -> at A[k*lda + m]
 *   b_kmajor: 1 -> B element (n,k) at B[n*ldb + k]; 0 -> at B[k*ldb + n]
 *   The contiguous dimension of each operand must be a multiple of 8 and
 *   every row 16-byte aligned. N must be a multiple of 4.
 *   out_mode 0: C fp32 = acc; 1: C fp32 += acc; 2: C bf16 = acc;
 *            3: C bf16 = max(acc, 0); 4: C bf16 += acc (bf16 in place).
 *   batch strides are in elements. */
gpt_status gpt_op_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const uint16_t* A,
                       int64_t lda, int64_t stride_a, int32_t a_kmajor, const uint16_t* B,
                       int64_t ldb, int64_t stride_b, int32_t b_kmajor, void* C, int64_t ldc,
                       int64_t stride_c, int32_t out_mode, void* stream);

/* QKV projection with QK-norm and RoPE ([CT50] "1. Modelo GPT": q and k are
 * RMS-normalised per head of 128, then rotated, pair (j, j+64) by angle
 * t * 10000^(-j/64) at position t = row % seq), the step's first product of
 * each block in one launch: qkv = xn w^T, then the q and k heads of every row
 * normalised (eps 1e-6) and rotated, v heads as they are.
 *   xn [batch*seq, d] bf16; w [(heads + 2*kv_heads)*128, d] bf16 (rows:
 *   q heads, k heads, v heads); d a multiple of 32.
 *   Writes qkv [batch*seq, (heads + 2*kv_heads)*128] bf16 and rstd
 *   [batch*seq, heads + kv_heads] fp32 (the norm scales, for the backward).
 *   rope_scratch: device, seq*128 floats (the (cos, sin) table is built
 *   there). All buffers are the caller's; GPT_EINVAL on bad sizes. */
gpt_status gpt_op_qkv_projection(const uint16_t* xn, const uint16_t* w, uint16_t* qkv, float* rstd,
                                 float* rope_scratch, int32_t batch, int32_t seq, int32_t d, int32_t heads,
                                 int32_t kv_heads, void* stream);

/* Causal attention forward over qkv [batch*seq, 3*heads*128] bf16 (q | k | v
 * column blocks, 128 columns per head). Writes o [batch*seq, heads*128] bf16
 * and lse [batch, heads, seq] fp32: the base-2 logarithm of the softmax
 * normaliser sum_j 2^(s_ij), where s_ij = (q_i . k_j) * log2(e) / sqrt(128).
 * window: -1 for the causal mask, else W >= 0: query i sees keys i - W .. i.
 * kv_heads: key/value heads (dividing heads); qkv is then
 * [batch*seq, (heads + 2*kv_heads)*128]. */
gpt_status gpt_op_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int32_t batch,
                                int32_t seq, int32_t heads, int32_t kv_heads, int32_t window, void* stream);

/* Causal attention backward: from qkv, o, lse (as written by the forward with
 * the same window) and dO [batch*seq, heads*128] bf16, write dqkv
 * [batch*seq, (heads + 2*kv_heads)*128] bf16. scratch: device, >= batch*heads*seq
 * floats. */
gpt_status gpt_op_attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse,
                                const uint16_t* dO, uint16_t* dqkv, float* scratch, int32_t batch,
                                int32_t seq, int32_t heads, int32_t kv_heads, int32_t window, void* stream);

/* The same backward through QK-norm and RoPE, as the step runs it: q and k in
 * qkv are rope(norm(x)) as gpt_op_qkv_projection wrote them, rstd its norm
 * scales [batch*seq, heads + kv_heads] and rope_table its (cos, sin) table
 * (seq*128 floats); the q and k parts of dqkv are then gradients w.r.t. the
 * projections x before the norm ([CT50] "1. Modelo GPT"), v's as above. */
gpt_status gpt_op_attention_bwd_qknorm(const uint16_t* qkv, const uint16_t* o, const float* lse,
                                       const uint16_t* dO, const float* rstd, const float* rope_table,
                                       uint16_t* dqkv, float* scratch, int32_t batch, int32_t seq, int32_t heads,
                                       int32_t kv_heads, int32_t window, void* stream);

/* Newton-Schulz on `count` fp32 matrices X [count, rows, cols] (rows >= cols)
 * in place: X0 = X / (||X||_F + 1e-7), then ns_steps iterations with the
 * host table ns_coeffs. scratch >= gpt_op_ns_scratch_bytes(count, rows, cols). */
size_t gpt_op_ns_scratch_bytes(int32_t count, int32_t rows, int32_t cols);
gpt_status gpt_op_newton_schulz(float* X, int32_t count, int32_t rows, int32_t cols,
                                const float* ns_coeffs, int32_t ns_steps, void* scratch,
                                size_t scratch_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it):
 * gpt_op_newton_schulz with its scratch in a fixed device array of
 * GPT_NS_STATIC_SCRATCH_BYTES that the library holds on each device it runs
 * on until the process ends. Nothing is allocated; arguments and result as
 * for gpt_op_newton_schulz (same kernels, same bits). Returns GPT_EWORKSPACE
 * when gpt_op_ns_scratch_bytes(count, rows, cols) exceeds the array (checked
 * on the host before any launch; up to four 1280 x 1280 matrices, or one
 * 5120 x 1280, fit). Every call on a device shares that device's array: calls
 * that overlap on one device (other streams, other host threads) race and must
 * be serialised by the caller. The array keeps the last call's contents;
 * nothing in it needs to start at zero. */
#define GPT_NS_STATIC_SCRATCH_BYTES (128u << 20)
gpt_status gpt_op_newton_schulz_noalloc(float* X, int32_t count, int32_t rows, int32_t cols,
                                        const float* ns_coeffs, int32_t ns_steps, void* stream);

/*
 * BOS-aligned best-fit packing of a document stream into token rows, on the
 * host ([CT50] "4. Carregamento de Dados": each row starts with BOS, rows are
 * filled best-fit with whole documents, and a document is cut to fill a row
 * when none fits). Before each choice the buffer is topped up from the stream
 * to buffer_cap documents; the longest buffered document that fits the space
 * left goes in whole (the earliest among equal lengths); if none fits, the
 * shortest (earliest among equals) fills the row with its first tokens and its
 * tail is dropped. A chosen document leaves the buffer; the others keep their
 * order. Documents carry their own leading BOS; nothing is inserted.
 *   tokens, offsets  HOST: document d is tokens[offsets[d] .. offsets[d+1]),
 *                    d < n_docs; every document non-empty
 *   buffer           HOST int64 [buffer_cap]: ids of the buffered documents in
 *                    order, *buffer_count of them (in/out; start with 0)
 *   next_doc         HOST in/out: the next stream document to buffer (start 0)
 *   rows, row_len    rows to fill and tokens per row (sequence length + 1 for
 *                    inputs and shifted targets)
 *   out              HOST int32 [rows, row_len], written row by row
 *   tokens_cut       HOST out (may be NULL): tokens dropped by cuts in this call
 * The caller owns every array; nothing is allocated, no GPU is used. Returns
 * GPT_EINVAL for null pointers, sizes or a state out of range, GPT_EDATA when
 * an empty document or decreasing offsets reach the buffer or the stream runs
 * out in mid-row; the state is written back either way (the rows before the
 * failing one are complete).
 */
gpt_status gpt_pack_best_fit(const int32_t* tokens, const int64_t* offsets, int64_t n_docs, int64_t* buffer,
                             int32_t* buffer_count, int32_t buffer_cap, int64_t* next_doc, int32_t rows,
                             int32_t row_len, int32_t* out, int64_t* tokens_cut);

/* Measurement probe, not part of the step: launches `blocks` workgroups of
 * 4 waves, each issuing 4 independent chains of `iters` dense bf16 MFMAs
 * (32 x 32 x 16) from registers, and writes the flops the launch performs to
 * *flops (host). Timing the launch on `stream` gives the matrix-core rate the
 * chip sustains (a measured peak beside the published one).
 *   sink  device, >= blocks floats (one value per workgroup, keeps the work live)
 * Returns GPT_EINVAL for blocks or iters < 1 or null pointers. */
gpt_status gpt_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_STEP_GPT_H */
