// Host runtime of the pretraining step: the model plan (shapes and flat
// parameter layout), workspace carving, the launch sequences of gpt_fwd_bwd
// and muon_step, and the C ABI declared in include/gpt.h.
//
// Sources (cited by page title and section):
//   [CT50] dev.to, "Como treinar seu próprio ChatGPT por 50 dólares".
//   [HADA] GeekNews (hada.io) summary of the nanochat launch README.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "common.h"
#include "kernels.h"
#include "attention.h"
#include "optimizer.h"

namespace {

// One timed launch: events recorded on the launch stream around it.
struct ProfSlot {
  hipEvent_t start = nullptr, stop = nullptr;
  int cat = 0;
  double flops = 0.0;
};

}  // namespace

struct gpt_model {
  int depth = 0, d = 0, H = 0, F = 0, V = 0, max_seq = 0;
  int Hkv = 0, dkv = 0;  // key/value heads (Hkv < H: grouped-query attention) and their width
  // Residual scalars and backout: element offsets of resid_lambdas [L],
  // x0_lambdas [L], backout_lambda (-1 when absent); the backout layer.
  int64_t off_rl = -1, off_xl = -1, off_bl = -1, off_scalars = -1, n_scalars = 0;
  int64_t off_sg = -1, off_sl = -1;  // smear_gate [24], smear_lambda (-1 when absent)
  // Value embeddings: per layer, offsets of h{l}.ve [V, dkv] and h{l}.ve_gate [Hkv, 32] (-1: none).
  std::vector<int64_t> ve_off, veg_off;
  bool any_ve = false;
  int backout_layer = -1;
  std::vector<gpt_tensor> tensors;
  int64_t nparams = 0;
  int64_t off_wte = 0, off_layer0 = 0, layer_stride = 0, off_lm = 0;
  // Attention window per layer (-1: the full causal context).
  std::vector<int32_t> windows;
  // Opt-in launch timing (gpt_profile_*): a pool of event pairs, reused.
  bool prof_on = false;
  std::vector<ProfSlot> prof;
  size_t prof_used = 0;
  // Second stream (default priority) on which the Muon step runs its second
  // matrix group beside the first, with fork / join events; made on first
  // use, for the device current then (aux_dev).
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipEvent_t ev_slot[8] = {};  // weight-gradient partials: 4 GEMM done, 4 reduction done
  int aux_dev = -1;
  ~gpt_model() {
    for (auto& s : prof) {
      if (s.start) (void)hipEventDestroy(s.start);
      if (s.stop) (void)hipEventDestroy(s.stop);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
    for (hipEvent_t e : ev_slot)
      if (e) (void)hipEventDestroy(e);
    if (aux) (void)hipStreamDestroy(aux);
  }
};

namespace {

// Brackets one launch with events when profiling is on.
struct ProfScope {
  gpt_model* m;
  hipStream_t s;
  ProfSlot* slot = nullptr;
  ProfScope(gpt_model* m_, hipStream_t s_, int cat, double flops) : m(m_), s(s_) {
    if (!m || !m->prof_on) return;
    if (m->prof_used == m->prof.size()) {
      ProfSlot ns;
      if (hipEventCreate(&ns.start) != hipSuccess || hipEventCreate(&ns.stop) != hipSuccess) return;
      m->prof.push_back(ns);
    }
    slot = &m->prof[m->prof_used++];
    slot->cat = cat;
    slot->flops = flops;
    (void)hipEventRecord(slot->start, s);
  }
  ~ProfScope() {
    if (slot) (void)hipEventRecord(slot->stop, s);
  }
};

enum { PROF_GEMM = 0, PROF_ATTN_FWD = 1, PROF_ATTN_BWD = 2, PROF_NS = 3, PROF_NCAT = 4 };

// Visible (query, key) pairs of one sequence of T under window w (-1: causal).
double attn_pairs(long T, long w) {
  if (w < 0 || w >= T - 1) return 0.5 * T * (T + 1);
  return 0.5 * (w + 1) * (w + 2) + (double)(T - 1 - w) * (w + 1);
}

// Thread-local current model for the GEMM helpers' profiling.
thread_local gpt_model* g_prof_model = nullptr;

// MFMA work a launch executes (a symmetric launch computes only the
// T (T + 1) / 2 upper-triangle tiles of its T x T tile grid).
inline double gemm_flops(const GemmArgs& g) {
  double f = 2.0 * g.M * (double)g.N * g.K * g.batch;
  if (g.sym) {
    const double t = (g.M + 255) / 256;
    f *= (t + 1) / (2.0 * t);
  }
  return f;
}

hipError_t launch_gemm_prof(const GemmArgs& g, hipStream_t s, int cat = PROF_GEMM) {
  ProfScope ps(g_prof_model, s, cat, gemm_flops(g));
  return launch_gemm(g, s);
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Linear carve of one workspace.
struct Carve {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t o = cur;
    cur = align_up(cur + bytes);
    return o;
  }
};

// Offsets of the gpt_fwd_bwd workspace for a (batch, seq).
struct FwdPlan {
  long N = 0;
  int T = 0, B = 0;
  size_t hdr = 0, cs = 0;
  // per-layer saved activations: base offsets of layer 0 and the stride
  size_t xn1 = 0, rstd1 = 0, qkv = 0, rstdqk = 0, o = 0, lse = 0, xn2 = 0, rstd2 = 0, r = 0;
  size_t layer_bytes = 0;
  size_t x = 0, xnf = 0, rstdf = 0, dx = 0, dxb = 0, dxn = 0, du = 0, dO = 0, delta = 0, dqkv = 0;
  size_t logits = 0, loss_rows = 0, part = 0;
  size_t sc_ids = 0, sc_nruns = 0;  // run tables of the ordered embedding scatter (partials in du)
  // residual scalars / backout (0 when the model has none)
  size_t x0 = 0, dx0 = 0, red = 0, xprev = 0, xbo = 0, dback = 0;
  size_t xe = 0, sa = 0, sred = 0;  // smear: embedding output, gate logits, partials
  size_t velog = 0, vedl = 0, vered = 0;  // value embeddings: logits per layer, dlogit, partials
  long nc = 0;       // CE chunk rows
  size_t part_bytes = 0;
  size_t total = 0;
};

struct SplitK {
  int splits = 1;
  int k_chunk = 0;
};

// Split-K for the weight-gradient GEMMs (K = tokens, small outputs). The
// split count fills whole rounds of workgroups over the chip's compute units
// (one 256 x 256 workgroup per CU at a time): it maximises
// tiles * splits / (rounds * CUs), the busy fraction of the last round
// included, preferring fewer splits (less partial-sum traffic) on ties, with
// at least 1024 k per split.
constexpr int kPlanCUs = 256;  // MI355X compute units

SplitK plan_splitk(long out_rows, long out_cols, long K) {
  SplitK s;
  const long tiles = ((out_rows + 255) / 256) * ((out_cols + 255) / 256);
  const long max_by_k = std::max<long>(1, K / 1024);
  long best = 1;
  double best_eff = -1.0;
  for (long sp = 1; sp <= std::min<long>(16, max_by_k); ++sp) {
    const long chunk = ((K + sp - 1) / sp + 63) / 64 * 64;
    const long real = (K + chunk - 1) / chunk;
    const long wgs = tiles * real;
    const long rounds = (wgs + kPlanCUs - 1) / kPlanCUs;
    const double eff = (double)wgs / (double)(rounds * kPlanCUs);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = sp;
    }
  }
  long chunk = (K + best - 1) / best;
  chunk = (chunk + 63) / 64 * 64;
  s.k_chunk = (int)chunk;
  s.splits = (int)((K + chunk - 1) / chunk);
  return s;
}

FwdPlan plan_fwd(const gpt_model& m, int B, int T) {
  FwdPlan p;
  p.B = B;
  p.T = T;
  p.N = (long)B * T;
  const long N = p.N;
  const long d = m.d, F = m.F, H = m.H, V = m.V;
  const long Q = d + 2L * m.dkv;  // qkv row: H q heads, Hkv k heads, Hkv v heads
  Carve c;
  p.hdr = c.take(256);
  p.cs = c.take((size_t)T * 64 * 2 * 4);
  // Per-layer block, laid out once and repeated.
  Carve lc;
  p.xn1 = lc.take(N * d * 2);
  p.rstd1 = lc.take(N * 4);
  p.qkv = lc.take(N * Q * 2);
  p.rstdqk = lc.take(N * (H + m.Hkv) * 4);
  p.o = lc.take(N * d * 2);
  p.lse = lc.take(N * H * 4);
  p.xn2 = lc.take(N * d * 2);
  p.rstd2 = lc.take(N * 4);
  p.r = lc.take(N * F * 2);  // h = relu(u)^2, bf16
  p.layer_bytes = lc.cur;
  const size_t layers_base = c.take(p.layer_bytes * m.depth);
  p.xn1 += layers_base;
  p.rstd1 += layers_base;
  p.qkv += layers_base;
  p.rstdqk += layers_base;
  p.o += layers_base;
  p.lse += layers_base;
  p.xn2 += layers_base;
  p.rstd2 += layers_base;
  p.r += layers_base;
  p.x = c.take(N * d * 4);
  p.xnf = c.take(N * d * 2);
  p.rstdf = c.take(N * 4);
  p.dx = c.take(N * d * 4);
  p.dxb = c.take(N * d * 2);
  p.dxn = c.take(N * d * 4);
  // du also holds the partial rows of the ordered embedding scatters (free by then).
  p.du = c.take(std::max<size_t>((size_t)N * F * 2, scatter_part_bytes(N, d)));
  p.dO = c.take(N * d * 2);
  p.delta = c.take(N * H * 4);
  p.dqkv = c.take(N * Q * 2);
  const long cap_rows = std::max<long>(256, (1L << 30) / (2 * V));
  p.nc = std::min<long>(N, cap_rows);
  p.logits = c.take((size_t)p.nc * V * 2);
  p.loss_rows = c.take(N * 4);
  p.sc_ids = c.take(scatter_ids_bytes(N));
  p.sc_nruns = c.take((size_t)scatter_groups(N) * 4);
  if (m.off_rl >= 0 || m.off_bl >= 0) {
    p.x0 = c.take(N * d * 4);
    p.dx0 = c.take(N * d * 4);
    p.red = c.take((size_t)resid_partials_count() * 8);
  }
  if (m.off_rl >= 0) p.xprev = c.take((size_t)m.depth * N * d * 4);
  if (m.off_bl >= 0) {
    p.xbo = c.take(N * d * 4);
    p.dback = c.take(N * d * 4);
  }
  if (m.any_ve) {
    p.velog = c.take((size_t)m.depth * N * m.Hkv * 4);
    p.vedl = c.take(N * m.Hkv * 4);
    p.vered = c.take((size_t)ve_partials_floats(m.Hkv) * 4);
  }
  if (m.off_sg >= 0) {
    p.xe = c.take(N * d * 4);
    p.sa = c.take(N * 4);
    p.sred = c.take((size_t)smear_partials_floats() * 4);
  }
  size_t part = 0;
  const long shapes[4][2] = {{Q, d}, {d, d}, {F, d}, {d, F}};
  for (auto& sh : shapes) {
    const SplitK s = plan_splitk(sh[0], sh[1], N);
    if (s.splits > 1) part = std::max(part, (size_t)s.splits * sh[0] * sh[1] * 4);
  }
  // One partials slot per weight gradient of a block (their reductions may
  // still run on the second stream when the next one's GEMM starts).
  p.part_bytes = (std::max<size_t>(part, 256) + 255) / 256 * 256;
  p.part = c.take(4 * p.part_bytes);
  p.total = c.cur;
  return p;
}

// Muon groups of a model, each a batch of same-shaped matrices for the
// Newton-Schulz iteration. Without grouped-query attention: the four d x d
// matrices of each layer (wq, wk, wv, wo), then the MLP pair (wfc stored
// [4d, d]; wproj stored [d, 4d], handled transposed). With Hkv < H: wq and
// wo, then wk and wv ([dkv, d], handled transposed), then the MLP pair.
// Layer layout: wq [d, d], wk [dkv, d], wv [dkv, d], wo [d, d], wfc, wproj.
int muon_groups(const gpt_model& m, MuonGroup* out) {
  const long d = m.d, F = m.F, dkv = m.dkv;
  int n = 0;
  if (dkv == d) {
    MuonGroup sq{};
    sq.base = m.off_layer0;
    sq.layer_stride = m.layer_stride;
    sq.per_layer = 4;
    sq.mat_stride = d * d;
    sq.count = 4 * m.depth;
    sq.rows = (int)d;
    sq.cols = (int)d;
    sq.transposed_mask = 0;
    sq.x_rows = d;
    sq.x_cols = d;
    out[n++] = sq;
  } else {
    MuonGroup qo{};  // wq at 0, wo after wk and wv
    qo.base = m.off_layer0;
    qo.layer_stride = m.layer_stride;
    qo.per_layer = 2;
    qo.mat_stride = d * d + 2 * dkv * d;
    qo.count = 2 * m.depth;
    qo.rows = (int)d;
    qo.cols = (int)d;
    qo.transposed_mask = 0;
    qo.x_rows = d;
    qo.x_cols = d;
    out[n++] = qo;
    MuonGroup kv{};  // wk, wv: [dkv, d], wide
    kv.base = m.off_layer0 + d * d;
    kv.layer_stride = m.layer_stride;
    kv.per_layer = 2;
    kv.mat_stride = dkv * d;
    kv.count = 2 * m.depth;
    kv.rows = (int)dkv;
    kv.cols = (int)d;
    kv.transposed_mask = 3;
    kv.x_rows = d;
    kv.x_cols = dkv;
    out[n++] = kv;
  }
  MuonGroup tall{};
  tall.base = m.off_layer0 + 2 * d * d + 2 * dkv * d;
  tall.layer_stride = m.layer_stride;
  tall.per_layer = 2;
  tall.mat_stride = F * d;
  tall.count = 2 * m.depth;
  tall.rows = (int)F;  // wfc; wproj is the transposed one (mask bit 1)
  tall.cols = (int)d;
  tall.transposed_mask = 2;
  tall.x_rows = F;
  tall.x_cols = d;
  out[n++] = tall;
  return n;
}
constexpr int kMaxMuonGroups = 3;

// Newton-Schulz buffers for `count` matrices of xr x xc.
struct NsPlan {
  size_t x32 = 0, xb = 0, xh0 = 0, xh1 = 0, ah = 0, al = 0, bh = 0, bl = 0, part = 0;
  size_t total = 0;
  int nb = 0;
};

// Newton-Schulz buffers: x32 the fp32 X (X0 in, the result out), xb the bf16
// X0 the preparation writes, xh0 / xh1 the fp16 X between iterations
// (ping-pong), ah / al
// and bh / bl the first iteration's A and B as bf16 hi / lo (ah and bh hold
// the fp16 A and B afterwards), part the normalisation partial sums.
NsPlan plan_ns(long count, long xr, long xc, size_t base) {
  NsPlan p;
  Carve c;
  c.cur = base;
  const long nx = count * xr * xc;
  const long na = count * xc * xc;
  p.x32 = c.take(nx * 4);
  p.xb = c.take(nx * 2);
  p.xh0 = c.take(nx * 2);
  p.xh1 = c.take(nx * 2);
  p.ah = c.take(na * 2);
  p.al = c.take(na * 2);
  p.bh = c.take(na * 2);
  p.bl = c.take(na * 2);
  p.nb = 64;
  p.part = c.take(count * p.nb * 4);
  p.total = c.cur;
  return p;
}

// Operand precision of the iterations. Every product accumulates in fp32.
// The first iteration takes bf16 operands: X0 = G / ||G||_F has entries of
// order 1 / sqrt(rows * cols), where fp16 would be subnormal for the larger
// matrices; its A is kept as bf16 hi + lo for the linear term of B. The
// others take fp16 operands (same MFMA rate, 3 more mantissa bits), with A, B
// and X stored in fp16 between them: the a X term of a middle iteration reads
// the same fp16 X its product reads, and only the last writes X in fp32. A CPU
// emulation of exactly these roundings against the fp64 iteration gives a
// relative L2 error of 1.3e-3 to 1.7e-3 for Gaussian and 2.1e-3 to 2.6e-3 for
// 1/k-spectrum matrices at the block shapes (1280 x 1280, 5120 x 1280), and at
// most 5.8e-3 on a small Gaussian 384 x 128; bf16 operands throughout give
// 1.5e-2 to 2.4e-2 on the same Gaussian matrices.
//
// Run ns_steps iterations on prepared X (x32 and xb filled). Result in x32.
hipError_t run_ns(char* ws, const NsPlan& p, int count, long xr, long xc, const float* coeffs,
                  int steps, hipStream_t s) {
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(ws + p.xb);
  uint16_t* xh[2] = {reinterpret_cast<uint16_t*>(ws + p.xh0), reinterpret_cast<uint16_t*>(ws + p.xh1)};
  uint16_t* ah = reinterpret_cast<uint16_t*>(ws + p.ah);
  uint16_t* al = reinterpret_cast<uint16_t*>(ws + p.al);
  uint16_t* bh = reinterpret_cast<uint16_t*>(ws + p.bh);
  uint16_t* bl = reinterpret_cast<uint16_t*>(ws + p.bl);
  float* x32 = reinterpret_cast<float*>(ws + p.x32);
  int cur = 0;  // xh[cur] holds X in fp16 from the second iteration on
  for (int it = 0; it < steps; ++it) {
    const float a = coeffs[3 * it], b = coeffs[3 * it + 1], c = coeffs[3 * it + 2];
    const bool first = it == 0;
    const uint16_t* x = first ? xb : xh[cur];
    // A = X^T X
    GemmArgs g;
    gemm_args_init(g);
    g.a = x; g.b = x;
    g.M = (int)xc; g.N = (int)xc; g.K = (int)xr;
    g.lda = xc; g.ldb = xc; g.sa = xr * xc; g.sb = xr * xc;
    g.a_kmajor = 0; g.b_kmajor = 0;
    g.c = ah; g.c2 = al; g.ldc = xc; g.sc = xc * xc;
    g.batch = count;
    g.sym = 1;  // A is symmetric: upper-triangle tiles only, mirrored on store
    g.epi = first ? EPI_HILO : EPI_H_GRAM;
    hipError_t e = launch_gemm_prof(g, s, PROF_NS);
    if (e != hipSuccess) return e;
    // B = b A + c A A (A symmetric, so A A = A A^T).
    gemm_args_init(g);
    g.a = ah; g.b = ah;
    g.M = (int)xc; g.N = (int)xc; g.K = (int)xc;
    g.lda = xc; g.ldb = xc; g.sa = xc * xc; g.sb = xc * xc;
    g.a_kmajor = 1; g.b_kmajor = 1;
    g.c = bh; g.c2 = bl; g.ldc = xc; g.sc = xc * xc;
    g.d = ah; g.d2 = al; g.ldd = xc; g.sd = xc * xc;
    g.alpha = c; g.beta = b;
    g.batch = count;
    g.sym = 1;  // B = bA + cA^2 is symmetric too
    g.epi = first ? EPI_NS_POLY : EPI_H_NS_POLY;
    e = launch_gemm_prof(g, s, PROF_NS);
    if (e != hipSuccess) return e;
    // X = a X + X B (B symmetric, so X B = X B^T). The first iteration reads
    // the fp32 X0 and writes X in fp16; the middle ones read and write fp16 X
    // only (the other buffer); the last writes the fp32 result.
    const bool last = it == steps - 1;
    uint16_t* xnext = first ? xh[cur] : xh[cur ^ 1];
    gemm_args_init(g);
    g.a = x; g.b = bh;
    g.M = (int)xr; g.N = (int)xc; g.K = (int)xc;
    g.lda = xc; g.ldb = xc; g.sa = xr * xc; g.sb = xc * xc;
    g.a_kmajor = 1; g.b_kmajor = 1;
    g.c = xnext; g.ldc = xc; g.sc = xr * xc;
    g.c3 = (first && !last) ? nullptr : x32;  // the first iteration's fp32 X only when it is also the last
    g.d = first ? (const void*)x32 : (const void*)x; g.ldd = xc; g.sd = xr * xc;
    g.alpha = 1.f; g.beta = a;
    g.batch = count;
    g.epi = first ? EPI_NS_UPDATE : last ? EPI_H_NS_LAST : EPI_H_NS_UPDATE;
    e = launch_gemm_prof(g, s, PROF_NS);
    if (e != hipSuccess) return e;
    if (!first) cur ^= 1;
  }
  return hipSuccess;
}

inline gpt_status hip_status(hipError_t e) {
  if (e == hipSuccess) return GPT_OK;
  std::fprintf(stderr, "gpt: HIP error %s\n", hipGetErrorString(e));
  return GPT_EHIP;
}

#define HIP_TRY(expr)                                \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_status(e_);     \
  } while (0)

// GEMM helpers for the step.
hipError_t gemm_nt(const uint16_t* A, long lda, const uint16_t* B, long ldb, int M, int N, int K,
                   void* C, long ldc, int epi, hipStream_t s, const void* D = nullptr, long ldd = 0) {
  GemmArgs g;
  gemm_args_init(g);
  g.a = A; g.b = B;
  g.M = M; g.N = N; g.K = K;
  g.lda = lda; g.ldb = ldb;
  g.a_kmajor = 1; g.b_kmajor = 1;
  g.c = C; g.ldc = ldc;
  g.d = D; g.ldd = ldd;
  g.epi = epi;
  return launch_gemm_prof(g, s);
}

// C[M,N] (fp32) += A[M,K] . B[N,K]^T: the update of the fp32 residual stream.
hipError_t gemm_nt_add_f32(const uint16_t* A, long lda, const uint16_t* B, long ldb, int M, int N,
                           int K, float* C, long ldc, hipStream_t s) {
  GemmArgs g;
  gemm_args_init(g);
  g.a = A; g.b = B;
  g.M = M; g.N = N; g.K = K;
  g.lda = lda; g.ldb = ldb;
  g.a_kmajor = 1; g.b_kmajor = 1;
  g.c = C; g.ldc = ldc;
  g.epi = EPI_F32_ACC;
  g.beta = 1.f;
  return launch_gemm_prof(g, s);
}

// C[M,N] = A[M,K] . B where B is stored [K][N] (a weight read along its out dim).
hipError_t gemm_nn(const uint16_t* A, long lda, const uint16_t* B, long ldb, int M, int N, int K,
                   void* C, long ldc, int epi, hipStream_t s, const void* D = nullptr, long ldd = 0) {
  GemmArgs g;
  gemm_args_init(g);
  g.a = A; g.b = B;
  g.M = M; g.N = N; g.K = K;
  g.lda = lda; g.ldb = ldb;
  g.a_kmajor = 1; g.b_kmajor = 0;
  g.c = C; g.ldc = ldc;
  g.d = D; g.ldd = ldd;
  g.epi = epi;
  return launch_gemm_prof(g, s);
}

// Weight gradient: G[M,N] (+)= sum_t A[t][m] * B[t][n], A stored [K][M], B [K][N].
// The second stream and its events, for the current device (false: none,
// the groups then run one after the other on the caller's stream).
bool aux_stream(gpt_model* m) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (m->aux) return m->aux_dev == dev;
  if (hipStreamCreateWithFlags(&m->aux, hipStreamNonBlocking) != hipSuccess) {
    m->aux = nullptr;
    return false;
  }
  bool ok = hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming) == hipSuccess;
  for (hipEvent_t& e : m->ev_slot) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
    if (m->ev_join) (void)hipEventDestroy(m->ev_join);
    for (hipEvent_t& e : m->ev_slot) {
      if (e) (void)hipEventDestroy(e);
      e = nullptr;
    }
    (void)hipStreamDestroy(m->aux);
    m->aux = nullptr;
    m->ev_fork = m->ev_join = nullptr;
    return false;
  }
  m->aux_dev = dev;
  return true;
}

// Split-K reductions of the weight gradients on the second stream. Each of a
// block's four weight gradients has its own partials slot; its reduction
// waits on an event recorded after the GEMM and runs beside the main
// stream's next kernels (the attention backward leaves registers and LDS for
// it), and the next GEMM into the same slot waits for it. The caller joins
// the second stream before it returns.
struct SideReduce {
  hipStream_t side = nullptr;
  hipEvent_t* gemm_done = nullptr;  // [4]
  hipEvent_t* red_done = nullptr;   // [4]
  bool used[4] = {};
  bool any = false;
};

hipError_t gemm_wgrad(const uint16_t* A, long lda, const uint16_t* B, long ldb, int M, int N, long K,
                      float* G, int accumulate, float* part, hipStream_t s, SideReduce* side = nullptr,
                      int slot = 0) {
  const SplitK sk = plan_splitk(M, N, K);
  GemmArgs g;
  gemm_args_init(g);
  g.a = A; g.b = B;
  g.M = M; g.N = N; g.K = (int)K;
  g.lda = lda; g.ldb = ldb;
  g.a_kmajor = 0; g.b_kmajor = 0;
  if (sk.splits > 1) {
    g.c = part; g.ldc = N;
    g.splits = sk.splits; g.k_chunk = sk.k_chunk;
    g.s_split = (long)M * N;
    g.epi = EPI_SPLITK;
    hipError_t e = hipSuccess;
    if (side && side->used[slot]) e = hipStreamWaitEvent(s, side->red_done[slot], 0);
    if (e == hipSuccess) e = launch_gemm_prof(g, s);
    if (e != hipSuccess || !side) {
      return e != hipSuccess ? e : launch_splitk_reduce(part, (long)M * N, sk.splits, G, (long)M * N, accumulate, s);
    }
    side->any = true;
    e = hipEventRecord(side->gemm_done[slot], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->side, side->gemm_done[slot], 0);
    if (e == hipSuccess)
      e = launch_splitk_reduce(part, (long)M * N, sk.splits, G, (long)M * N, accumulate, side->side);
    if (e == hipSuccess) e = hipEventRecord(side->red_done[slot], side->side);
    side->used[slot] = true;
    return e;
  }
  g.c = G; g.ldc = N;
  g.epi = EPI_F32_ACC;
  g.alpha = 1.f;
  g.beta = accumulate ? 1.f : 0.f;
  return launch_gemm_prof(g, s);
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* gpt_status_str(gpt_status s) {
  switch (s) {
    case GPT_OK: return "ok";
    case GPT_EINVAL: return "invalid argument";
    case GPT_ESHAPE: return "unsupported shape";
    case GPT_EHIP: return "HIP runtime error";
    case GPT_ETOKEN: return "token or target id outside the vocabulary";
    case GPT_EWORKSPACE: return "workspace missing or too small";
    case GPT_EDATA: return "document data unusable or exhausted";
  }
  return "unknown status";
}

gpt_status gpt_create(int32_t depth, int32_t vocab, int32_t max_seq, gpt_model** out) {
  return gpt_create_gqa(depth, vocab, max_seq, 0, out);
}

gpt_status gpt_create_gqa(int32_t depth, int32_t vocab, int32_t max_seq, int32_t kv_heads, gpt_model** out) {
  gpt_config c{};
  c.depth = depth;
  c.vocab = vocab;
  c.max_seq = max_seq;
  c.kv_heads = kv_heads;
  c.resid_scalars = 0;
  c.backout_layer = -1;
  c.smear = 0;
  c.ve_layers = 0;
  return gpt_create_config(&c, out);
}

gpt_status gpt_create_config(const gpt_config* cfg, gpt_model** out) {
  if (!out) return GPT_EINVAL;
  if (!cfg) {
    *out = nullptr;
    return GPT_EINVAL;
  }
  const int32_t depth = cfg->depth, vocab = cfg->vocab, max_seq = cfg->max_seq, kv_heads = cfg->kv_heads;
  *out = nullptr;
  if (cfg->resid_scalars != 0 && cfg->resid_scalars != 1) return GPT_EINVAL;
  if (cfg->backout_layer < -1 || cfg->backout_layer >= depth) return GPT_EINVAL;
  if (cfg->smear != 0 && cfg->smear != 1) return GPT_EINVAL;
  if (cfg->ve_layers < 0 || (depth < 63 && (cfg->ve_layers >> depth) != 0)) return GPT_EINVAL;
  if (depth < 1 || depth > 64) return GPT_EINVAL;
  if (vocab < 64 || vocab > 262144 || vocab % 64 != 0) return GPT_EINVAL;
  if (max_seq < 1 || max_seq > 16384) return GPT_EINVAL;
  const int d_ = 128 * ((64 * depth + 127) / 128);
  const int H_ = d_ / 128;
  if (kv_heads < 0 || kv_heads > H_ || (kv_heads > 0 && H_ % kv_heads != 0)) return GPT_EINVAL;
  gpt_model* m = new (std::nothrow) gpt_model();
  if (!m) return GPT_EINVAL;
  m->depth = depth;
  m->d = d_;
  m->H = H_;
  m->Hkv = kv_heads > 0 ? kv_heads : H_;
  m->dkv = 128 * m->Hkv;
  m->F = 4 * m->d;
  m->V = vocab;
  m->max_seq = max_seq;
  m->windows.assign(depth, -1);
  const int64_t d = m->d, F = m->F, dkv = m->dkv;
  int64_t off = 0;
  auto add = [&](const std::string& name, int32_t rows, int32_t cols, int32_t kind, int32_t layer) {
    gpt_tensor t{};
    std::snprintf(t.name, sizeof(t.name), "%s", name.c_str());
    t.offset = off;
    t.rows = rows;
    t.cols = cols;
    t.kind = kind;
    t.layer = layer;
    m->tensors.push_back(t);
    off += (int64_t)rows * cols;
  };
  m->off_wte = 0;
  add("wte", vocab, (int32_t)d, GPT_KIND_EMB, -1);
  m->off_layer0 = off;
  for (int l = 0; l < depth; ++l) {
    const std::string p = "h" + std::to_string(l) + ".";
    add(p + "wq", (int32_t)d, (int32_t)d, GPT_KIND_MATRIX, l);
    add(p + "wk", (int32_t)dkv, (int32_t)d, GPT_KIND_MATRIX, l);
    add(p + "wv", (int32_t)dkv, (int32_t)d, GPT_KIND_MATRIX, l);
    add(p + "wo", (int32_t)d, (int32_t)d, GPT_KIND_MATRIX, l);
    add(p + "wfc", (int32_t)F, (int32_t)d, GPT_KIND_MATRIX, l);
    add(p + "wproj", (int32_t)d, (int32_t)F, GPT_KIND_MATRIX, l);
  }
  m->layer_stride = 2 * d * d + 2 * dkv * d + 2 * F * d;
  m->off_lm = off;
  add("lm_head", vocab, (int32_t)d, GPT_KIND_LM_HEAD, -1);
  // Value embeddings (AdamW group, before the scalars so that lm_head and
  // these tables form one 16-byte aligned run).
  m->ve_off.assign(depth, -1);
  m->veg_off.assign(depth, -1);
  if (cfg->ve_layers != 0 && m->Hkv > 16) {
    delete m;
    return GPT_EINVAL;
  }
  for (int l = 0; l < depth; ++l) {
    if (!((cfg->ve_layers >> l) & 1)) continue;
    const std::string p = "h" + std::to_string(l) + ".";
    m->ve_off[l] = off;
    add(p + "ve", vocab, (int32_t)dkv, GPT_KIND_EMB, l);
    m->veg_off[l] = off;
    add(p + "ve_gate", m->Hkv, 32, GPT_KIND_GATE, l);
    m->any_ve = true;
  }
  m->off_scalars = off;
  if (cfg->resid_scalars) {
    m->off_rl = off;
    add("resid_lambdas", 1, depth, GPT_KIND_SCALAR, -1);
    m->off_xl = off;
    add("x0_lambdas", 1, depth, GPT_KIND_SCALAR, -1);
  }
  if (cfg->backout_layer >= 0) {
    m->backout_layer = cfg->backout_layer;
    m->off_bl = off;
    add("backout_lambda", 1, 1, GPT_KIND_SCALAR, -1);
  }
  if (cfg->smear) {
    m->off_sg = off;
    add("smear_gate", 1, 24, GPT_KIND_SCALAR, -1);
    m->off_sl = off;
    add("smear_lambda", 1, 1, GPT_KIND_SCALAR, -1);
  }
  m->n_scalars = off - m->off_scalars;
  m->nparams = off;
  *out = m;
  return GPT_OK;
}

void gpt_destroy(gpt_model* m) { delete m; }

gpt_status gpt_dims(const gpt_model* m, int32_t dims[6]) {
  if (!m || !dims) return GPT_EINVAL;
  dims[0] = m->depth;
  dims[1] = m->d;
  dims[2] = m->H;
  dims[3] = m->F;
  dims[4] = m->V;
  dims[5] = m->max_seq;
  return GPT_OK;
}

int32_t gpt_kv_heads(const gpt_model* m) { return m ? m->Hkv : 0; }
int32_t gpt_backout_layer(const gpt_model* m) { return m ? m->backout_layer : -1; }

int64_t gpt_num_params(const gpt_model* m) { return m ? m->nparams : 0; }
int32_t gpt_num_tensors(const gpt_model* m) { return m ? (int32_t)m->tensors.size() : 0; }

gpt_status gpt_tensor_info(const gpt_model* m, int32_t i, gpt_tensor* out) {
  if (!m || !out || i < 0 || i >= (int32_t)m->tensors.size()) return GPT_EINVAL;
  *out = m->tensors[i];
  return GPT_OK;
}

size_t gpt_workspace_bytes(const gpt_model* m, int32_t batch, int32_t seq) {
  if (!m || batch < 1 || seq < 1 || seq > m->max_seq) return 0;
  return plan_fwd(*m, batch, seq).total;
}

gpt_status gpt_fwd_bwd(gpt_model* m, const uint16_t* pbf, const int32_t* tokens,
                       const int32_t* targets, int32_t batch, int32_t seq, float* loss,
                       float* grads, int32_t accumulate, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!m || !pbf || !tokens || !targets || !loss || !grads) return GPT_EINVAL;
  if (batch < 1 || seq < 1) return GPT_EINVAL;
  if (seq > m->max_seq) return GPT_ESHAPE;
  if ((long)batch * seq > (long)kScatterMaxGroups * 256) return GPT_ESHAPE;
  if (accumulate != 0 && accumulate != 1) return GPT_EINVAL;
  const FwdPlan p = plan_fwd(*m, batch, seq);
  if (!workspace || workspace_bytes < p.total) return GPT_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return GPT_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  g_prof_model = m;
  const long N = p.N;
  const int T = seq, d = m->d, F = m->F, H = m->H, V = m->V, L = m->depth, Hkv = m->Hkv;
  const int Q = d + 2 * m->dkv;  // qkv row width
  int* hdr = reinterpret_cast<int*>(ws + p.hdr);
  int* err = hdr;
  int* n_valid = hdr + 1;
  float* cs = reinterpret_cast<float*>(ws + p.cs);
  auto lay = [&](size_t base, int l) { return ws + base + (size_t)l * p.layer_bytes; };
  float* x = reinterpret_cast<float*>(ws + p.x);
  uint16_t* xnf = reinterpret_cast<uint16_t*>(ws + p.xnf);
  float* rstdf = reinterpret_cast<float*>(ws + p.rstdf);
  float* dx = reinterpret_cast<float*>(ws + p.dx);
  uint16_t* dxb = reinterpret_cast<uint16_t*>(ws + p.dxb);
  float* dxn = reinterpret_cast<float*>(ws + p.dxn);
  uint16_t* du = reinterpret_cast<uint16_t*>(ws + p.du);
  uint16_t* dO = reinterpret_cast<uint16_t*>(ws + p.dO);
  float* delta = reinterpret_cast<float*>(ws + p.delta);
  uint16_t* dqkv = reinterpret_cast<uint16_t*>(ws + p.dqkv);
  uint16_t* logits = reinterpret_cast<uint16_t*>(ws + p.logits);
  float* loss_rows = reinterpret_cast<float*>(ws + p.loss_rows);
  auto part_slot = [&](int k) { return reinterpret_cast<float*>(ws + p.part + (size_t)k * p.part_bytes); };
  // Weight-gradient reductions on the second stream (not while launch timing
  // is on, so that each GEMM launch is timed alone); joined on every return.
  SideReduce side_r;
  SideReduce* side = nullptr;
  if (!m->prof_on && aux_stream(m)) {
    side_r.side = m->aux;
    side_r.gemm_done = m->ev_slot;
    side_r.red_done = m->ev_slot + 4;
    side = &side_r;
  }
  struct JoinSide {
    gpt_model* m;
    SideReduce* side;
    hipStream_t s;
    ~JoinSide() {
      if (side && side->any && hipEventRecord(m->ev_join, m->aux) == hipSuccess)
        (void)hipStreamWaitEvent(s, m->ev_join, 0);
    }
  } join_side{m, side, s};
  const uint16_t* wte = pbf + m->off_wte;
  const uint16_t* wlm = pbf + m->off_lm;

  // ---- prologue
  HIP_TRY(launch_fill_u32(hdr, 0, 2, s));
  HIP_TRY(launch_rope_table(cs, T, s));
  HIP_TRY(launch_count_targets(targets, N, V, n_valid, err, s));
  float* xe = p.xe ? reinterpret_cast<float*>(ws + p.xe) : nullptr;
  float* sa = p.sa ? reinterpret_cast<float*>(ws + p.sa) : nullptr;
  const uint16_t* psg = m->off_sg >= 0 ? pbf + m->off_sg : nullptr;
  const uint16_t* psl = m->off_sl >= 0 ? pbf + m->off_sl : nullptr;
  HIP_TRY(launch_embed_fwd(tokens, wte, xe ? xe : x, err, N, d, V, s));
  // Smear: x_t = xe_t + lambda sigmoid(w . xe_t[0:24]) xe_(t-1).
  if (xe) HIP_TRY(launch_smear_fwd(xe, x, sa, psg, psl, N, T, d, s));
  const long Nd = N * d;
  float* x0 = p.x0 ? reinterpret_cast<float*>(ws + p.x0) : nullptr;
  float* dx0 = p.dx0 ? reinterpret_cast<float*>(ws + p.dx0) : nullptr;
  float2* red = p.red ? reinterpret_cast<float2*>(ws + p.red) : nullptr;
  float* xbo = p.xbo ? reinterpret_cast<float*>(ws + p.xbo) : nullptr;
  float* dback = p.dback ? reinterpret_cast<float*>(ws + p.dback) : nullptr;
  auto xprev = [&](int l) { return reinterpret_cast<float*>(ws + p.xprev) + (size_t)l * Nd; };
  const uint16_t* prl = m->off_rl >= 0 ? pbf + m->off_rl : nullptr;
  const uint16_t* pxl = m->off_xl >= 0 ? pbf + m->off_xl : nullptr;
  const uint16_t* pbl = m->off_bl >= 0 ? pbf + m->off_bl : nullptr;
  if (x0) HIP_TRY(hipMemcpyAsync(x0, x, Nd * 4, hipMemcpyDeviceToDevice, s));
  auto ve_logits = [&](int l) { return reinterpret_cast<float*>(ws + p.velog) + (size_t)l * N * Hkv; };

  // ---- forward through the blocks
  for (int l = 0; l < L; ++l) {
    const uint16_t* W = pbf + m->off_layer0 + (long)l * m->layer_stride;
    const uint16_t* wqkv = W;
    const uint16_t* wo = W + (long)Q * d;
    const uint16_t* wfc = wo + (long)d * d;
    const uint16_t* wproj = wfc + (long)F * d;
    uint16_t* xn1 = reinterpret_cast<uint16_t*>(lay(p.xn1, l));
    float* rstd1 = reinterpret_cast<float*>(lay(p.rstd1, l));
    uint16_t* qkv = reinterpret_cast<uint16_t*>(lay(p.qkv, l));
    float* rstdqk = reinterpret_cast<float*>(lay(p.rstdqk, l));
    uint16_t* o = reinterpret_cast<uint16_t*>(lay(p.o, l));
    float* lse = reinterpret_cast<float*>(lay(p.lse, l));
    uint16_t* xn2 = reinterpret_cast<uint16_t*>(lay(p.xn2, l));
    float* rstd2 = reinterpret_cast<float*>(lay(p.rstd2, l));
    uint16_t* r = reinterpret_cast<uint16_t*>(lay(p.r, l));
    // Residual scalars: the block reads resid_lambdas[l] x + x0_lambdas[l] x0.
    if (prl) HIP_TRY(launch_resid_mix_fwd(x, x0, xprev(l), prl + l, pxl + l, Nd, s));
    if (l == m->backout_layer) HIP_TRY(hipMemcpyAsync(xbo, x, Nd * 4, hipMemcpyDeviceToDevice, s));
    HIP_TRY(launch_rmsnorm_fwd(x, xn1, rstd1, N, d, s));
    {
      // qkv = xn1 Wqkv^T with QK-norm and RoPE applied to the q and k heads in
      // the epilogue (their norm scales to rstdqk).
      GemmArgs g;
      gemm_args_init(g);
      g.a = xn1; g.b = wqkv;
      g.M = (int)N; g.N = Q; g.K = d;
      g.lda = d; g.ldb = d;
      g.a_kmajor = 1; g.b_kmajor = 1;
      g.c = qkv; g.ldc = Q;
      g.epi = EPI_QKN_BF16;
      g.qk_rstd = rstdqk; g.qk_cs = cs; g.qk_T = T; g.qk_heads = H + Hkv;
      HIP_TRY(launch_gemm_prof(g, s));
    }
    if (m->ve_off[l] >= 0)
      HIP_TRY(launch_ve_fwd(qkv, xn1, tokens, pbf + m->ve_off[l], pbf + m->veg_off[l], ve_logits(l), N, d, Hkv, V,
                            s));
    {
      ProfScope ps(m, s, PROF_ATTN_FWD, 4.0 * batch * H * 128.0 * attn_pairs(T, m->windows[l]));
      HIP_TRY(launch_attention_fwd_window(qkv, o, lse, batch, T, H, Hkv, m->windows[l], s));
    }
    HIP_TRY(gemm_nt_add_f32(o, d, wo, d, (int)N, d, d, x, d, s));
    HIP_TRY(launch_rmsnorm_fwd(x, xn2, rstd2, N, d, s));
    // h = relu(u)^2 is stored once; the down projection reads it directly.
    HIP_TRY(gemm_nt(xn2, d, wfc, d, (int)N, F, d, r, F, EPI_RELU2_BF16, s));
    HIP_TRY(gemm_nt_add_f32(r, F, wproj, F, (int)N, d, F, x, d, s));
  }
  // Backout: subtract backout_lambda times the stream kept at the backout block.
  if (pbl) HIP_TRY(launch_axpy_f32(x, xbo, pbl, -1.f, Nd, s));
  HIP_TRY(launch_rmsnorm_fwd(x, xnf, rstdf, N, d, s));

  // ---- head: logits, softmax cross-entropy, and its backward, by token chunks
  float* g_lm = grads + m->off_lm;
  for (long r0 = 0; r0 < N; r0 += p.nc) {
    const int nc = (int)std::min<long>(p.nc, N - r0);
    HIP_TRY(gemm_nt(xnf + r0 * d, d, wlm, d, nc, V, d, logits, V, EPI_BF16, s));
    HIP_TRY(launch_ce_softmax(logits, targets + r0, loss_rows + r0, nc, V, n_valid, s));
    HIP_TRY(gemm_nn(logits, V, wlm, d, nc, d, V, dxn + r0 * d, d, EPI_F32, s));
    {
      GemmArgs g;
      gemm_args_init(g);
      g.a = logits; g.b = xnf + r0 * d;
      g.M = V; g.N = d; g.K = nc;
      g.lda = V; g.ldb = d;
      g.a_kmajor = 0; g.b_kmajor = 0;
      g.c = g_lm; g.ldc = d;
      g.epi = EPI_F32_ACC;
      g.beta = (r0 > 0 || accumulate) ? 1.f : 0.f;
      HIP_TRY(launch_gemm_prof(g, s));
    }
  }
  HIP_TRY(launch_loss_reduce(loss_rows, N, n_valid, loss, s));
  HIP_TRY(launch_rmsnorm_bwd(dxn, xnf, rstdf, dx, dxb, N, d, 0, s));
  if (pbl) HIP_TRY(launch_backout_bwd(dx, xbo, dback, Nd, red, grads + m->off_bl, accumulate, s));
  // Ordered scatter-adds of the embedding and value-embedding table gradients.
  const ScatterWs scw{reinterpret_cast<float*>(ws + p.du), reinterpret_cast<int32_t*>(ws + p.sc_ids),
                      reinterpret_cast<int32_t*>(ws + p.sc_nruns)};
  if (dx0) HIP_TRY(launch_fill_u32(dx0, 0, Nd, s));

  // ---- backward through the blocks
  for (int l = L - 1; l >= 0; --l) {
    const long woff = m->off_layer0 + (long)l * m->layer_stride;
    const uint16_t* W = pbf + woff;
    const uint16_t* wqkv = W;
    const uint16_t* wo = W + (long)Q * d;
    const uint16_t* wfc = wo + (long)d * d;
    const uint16_t* wproj = wfc + (long)F * d;
    float* G = grads + woff;
    float* gqkv = G;
    float* go = G + (long)Q * d;
    float* gfc = go + (long)d * d;
    float* gproj = gfc + (long)F * d;
    const uint16_t* xn1 = reinterpret_cast<const uint16_t*>(lay(p.xn1, l));
    const float* rstd1 = reinterpret_cast<const float*>(lay(p.rstd1, l));
    const uint16_t* qkv = reinterpret_cast<const uint16_t*>(lay(p.qkv, l));
    const float* rstdqk = reinterpret_cast<const float*>(lay(p.rstdqk, l));
    const uint16_t* o = reinterpret_cast<const uint16_t*>(lay(p.o, l));
    const float* lse = reinterpret_cast<const float*>(lay(p.lse, l));
    const uint16_t* xn2 = reinterpret_cast<const uint16_t*>(lay(p.xn2, l));
    const float* rstd2 = reinterpret_cast<const float*>(lay(p.rstd2, l));
    const uint16_t* r = reinterpret_cast<const uint16_t*>(lay(p.r, l));
    // MLP: x_out = x_mid + relu(u)^2 Wproj^T
    HIP_TRY(gemm_nn(dxb, d, wproj, F, (int)N, F, d, du, F, EPI_DRELU2_BF16, s, r, F));
    HIP_TRY(gemm_wgrad(dxb, d, r, F, d, F, N, gproj, accumulate, part_slot(0), s, side, 0));
    HIP_TRY(gemm_nn(du, F, wfc, d, (int)N, d, F, dxn, d, EPI_F32, s));
    HIP_TRY(gemm_wgrad(du, F, xn2, d, F, d, N, gfc, accumulate, part_slot(1), s, side, 1));
    HIP_TRY(launch_rmsnorm_bwd(dxn, xn2, rstd2, dx, dxb, N, d, 1, s));
    // Attention: x_mid = x_in + o Wo^T
    HIP_TRY(gemm_nn(dxb, d, wo, d, (int)N, d, d, dO, d, EPI_BF16, s));
    HIP_TRY(gemm_wgrad(dxb, d, o, d, d, d, N, go, accumulate, part_slot(2), s, side, 2));
    {
      ProfScope ps(m, s, PROF_ATTN_BWD, 10.0 * batch * H * 128.0 * attn_pairs(T, m->windows[l]));
      // dqkv leaves with the QK-norm + RoPE backward applied to its q and k parts.
      HIP_TRY(launch_attention_bwd_window(qkv, o, lse, dO, dqkv, delta, batch, T, H, Hkv, m->windows[l], s,
                                          rstdqk, cs));
    }
    HIP_TRY(gemm_nn(dqkv, Q, wqkv, d, (int)N, d, Q, dxn, d, EPI_F32, s));
    if (m->ve_off[l] >= 0)
      HIP_TRY(launch_ve_bwd(dqkv, xn1, tokens, pbf + m->ve_off[l], pbf + m->veg_off[l], ve_logits(l),
                            grads + m->ve_off[l], reinterpret_cast<float*>(ws + p.vedl),
                            reinterpret_cast<float*>(ws + p.vered), grads + m->veg_off[l], dxn, N, d, Hkv, V,
                            accumulate, scw, s));
    HIP_TRY(gemm_wgrad(dqkv, Q, xn1, d, Q, d, N, gqkv, accumulate, part_slot(3), s, side, 3));
    HIP_TRY(launch_rmsnorm_bwd(dxn, xn1, rstd1, dx, dxb, N, d, 1, s));
    // dx is now the gradient of the stream entering block l.
    if (l == m->backout_layer) HIP_TRY(launch_backout_add(dx, dxb, dback, pbl, Nd, s));
    if (prl)
      HIP_TRY(launch_resid_mix_bwd(dx, dxb, xprev(l), x0, dx0, prl + l, pxl + l, Nd, red, grads + m->off_rl + l,
                                   grads + m->off_xl + l, accumulate, s));
  }

  // ---- embedding gradient (the embedding output is also x0 of every mix)
  if (dx0) HIP_TRY(launch_axpy_f32(dx, dx0, nullptr, 1.f, Nd, s));
  if (xe) {
    // Through the smear into the raw embedding rows (dxn is free here).
    HIP_TRY(launch_smear_bwd(dx, xe, sa, dxn, psg, psl, N, T, d, reinterpret_cast<float*>(ws + p.sred),
                             grads + m->off_sg, grads + m->off_sl, accumulate, s));
    dx = dxn;
  }
  HIP_TRY(launch_embed_bwd(tokens, dx, grads + m->off_wte, N, d, V, accumulate, scw, s));
  return GPT_OK;
}

// Each Muon group has Newton-Schulz buffers of its own (the groups run on two
// streams at once), one after the other; then the NorMuon scratch: per X row
// of each group, the scale and the two norm terms.
static size_t ns_region_end(const MuonGroup& g, size_t base) {
  return (plan_ns(g.count, g.x_rows, g.x_cols, base).total + 255) / 256 * 256;
}
static size_t ns_workspace_bytes(const gpt_model& m, size_t* normuon_off) {
  MuonGroup groups[kMaxMuonGroups];
  const int ng = muon_groups(m, groups);
  size_t off = 0, rows = 0;
  for (int i = 0; i < ng; ++i) {
    off = ns_region_end(groups[i], off);
    rows += (size_t)groups[i].count * groups[i].x_rows;
  }
  if (normuon_off) *normuon_off = off;
  return off + (3 * rows * 4 + 255) / 256 * 256;
}


size_t muon_workspace_bytes(const gpt_model* m) {
  if (!m) return 0;
  return ns_workspace_bytes(*m, nullptr);
}

int64_t normuon_state_elems(const gpt_model* m) {
  if (!m) return 0;
  MuonGroup groups[kMaxMuonGroups];
  const int ng = muon_groups(*m, groups);
  int64_t n = 0;
  for (int i = 0; i < ng; ++i) n += (int64_t)groups[i].count * groups[i].x_rows;
  return n;
}

// Default Newton-Schulz table (rows of a, b, c). Rows 1-2 are the two triples
// printed in the Polar Express list of "2. Otimizador Muon" ([CT50]); the page
// stops there. Rows 3-5 continue the list by the same construction: each row
// is the odd quintic a s + b s^3 + c s^5 minimising max |1 - p(s)| over the
// interval of singular values the rows before it leave, starting from
// [1e-3, 1] (rounded to 6 decimals).
static const float kDefaultNsCoeffs[5][3] = {
    {8.156f, -22.483f, 15.879f},
    {4.043f, -2.809f, 0.500f},
    {3.982257f, -2.970416f, 0.565427f},
    {3.335133f, -2.500934f, 0.511459f},
    {2.315341f, -1.682053f, 0.420229f},
};
constexpr int kDefaultNsRows = 5;

int32_t gpt_ns_default_coeffs(float* out, int32_t max_rows) {
  if (out) {
    for (int r = 0; r < kDefaultNsRows && r < max_rows; ++r)
      for (int c = 0; c < 3; ++c) out[3 * r + c] = kDefaultNsCoeffs[r][c];
  }
  return kDefaultNsRows;
}

// Momentum, Newton-Schulz and the update for both groups; with second_moment,
// NorMuon rescales each group's orthogonalised update before the update.
static gpt_status muon_impl(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                            float* momentum, float* second_moment, float lr, float momentum_coef, float beta2,
                            const float* ns_coeffs, int32_t ns_steps, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!m || !params || !params_bf16 || !grads || !momentum) return GPT_EINVAL;
  if (ns_steps < 1 || ns_steps > 8) return GPT_EINVAL;
  if (!ns_coeffs) {
    if (ns_steps > kDefaultNsRows) return GPT_EINVAL;
    ns_coeffs = &kDefaultNsCoeffs[0][0];
  }
  size_t nm_off = 0;
  if (!workspace || workspace_bytes < ns_workspace_bytes(*m, &nm_off)) return GPT_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return GPT_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  g_prof_model = m;
  MuonGroup groups[kMaxMuonGroups];
  const int ng = muon_groups(*m, groups);
  // One group's chain: momentum, X0, Newton-Schulz, (NorMuon,) update, in its
  // own workspace region and stream.
  auto run_group = [&](int gi, size_t base, float* rs, float* state, hipStream_t sg) -> gpt_status {
    const MuonGroup& g = groups[gi];
    const NsPlan p = plan_ns(g.count, g.x_rows, g.x_cols, base);
    float* part = reinterpret_cast<float*>(ws + p.part);
    float* x32 = reinterpret_cast<float*>(ws + p.x32);
    HIP_TRY(launch_muon_momentum(g, grads, momentum, momentum_coef, part, p.nb, sg));
    HIP_TRY(launch_muon_pack(g, momentum, part, p.nb, x32, reinterpret_cast<uint16_t*>(ws + p.xb), sg));
    HIP_TRY(run_ns(ws, p, g.count, g.x_rows, g.x_cols, ns_coeffs, ns_steps, sg));
    if (state) {
      const long rows = (long)g.count * g.x_rows;
      HIP_TRY(launch_normuon(g, x32, state, beta2, rs, rs + rows, sg));
      HIP_TRY(launch_muon_update_scaled(g, x32, params, params_bf16, lr, rs, sg));
    } else {
      HIP_TRY(launch_muon_update(g, x32, params, params_bf16, lr, sg));
    }
    return GPT_OK;
  };
  // Group 0 on the caller's stream, the others on the second stream after a
  // fork; the caller's stream then waits for them (joined on every path).
  // With launch timing on, the groups run one after the other so that each
  // launch's events time it alone.
  const bool two = ng > 1 && !m->prof_on && aux_stream(m);
  if (two) {
    HIP_TRY(hipEventRecord(m->ev_fork, s));
    HIP_TRY(hipStreamWaitEvent(m->aux, m->ev_fork, 0));
  }
  gpt_status st = GPT_OK;
  size_t base = 0;
  float* rs = reinterpret_cast<float*>(ws + nm_off);
  float* state = second_moment;
  for (int gi = 0; gi < ng && st == GPT_OK; ++gi) {
    st = run_group(gi, base, rs, state, (two && gi > 0) ? m->aux : s);
    const long rows = (long)groups[gi].count * groups[gi].x_rows;
    base = ns_region_end(groups[gi], base);
    rs += 3 * rows;
    if (state) state += rows;
  }
  if (two) {
    const hipError_t e1 = hipEventRecord(m->ev_join, m->aux);
    const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(s, m->ev_join, 0) : e1;
    if (st == GPT_OK && e2 != hipSuccess) st = hip_status(e2);
  }
  return st;
}

gpt_status muon_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                     float* momentum, float lr, float momentum_coef, const float* ns_coeffs,
                     int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream) {
  return muon_impl(m, params, params_bf16, grads, momentum, nullptr, lr, momentum_coef, 0.f, ns_coeffs,
                   ns_steps, workspace, workspace_bytes, stream);
}

gpt_status normuon_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                        float* momentum, float* second_moment, float lr, float momentum_coef, float beta2,
                        const float* ns_coeffs, int32_t ns_steps, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!second_moment || !(beta2 >= 0.f && beta2 < 1.f)) return GPT_EINVAL;
  return muon_impl(m, params, params_bf16, grads, momentum, second_moment, lr, momentum_coef, beta2,
                   ns_coeffs, ns_steps, workspace, workspace_bytes, stream);
}

int64_t adamw_state_elems(const gpt_model* m) {
  if (!m) return 0;
  // wte, then everything from lm_head on (lm_head, value embeddings, scalars).
  return (int64_t)m->V * m->d + (m->nparams - m->off_lm);
}

gpt_status adamw_step(gpt_model* m, float* params, uint16_t* params_bf16, const float* grads,
                      float* exp_avg, float* exp_avg_sq, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int32_t step, void* stream) {
  if (!m || !params || !params_bf16 || !grads || !exp_avg || !exp_avg_sq) return GPT_EINVAL;
  if (step < 1 || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f)) return GPT_EINVAL;
  if (!(eps >= 0.f) || !std::isfinite(lr) || !std::isfinite(weight_decay)) return GPT_EINVAL;
  // The moments' bias corrections, formed in double on the host.
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  if (!(bc1 > 0.0) || !(bc2 > 0.0)) return GPT_EINVAL;
  const long n = (long)m->V * m->d;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long ow = m->off_wte, ol = m->off_lm, os = m->off_scalars;
  HIP_TRY(launch_adamw_range(params + ow, params_bf16 + ow, grads + ow, exp_avg, exp_avg_sq, n, lr, beta1, beta2,
                             eps, weight_decay, (float)bc1, (float)bc2, s));
  // lm_head and the value embeddings: one aligned run (lengths are multiples of 4).
  HIP_TRY(launch_adamw_range(params + ol, params_bf16 + ol, grads + ol, exp_avg + n, exp_avg_sq + n, os - ol, lr,
                             beta1, beta2, eps, weight_decay, (float)bc1, (float)bc2, s));
  if (m->n_scalars > 0) {
    const long ms = n + (os - ol);
    HIP_TRY(launch_adamw_small(params + os, params_bf16 + os, grads + os, exp_avg + ms, exp_avg_sq + ms,
                               (long)m->n_scalars, lr, beta1, beta2, eps, weight_decay, (float)bc1, (float)bc2, s));
  }
  return GPT_OK;
}

gpt_status gpt_refresh_bf16(const gpt_model* m, const float* params, uint16_t* params_bf16,
                            void* stream) {
  if (!m || !params || !params_bf16) return GPT_EINVAL;
  HIP_TRY(launch_f32_to_bf16(params, params_bf16, m->nparams, reinterpret_cast<hipStream_t>(stream)));
  return GPT_OK;
}

gpt_status gpt_check(const gpt_model* m, void* workspace, void* stream) {
  if (!m || !workspace) return GPT_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(hipStreamSynchronize(s));
  int flag = 0;
  HIP_TRY(hipMemcpy(&flag, workspace, sizeof(int), hipMemcpyDeviceToHost));
  if (flag) {
    const int zero = 0;
    HIP_TRY(hipMemcpy(workspace, &zero, sizeof(int), hipMemcpyHostToDevice));
    return GPT_ETOKEN;
  }
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// Step-level entry points
// ---------------------------------------------------------------------------
gpt_status gpt_op_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const uint16_t* A,
                       int64_t lda, int64_t stride_a, int32_t a_kmajor, const uint16_t* B,
                       int64_t ldb, int64_t stride_b, int32_t b_kmajor, void* C, int64_t ldc,
                       int64_t stride_c, int32_t out_mode, void* stream) {
  if (!A || !B || !C || M < 1 || N < 1 || K < 1 || batch < 1) return GPT_EINVAL;
  if (N % 4 != 0 || ldc % 4 != 0) return GPT_ESHAPE;
  if ((a_kmajor ? K : M) % 8 != 0 || (b_kmajor ? K : N) % 8 != 0) return GPT_ESHAPE;
  if (lda % 8 != 0 || ldb % 8 != 0) return GPT_ESHAPE;
  static const int modes[5] = {EPI_F32, EPI_F32_ACC, EPI_BF16, EPI_RELU_BF16, EPI_RESID_BF16};
  if (out_mode < 0 || out_mode > 4) return GPT_EINVAL;
  g_prof_model = nullptr;
  GemmArgs g;
  gemm_args_init(g);
  g.a = A; g.b = B;
  g.M = M; g.N = N; g.K = K;
  g.lda = lda; g.ldb = ldb; g.sa = stride_a; g.sb = stride_b;
  g.a_kmajor = a_kmajor ? 1 : 0; g.b_kmajor = b_kmajor ? 1 : 0;
  g.c = C; g.ldc = ldc; g.sc = stride_c;
  g.batch = batch;
  g.epi = modes[out_mode];
  g.alpha = 1.f;
  g.beta = 1.f;
  HIP_TRY(launch_gemm_prof(g, reinterpret_cast<hipStream_t>(stream)));
  return GPT_OK;
}

gpt_status gpt_op_qkv_projection(const uint16_t* xn, const uint16_t* w, uint16_t* qkv, float* rstd,
                                 float* rope_scratch, int32_t batch, int32_t seq, int32_t d, int32_t heads,
                                 int32_t kv_heads, void* stream) {
  if (!xn || !w || !qkv || !rstd || !rope_scratch || batch < 1 || seq < 1 || d < 32 || d % 32 != 0 ||
      heads < 1 || kv_heads < 1 || heads % kv_heads != 0)
    return GPT_EINVAL;
  const long rows = (long)batch * seq;
  if (rows > INT32_MAX) return GPT_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_rope_table(rope_scratch, seq, s));
  GemmArgs g;
  gemm_args_init(g);
  g.a = xn; g.b = w;
  g.M = (int)rows; g.N = (heads + 2 * kv_heads) * 128; g.K = d;
  g.lda = d; g.ldb = d;
  g.a_kmajor = 1; g.b_kmajor = 1;
  g.c = qkv; g.ldc = g.N;
  g.epi = EPI_QKN_BF16;
  g.qk_rstd = rstd; g.qk_cs = rope_scratch; g.qk_T = seq; g.qk_heads = heads + kv_heads;
  HIP_TRY(launch_gemm_prof(g, s));
  return GPT_OK;
}

gpt_status gpt_op_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int32_t batch,
                                int32_t seq, int32_t heads, int32_t kv_heads, int32_t window, void* stream) {
  if (!qkv || !o || !lse || batch < 1 || seq < 1 || heads < 1 || window < -1) return GPT_EINVAL;
  if (kv_heads < 1 || heads % kv_heads != 0) return GPT_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_attention_fwd_window(qkv, o, lse, batch, seq, heads, kv_heads, window, s));
  return GPT_OK;
}

gpt_status gpt_op_attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse,
                                const uint16_t* dO, uint16_t* dqkv, float* scratch, int32_t batch,
                                int32_t seq, int32_t heads, int32_t kv_heads, int32_t window, void* stream) {
  if (!qkv || !o || !lse || !dO || !dqkv || !scratch || batch < 1 || seq < 1 || heads < 1 || window < -1)
    return GPT_EINVAL;
  if (kv_heads < 1 || heads % kv_heads != 0) return GPT_EINVAL;
  HIP_TRY(launch_attention_bwd_window(qkv, o, lse, dO, dqkv, scratch, batch, seq, heads, kv_heads, window,
                                      reinterpret_cast<hipStream_t>(stream)));
  return GPT_OK;
}

gpt_status gpt_op_attention_bwd_qknorm(const uint16_t* qkv, const uint16_t* o, const float* lse,
                                       const uint16_t* dO, const float* rstd, const float* rope_table,
                                       uint16_t* dqkv, float* scratch, int32_t batch, int32_t seq, int32_t heads,
                                       int32_t kv_heads, int32_t window, void* stream) {
  if (!qkv || !o || !lse || !dO || !rstd || !rope_table || !dqkv || !scratch || batch < 1 || seq < 1 ||
      heads < 1 || window < -1)
    return GPT_EINVAL;
  if (kv_heads < 1 || heads % kv_heads != 0) return GPT_EINVAL;
  HIP_TRY(launch_attention_bwd_window(qkv, o, lse, dO, dqkv, scratch, batch, seq, heads, kv_heads, window,
                                      reinterpret_cast<hipStream_t>(stream), rstd, rope_table));
  return GPT_OK;
}

gpt_status gpt_set_attention_windows(gpt_model* m, const int32_t* windows, int32_t n) {
  if (!m) return GPT_EINVAL;
  if (!windows) {
    m->windows.assign(m->depth, -1);
    return GPT_OK;
  }
  if (n != m->depth) return GPT_ESHAPE;
  for (int i = 0; i < n; ++i)
    if (windows[i] < -1) return GPT_EINVAL;
  m->windows.assign(windows, windows + n);
  return GPT_OK;
}

gpt_status gpt_get_attention_windows(const gpt_model* m, int32_t* windows, int32_t n) {
  if (!m || !windows) return GPT_EINVAL;
  if (n != m->depth) return GPT_ESHAPE;
  for (int i = 0; i < n; ++i) windows[i] = m->windows[i];
  return GPT_OK;
}

size_t gpt_op_ns_scratch_bytes(int32_t count, int32_t rows, int32_t cols) {
  if (count < 1 || rows < 1 || cols < 1) return 0;
  return plan_ns(count, rows, cols, 0).total;
}

// The iteration of gpt_op_newton_schulz on a scratch region already checked
// to hold plan_ns(count, rows, cols).
static gpt_status ns_op_run(float* X, int32_t count, int32_t rows, int32_t cols, const float* ns_coeffs,
                            int32_t ns_steps, char* ws, hipStream_t s) {
  const NsPlan p = plan_ns(count, rows, cols, 0);
  g_prof_model = nullptr;
  float* x32 = reinterpret_cast<float*>(ws + p.x32);
  const long n = (long)rows * cols;
  HIP_TRY(hipMemcpyAsync(x32, X, (size_t)count * n * 4, hipMemcpyDeviceToDevice, s));
  HIP_TRY(launch_ns_prepare(x32, reinterpret_cast<uint16_t*>(ws + p.xb), count, n,
                            reinterpret_cast<float*>(ws + p.part), p.nb, s));
  HIP_TRY(run_ns(ws, p, count, rows, cols, ns_coeffs, ns_steps, s));
  HIP_TRY(hipMemcpyAsync(X, x32, (size_t)count * n * 4, hipMemcpyDeviceToDevice, s));
  return GPT_OK;
}

static gpt_status ns_op_check(const float* X, int32_t count, int32_t rows, int32_t cols,
                              const float* ns_coeffs, int32_t ns_steps) {
  if (!X || !ns_coeffs || count < 1 || rows < 1 || cols < 1 || ns_steps < 1 || ns_steps > 8)
    return GPT_EINVAL;
  if (rows < cols || cols % 8 != 0 || rows % 8 != 0) return GPT_ESHAPE;
  return GPT_OK;
}

gpt_status gpt_op_newton_schulz(float* X, int32_t count, int32_t rows, int32_t cols,
                                const float* ns_coeffs, int32_t ns_steps, void* scratch,
                                size_t scratch_bytes, void* stream) {
  const gpt_status st = ns_op_check(X, count, rows, cols, ns_coeffs, ns_steps);
  if (st != GPT_OK) return st;
  if (!scratch || scratch_bytes < plan_ns(count, rows, cols, 0).total) return GPT_EWORKSPACE;
  return ns_op_run(X, count, rows, cols, ns_coeffs, ns_steps, reinterpret_cast<char*>(scratch),
                   reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Newton-Schulz without a caller-provided scratch: the same kernels on a
// fixed device array. Each device that runs it holds its own copy of the
// array until the process ends; its device address is looked up once per
// device (the host-side name only stands in for the symbol and is never used
// as an address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[GPT_NS_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

gpt_status gpt_op_newton_schulz_noalloc(float* X, int32_t count, int32_t rows, int32_t cols,
                                        const float* ns_coeffs, int32_t ns_steps, void* stream) {
  const gpt_status st = ns_op_check(X, count, rows, cols, ns_coeffs, ns_steps);
  if (st != GPT_OK) return st;
  if (plan_ns(count, rows, cols, 0).total > (size_t)GPT_NS_STATIC_SCRATCH_BYTES) return GPT_EWORKSPACE;
  void* ws = nullptr;
  HIP_TRY(static_scratch(&ws));
  return ns_op_run(X, count, rows, cols, ns_coeffs, ns_steps, reinterpret_cast<char*>(ws),
                   reinterpret_cast<hipStream_t>(stream));
}


// ---------------------------------------------------------------------------
// Launch timing
// ---------------------------------------------------------------------------
gpt_status gpt_profile_enable(gpt_model* m, int32_t enable) {
  if (!m) return GPT_EINVAL;
  m->prof_on = enable != 0;
  m->prof_used = 0;
  return GPT_OK;
}

gpt_status gpt_profile_read(gpt_model* m, int32_t category, double* ms, double* flops,
                            int64_t* launches) {
  if (!m || !ms || !flops || !launches || category < 0 || category >= PROF_NCAT) return GPT_EINVAL;
  *ms = 0.0;
  *flops = 0.0;
  *launches = 0;
  for (size_t i = 0; i < m->prof_used; ++i) {
    ProfSlot& sl = m->prof[i];
    if (sl.cat != category) continue;
    HIP_TRY(hipEventSynchronize(sl.stop));
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, sl.start, sl.stop));
    *ms += t;
    *flops += sl.flops;
    *launches += 1;
  }
  return GPT_OK;
}

gpt_status gpt_profile_reset(gpt_model* m) {
  if (!m) return GPT_EINVAL;
  m->prof_used = 0;
  return GPT_OK;
}

}  // extern "C"
