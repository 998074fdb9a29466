// Memory-bound kernels of the step on gfx950: embedding gather/scatter,
// parameter-free RMSNorm forward/backward, QK-norm + RoPE forward/backward,
// the softmax cross-entropy row pass, and the Muon elementwise passes.
//
// Sources (cited by page title and section):
//   [CT50] dev.to, "Como treinar seu próprio ChatGPT por 50 dólares".
//
// All row kernels use one wave64 per row and 16-byte accesses; statistics and
// reductions are fp32 and reduced with wave shuffles in a fixed order, so
// results are run-to-run deterministic.
#include "common.h"
#include "kernels.h"
#include "optimizer.h"

namespace {

constexpr float RMS_EPS = 1e-6f;

__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = bf_lo(u.x); f[1] = bf_hi(u.x);
  f[2] = bf_lo(u.y); f[3] = bf_hi(u.y);
  f[4] = bf_lo(u.z); f[5] = bf_hi(u.z);
  f[6] = bf_lo(u.w); f[7] = bf_hi(u.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                    pack_bf2(f[6], f[7]));
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = value;
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    out[i] = (uint16_t)f2bf(in[i]);
}

// cs[t][j] = (cos, sin) of t * 10000^(-j/64), angle formed in fp64.
// ([CT50] "1. Modelo GPT" lists RoPE; base 10000 and the half-split pairing
// (j, j + 64) are this library's reading.)
__global__ void rope_table_kernel(float* cs, int T) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * 64) return;
  const int t = i >> 6;
  const int j = i & 63;
  const double theta = exp(-(double)j / 64.0 * log(10000.0));
  double s, c;
  sincos((double)t * theta, &s, &c);
  cs[2 * i] = (float)c;
  cs[2 * i + 1] = (float)s;
}

// x[i] = wte[tok[i]] ([CT50] "1. Modelo GPT": untied input embedding). The
// residual stream x is kept in fp32.
__global__ void embed_fwd_kernel(const int32_t* __restrict__ tok, const uint16_t* __restrict__ wte,
                                 float* __restrict__ x, int* err, long N, int d, int V) {
  const int chunks = d / 8;
  for (long c = blockIdx.x * (long)blockDim.x + threadIdx.x; c < N * chunks;
       c += (long)gridDim.x * blockDim.x) {
    const long i = c / chunks;
    const int k = (int)(c - i * chunks);
    const int t = tok[i];
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t >= 0 && t < V) {
      unpack8(*reinterpret_cast<const uint4*>(wte + (long)t * d + 8 * k), f);
    } else if (k == 0) {
      atomicOr(err, GPT_DEV_ETOKEN);
    }
    float4* dst = reinterpret_cast<float4*>(x + i * d + 8 * k);
    dst[0] = make_float4(f[0], f[1], f[2], f[3]);
    dst[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

// ---------------------------------------------------------------------------
// Row scatter-add with a fixed summation order: out[v] (+)= sum over the
// positions i with idx[i] = v of src row i ([CT50] "1. Modelo GPT": the untied
// input table's gradient, and the value-embedding tables'). Rows of ids that do
// not occur are written as exact zeros (or left as they are when accumulating).
//   scatter_runs_kernel: one workgroup per group of 256 consecutive positions
//     sorts the keys (id, position) in LDS (bitonic), splits them into runs of
//     equal id and sums each run's src rows in position order into a partial
//     row part[group * 256 + run]; run_ids[group * 256 + run] holds its id
//     (ascending within the group) and nruns[group] the number of runs.
//   scatter_merge_kernel: one workgroup per SC_R consecutive ids gathers, for
//     each id, the partial rows of the groups that hold it and adds them in
//     group order.
// No atomics: the result is the same bits on every run. Zipf-skewed ids put
// at most 256 partial rows (one per group) behind the most frequent id.
// ---------------------------------------------------------------------------
constexpr int SC_G = 256;  // positions per group (= threads of the run kernel)
constexpr int SC_R = 1;    // ids per workgroup of the merge kernel (d20: 369 us at 4, 228 at 1)

// Plain fp32 rows [N, ld].
struct ScatterSrcF32 {
  const float* p;
  long ld;
  __device__ __forceinline__ float4 load(long row, int c4) const {
    return reinterpret_cast<const float4*>(p + row * ld)[c4];
  }
};
// Gated value rows of the value-embedding backward: 3 sigmoid(logit[row][h])
// times dv[row][c] (c in head h = c / 128), dv the v block of the bf16 dqkv
// rows (row stride ld, v at column offset 0 of the pointer).
struct ScatterSrcVe {
  const uint16_t* dv;
  long ld;
  const float* logits;
  int Hkv;
  __device__ __forceinline__ float4 load(long row, int c4) const {
    const int c = 4 * c4;
    const float lg = logits[row * Hkv + (c >> 7)];
    const float g = 3.f * (1.f / (1.f + __expf(-lg)));
    const uint2 u = *reinterpret_cast<const uint2*>(dv + row * ld + c);
    return make_float4(g * bf_lo(u.x), g * bf_hi(u.x), g * bf_lo(u.y), g * bf_hi(u.y));
  }
};

template <class Src>
__global__ void __launch_bounds__(SC_G) scatter_runs_kernel(Src src, const int32_t* __restrict__ idx, long N,
                                                             int V, int W4, float* __restrict__ part,
                                                             int32_t* __restrict__ run_ids,
                                                             int32_t* __restrict__ nruns) {
  __shared__ uint32_t key[SC_G];
  __shared__ int run_start[SC_G + 1];
  __shared__ int wave_runs[SC_G / 64], wave_valid[SC_G / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = blockIdx.x;
  const long base = (long)g * SC_G;
  // Key = id << 8 | position in the group; ids outside [0, V) (flagged by the
  // forward) and positions past N sort last and are skipped.
  uint32_t k = 0xffffffffu;
  if (base + t < N) {
    const int id = idx[base + t];
    if (id >= 0 && id < V) k = ((uint32_t)id << 8) | (uint32_t)t;
  }
  key[t] = k;
  __syncthreads();
  for (int size = 2; size <= SC_G; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int j = t ^ stride;
      if (j > t) {
        const uint32_t a = key[t], b = key[j];
        if ((a > b) == ((t & size) == 0)) {
          key[t] = b;
          key[j] = a;
        }
      }
      __syncthreads();
    }
  }
  k = key[t];
  const bool valid = k != 0xffffffffu;
  const bool head = valid && (t == 0 || (key[t - 1] >> 8) != (k >> 8));
  const unsigned long long mh = __ballot(head), mv = __ballot(valid);
  if (lane == 0) {
    wave_runs[wave] = __popcll(mh);
    wave_valid[wave] = __popcll(mv);
  }
  __syncthreads();
  int before = 0, runs = 0, nvalid = 0;
#pragma unroll
  for (int w = 0; w < SC_G / 64; ++w) {
    before += w < wave ? wave_runs[w] : 0;
    runs += wave_runs[w];
    nvalid += wave_valid[w];
  }
  if (head) {
    const int r = before + __popcll(mh & ((1ull << lane) - 1ull));
    run_start[r] = t;
    run_ids[base + r] = (int32_t)(k >> 8);
  }
  if (t == 0) {
    run_start[runs] = nvalid;
    nruns[g] = runs;
  }
  __syncthreads();
  // Work items are (run, 64-float4 column chunk) pairs, dealt round-robin to
  // the waves, so a long run (the most frequent id) spreads over all of them.
  // A run's rows are added in position order, four loads in flight.
  const int nch = (W4 + 63) / 64;
  for (int item = wave; item < runs * nch; item += SC_G / 64) {
    const int r = item / nch;
    const int c4 = (item - r * nch) * 64 + lane;
    if (c4 >= W4) continue;
    const int s0 = run_start[r], s1 = run_start[r + 1];
    float4* dst = reinterpret_cast<float4*>(part + (base + r) * (long)(4 * W4));
    auto add = [](float4& acc, const float4 v) {
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    };
    float4 acc = src.load(base + (key[s0] & 0xffu), c4);
    int j = s0 + 1;
    for (; j + 3 < s1; j += 4) {
      const float4 v0 = src.load(base + (key[j] & 0xffu), c4);
      const float4 v1 = src.load(base + (key[j + 1] & 0xffu), c4);
      const float4 v2 = src.load(base + (key[j + 2] & 0xffu), c4);
      const float4 v3 = src.load(base + (key[j + 3] & 0xffu), c4);
      add(acc, v0);
      add(acc, v1);
      add(acc, v2);
      add(acc, v3);
    }
    for (; j < s1; ++j) add(acc, src.load(base + (key[j] & 0xffu), c4));
    dst[c4] = acc;
  }
}

// Ids v0 .. v0 + SC_R - 1; list (dynamic LDS) holds, per id, the partial-row
// indices of the groups that contain it, in group order.
__global__ void __launch_bounds__(256) scatter_merge_kernel(const float* __restrict__ part,
                                                            const int32_t* __restrict__ run_ids,
                                                            const int32_t* __restrict__ nruns, int G, int V,
                                                            int W4, float* __restrict__ out, int accumulate) {
  extern __shared__ int list[];  // [SC_R][G]
  __shared__ int wave_cnt[4][SC_R];
  __shared__ int count[SC_R];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int v0 = blockIdx.x * SC_R;
  if (t < SC_R) count[t] = 0;
  __syncthreads();
  for (int c0 = 0; c0 < G; c0 += 256) {
    const int g = c0 + t;
    int r_of[SC_R];
#pragma unroll
    for (int i = 0; i < SC_R; ++i) r_of[i] = -1;
    if (g < G) {
      const int32_t* ids = run_ids + (long)g * SC_G;
      int lo = 0, hi = nruns[g];
      while (lo < hi) {  // first run with id >= v0
        const int mid = (lo + hi) >> 1;
        if (ids[mid] < v0) lo = mid + 1; else hi = mid;
      }
      const int n = nruns[g];
      for (int r = lo; r < n && ids[r] < v0 + SC_R; ++r) {
        const int di = ids[r] - v0;
#pragma unroll
        for (int i = 0; i < SC_R; ++i)
          if (di == i) r_of[i] = r;
      }
    }
#pragma unroll
    for (int i = 0; i < SC_R; ++i) {
      const unsigned long long m = __ballot(r_of[i] >= 0);
      if (lane == 0) wave_cnt[wave][i] = __popcll(m);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SC_R; ++i) {
      const unsigned long long m = __ballot(r_of[i] >= 0);
      if (r_of[i] >= 0) {
        int pos = count[i];
        for (int w = 0; w < wave; ++w) pos += wave_cnt[w][i];
        pos += __popcll(m & ((1ull << lane) - 1ull));
        list[i * G + pos] = g * SC_G + r_of[i];
      }
    }
    __syncthreads();
    if (t < SC_R) count[t] += wave_cnt[0][t] + wave_cnt[1][t] + wave_cnt[2][t] + wave_cnt[3][t];
    __syncthreads();
  }
  for (int i = 0; i < SC_R; ++i) {
    const int v = v0 + i;
    if (v >= V) break;
    const int n = count[i];
    const int* li = list + i * G;
    float4* dst = reinterpret_cast<float4*>(out + (long)v * (4 * W4));
    for (int c4 = t; c4 < W4; c4 += 256) {
      float4 acc = accumulate ? dst[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
      for (int e = 0; e < n; ++e) {
        const float4 p = reinterpret_cast<const float4*>(part + (long)li[e] * (4 * W4))[c4];
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
      }
      dst[c4] = acc;
    }
  }
}

// Parameter-free RMSNorm of the fp32 residual stream: xn = bf16(x * rstd),
// rstd = (mean(x^2) + eps)^-1/2.
__global__ void rmsnorm_fwd_kernel(const float* __restrict__ x, uint16_t* __restrict__ xn,
                                   float* __restrict__ rstd, long N, int d) {
  const int lane = threadIdx.x & 63;
  const long row = blockIdx.x * (long)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * d);
  const int chunks = d / 8;
  float ss = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    const float4 a = xr[2 * c], b = xr[2 * c + 1];
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    ss += b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
  }
  ss = warp_sum(ss);
  const float r = rsqrtf(ss / (float)d + RMS_EPS);
  uint16_t* yr = xn + row * d;
  for (int c = lane; c < chunks; c += 64) {
    const float4 a = xr[2 * c], b = xr[2 * c + 1];
    float f[8] = {a.x * r, a.y * r, a.z * r, a.w * r, b.x * r, b.y * r, b.z * r, b.w * r};
    *reinterpret_cast<uint4*>(yr + 8 * c) = pack8(f);
  }
  if (lane == 0) rstd[row] = r;
}

// The same with the row held in registers between the two passes (one read of
// x): lane l holds 8-element chunks l, l + 64, ..., at most MAXC of them.
template <int MAXC>
__global__ void rmsnorm_fwd_reg_kernel(const float* __restrict__ x, uint16_t* __restrict__ xn,
                                       float* __restrict__ rstd, long N, int d) {
  const int lane = threadIdx.x & 63;
  const long row = blockIdx.x * (long)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * d);
  const int chunks = d / 8;
  float4 v[MAXC][2];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      v[i][0] = xr[2 * c];
      v[i][1] = xr[2 * c + 1];
    } else {
      v[i][0] = v[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      ss += v[i][h].x * v[i][h].x + v[i][h].y * v[i][h].y + v[i][h].z * v[i][h].z + v[i][h].w * v[i][h].w;
  ss = warp_sum(ss);
  const float r = rsqrtf(ss / (float)d + RMS_EPS);
  uint16_t* yr = xn + row * d;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      const float4 a = v[i][0], bq = v[i][1];
      float f[8] = {a.x * r, a.y * r, a.z * r, a.w * r, bq.x * r, bq.y * r, bq.z * r, bq.w * r};
      *reinterpret_cast<uint4*>(yr + 8 * c) = pack8(f);
    }
  }
  if (lane == 0) rstd[row] = r;
}

// dx (+)= rstd * (dxn - xn * mean(dxn * xn)); dx_bf16 = bf16(dx).
__global__ void rmsnorm_bwd_kernel(const float* __restrict__ dxn, const uint16_t* __restrict__ xn,
                                   const float* __restrict__ rstd, float* __restrict__ dx,
                                   uint16_t* __restrict__ dxb, long N, int d, int accumulate) {
  const int lane = threadIdx.x & 63;
  const long row = blockIdx.x * (long)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float* gr = dxn + row * d;
  const uint16_t* yr = xn + row * d;
  const int chunks = d / 8;
  float dot = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    float y[8];
    unpack8(*reinterpret_cast<const uint4*>(yr + 8 * c), y);
    const float4 g0 = *reinterpret_cast<const float4*>(gr + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gr + 8 * c + 4);
    dot += g0.x * y[0] + g0.y * y[1] + g0.z * y[2] + g0.w * y[3] + g1.x * y[4] + g1.y * y[5] +
           g1.z * y[6] + g1.w * y[7];
  }
  dot = warp_sum(dot) / (float)d;
  const float r = rstd[row];
  float* dr = dx + row * d;
  uint16_t* br = dxb + row * d;
  for (int c = lane; c < chunks; c += 64) {
    float y[8];
    unpack8(*reinterpret_cast<const uint4*>(yr + 8 * c), y);
    const float4 g0 = *reinterpret_cast<const float4*>(gr + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gr + 8 * c + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float o[8];
    if (accumulate) {
      const float4 a0 = *reinterpret_cast<const float4*>(dr + 8 * c);
      const float4 a1 = *reinterpret_cast<const float4*>(dr + 8 * c + 4);
      const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = a[e] + r * (g[e] - y[e] * dot);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = r * (g[e] - y[e] * dot);
    }
    *reinterpret_cast<float4*>(dr + 8 * c) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dr + 8 * c + 4) = make_float4(o[4], o[5], o[6], o[7]);
    *reinterpret_cast<uint4*>(br + 8 * c) = pack8(o);
  }
}

// The backward with the row held in registers between the two passes (one
// read of dxn and xn); lane l holds chunks l, l + 64, ..., at most MAXC.
template <int MAXC>
__global__ void rmsnorm_bwd_reg_kernel(const float* __restrict__ dxn, const uint16_t* __restrict__ xn,
                                       const float* __restrict__ rstd, float* __restrict__ dx,
                                       uint16_t* __restrict__ dxb, long N, int d, int accumulate) {
  const int lane = threadIdx.x & 63;
  const long row = blockIdx.x * (long)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float4* gr = reinterpret_cast<const float4*>(dxn + row * d);
  const uint16_t* yr = xn + row * d;
  const int chunks = d / 8;
  float4 g[MAXC][2];
  uint4 yb[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      yb[i] = *reinterpret_cast<const uint4*>(yr + 8 * c);
      g[i][0] = gr[2 * c];
      g[i][1] = gr[2 * c + 1];
    } else {
      yb[i] = make_uint4(0, 0, 0, 0);
      g[i][0] = g[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    float y[8];
    unpack8(yb[i], y);
    dot += g[i][0].x * y[0] + g[i][0].y * y[1] + g[i][0].z * y[2] + g[i][0].w * y[3] +
           g[i][1].x * y[4] + g[i][1].y * y[5] + g[i][1].z * y[6] + g[i][1].w * y[7];
  }
  dot = warp_sum(dot) / (float)d;
  const float r = rstd[row];
  float4* dr = reinterpret_cast<float4*>(dx + row * d);
  uint16_t* br = dxb + row * d;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = lane + 64 * i;
    if (c >= chunks) continue;
    float y[8];
    unpack8(yb[i], y);
    const float gg[8] = {g[i][0].x, g[i][0].y, g[i][0].z, g[i][0].w,
                         g[i][1].x, g[i][1].y, g[i][1].z, g[i][1].w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r * (gg[e] - y[e] * dot);
    if (accumulate) {
      const float4 a0 = dr[2 * c], a1 = dr[2 * c + 1];
      o[0] += a0.x; o[1] += a0.y; o[2] += a0.z; o[3] += a0.w;
      o[4] += a1.x; o[5] += a1.y; o[6] += a1.z; o[7] += a1.w;
    }
    dr[2 * c] = make_float4(o[0], o[1], o[2], o[3]);
    dr[2 * c + 1] = make_float4(o[4], o[5], o[6], o[7]);
    *reinterpret_cast<uint4*>(br + 8 * c) = pack8(o);
  }
}

__global__ void count_targets_kernel(const int32_t* __restrict__ tgt, long N, int V, int* counter,
                                     int* err) {
  int local = 0;
  bool bad = false;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < N; i += (long)gridDim.x * blockDim.x) {
    const int t = tgt[i];
    if (t >= 0 && t < V) {
      ++local;
    } else if (t != -1) {
      bad = true;
    }
  }
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o, 64);
  if ((threadIdx.x & 63) == 0 && local) atomicAdd(counter, local);
  if (bad) atomicOr(err, GPT_DEV_ETOKEN);
}

// Softmax cross-entropy over one row of bf16 logits, in place:
//   lse = log sum_j exp(z_j); loss_row = lse - z_t;
//   dz_j = (exp(z_j - lse) - [j == t]) / n_valid, written as bf16.
// Rows whose target is ignored (or invalid) get loss 0 and dz 0.
__global__ void __launch_bounds__(256) ce_softmax_kernel(uint16_t* __restrict__ logits,
                                                         const int32_t* __restrict__ tgt,
                                                         float* __restrict__ loss_rows, int V,
                                                         const int* __restrict__ n_valid) {
  __shared__ float red[2][4];
  const long row = blockIdx.x;
  uint16_t* z = logits + row * (long)V;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  const int chunks = V / 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float m = -INFINITY, s = 0.f;
  for (int c = tid; c < chunks; c += 256) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(z + 8 * c), f);
    float cm = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
    const float nm = fmaxf(m, cm);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += exp2f((f[e] - nm) * GPT_LOG2E);
    s = s * exp2f((m - nm) * GPT_LOG2E) + acc;
    m = nm;
  }
  // Combine (m, s) across the wave, then across the 4 waves. A thread with
  // no chunk (V < 2048) holds (-inf, 0): it adds nothing (exp2 of -inf minus
  // -inf would be NaN).
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const float os = __shfl_xor(s, o, 64);
    const float nm = fmaxf(m, om);
    s = (m == -INFINITY ? 0.f : s * exp2f((m - nm) * GPT_LOG2E)) +
        (om == -INFINITY ? 0.f : os * exp2f((om - nm) * GPT_LOG2E));
    m = nm;
  }
  if (lane == 0) {
    red[0][wave] = m;
    red[1][wave] = s;
  }
  __syncthreads();
  float M = red[0][0], S = 0.f;
  for (int w = 1; w < 4; ++w) M = fmaxf(M, red[0][w]);
  for (int w = 0; w < 4; ++w)
    if (red[0][w] != -INFINITY) S += red[1][w] * exp2f((red[0][w] - M) * GPT_LOG2E);
  const float lse = M + logf(S);
  const int nv = *n_valid;
  const float scale = (valid && nv > 0) ? 1.f / (float)nv : 0.f;
  if (tid == 0) loss_rows[row] = valid ? lse - bf2f(z[t]) : 0.f;
  __syncthreads();  // z[t] read before it is overwritten
  for (int c = tid; c < chunks; c += 256) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(z + 8 * c), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float p = exp2f((f[e] - lse) * GPT_LOG2E);
      if (8 * c + e == t) p -= 1.f;
      f[e] = p * scale;
    }
    *reinterpret_cast<uint4*>(z + 8 * c) = pack8(f);
  }
}

// loss = sum(loss_rows) / n_valid, one workgroup, fixed order.
__global__ void __launch_bounds__(1024) loss_reduce_kernel(const float* __restrict__ rows, long N,
                                                          const int* n_valid, float* loss) {
  __shared__ float red[16];
  // rows is 256-byte aligned (a workspace region): float4 loads, then the tail.
  const long n4 = N / 4;
  const float4* r4 = reinterpret_cast<const float4*>(rows);
  float s = 0.f;
  for (long i = threadIdx.x; i < n4; i += blockDim.x) {
    const float4 v = r4[i];
    s += v.x;
    s += v.y;
    s += v.z;
    s += v.w;
  }
  for (long i = 4 * n4 + threadIdx.x; i < N; i += blockDim.x) s += rows[i];
  s = warp_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
    const int nv = *n_valid;
    *loss = nv > 0 ? tot / (float)nv : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Muon ([CT50] "2. Otimizador Muon")
// ---------------------------------------------------------------------------
__device__ __forceinline__ long muon_mat_offset(const MuonGroup& g, int j) {
  const int layer = j / g.per_layer;
  const int k = j - layer * g.per_layer;
  return g.base + layer * g.layer_stride + k * g.mat_stride;
}

// M <- mu M + G over matrix blockIdx.y; partial sum of squares of the new M.
// A thread walks its float4s with stride gridDim.x * 256, four at a time
// (their loads issued together); the sum of squares keeps the walk's order.
__global__ void muon_momentum_kernel(const MuonGroup g, const float* __restrict__ grads,
                                     float* __restrict__ mom, float mu, float* __restrict__ partials) {
  __shared__ float red[4];
  const int j = blockIdx.y;
  const long off = muon_mat_offset(g, j);
  const long n4 = (long)g.rows * g.cols / 4;
  const float4* gp = reinterpret_cast<const float4*>(grads + off);
  float4* mp = reinterpret_cast<float4*>(mom + off);
  const long stride = (long)gridDim.x * blockDim.x;
  float ss = 0.f;
  auto step = [&](float4 m, const float4 gv, long i) {
    m.x = mu * m.x + gv.x;
    m.y = mu * m.y + gv.y;
    m.z = mu * m.z + gv.z;
    m.w = mu * m.w + gv.w;
    mp[i] = m;
    ss += m.x * m.x + m.y * m.y + m.z * m.z + m.w * m.w;
  };
  long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float4 m[4], gv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      m[u] = mp[i + u * stride];
      gv[u] = gp[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) step(m[u], gv[u], i + u * stride);
  }
  for (; i < n4; i += stride) step(mp[i], gp[i], i);
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[(long)j * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float sum_partials(const float* partials, int j, int nb) {
  float s = 0.f;
  for (int i = 0; i < nb; ++i) s += partials[(long)j * nb + i];
  return s;
}

// X0 element i as fp32 and bf16.
__device__ __forceinline__ void x0_store(float v, float* x32, uint16_t* xb, long i) {
  x32[i] = v;
  xb[i] = (uint16_t)f2bf(v);
}

// Four consecutive elements i .. i+3 (i % 4 == 0) of X0 as fp32 and bf16.
__device__ __forceinline__ void x0_store4(const float (&v)[4], float* x32, uint16_t* xb, long i) {
  *reinterpret_cast<float4*>(x32 + i) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<uint2*>(xb + i) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}

// X = M / (||M||_F + 1e-7) in the tall orientation, as fp32 and bf16.
// X is [x_rows, x_cols]. A matrix flagged in transposed_mask is stored wide,
// as [x_cols, x_rows]; it is transposed through 32x33 LDS tiles.
// Grid: (ceil(x_cols / 128), x_rows / 32, count); 256 threads. A workgroup
// covers 32 rows and up to four 32-column tiles of X; thread t covers row
// t / 8 and columns 4 (t % 8) .. +3 of each tile, its four loads issued
// together.
__global__ void muon_pack_kernel(const MuonGroup g, const float* __restrict__ mom,
                                 const float* __restrict__ partials, int nb, float* __restrict__ x32,
                                 uint16_t* __restrict__ xb) {
  __shared__ float tile[4][32][33];
  const int j = blockIdx.z;
  const long off = muon_mat_offset(g, j);
  const int k = j % g.per_layer;
  const bool tr = (g.transposed_mask >> k) & 1;
  const float inv = 1.f / (sqrtf(sum_partials(partials, j, nb)) + 1e-7f);
  const long xr = g.x_rows, xc = g.x_cols;
  const long xoff = (long)j * xr * xc;
  const float* src = mom + off;
  const int q = threadIdx.x & 7;   // float4 column group
  const int ry = threadIdx.x >> 3;  // 0..31
  const long r0 = blockIdx.y * 32L, c0 = blockIdx.x * 128L;  // X block origin
  const int nsub = (int)min(4L, (xc - c0) / 32);               // workgroup-uniform
  float4 m[4];
  if (!tr) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nsub) m[t] = *reinterpret_cast<const float4*>(src + (r0 + ry) * xc + c0 + 32 * t + 4 * q);
  } else {
    // Stored M[c][r] = X[r][c]; stored rows have x_rows elements. Thread
    // (ry, q) loads stored row c0 + 32 t + ry, X rows r0 + 4q .. +3.
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nsub) m[t] = *reinterpret_cast<const float4*>(src + (c0 + 32 * t + ry) * xr + r0 + 4 * q);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nsub) {
        tile[t][ry][4 * q] = m[t].x;
        tile[t][ry][4 * q + 1] = m[t].y;
        tile[t][ry][4 * q + 2] = m[t].z;
        tile[t][ry][4 * q + 3] = m[t].w;
      }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nsub) m[t] = make_float4(tile[t][4 * q][ry], tile[t][4 * q + 1][ry], tile[t][4 * q + 2][ry],
                                       tile[t][4 * q + 3][ry]);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t < nsub) {
      const float v[4] = {m[t].x * inv, m[t].y * inv, m[t].z * inv, m[t].w * inv};
      x0_store4(v, x32 + xoff, xb + xoff, (r0 + ry) * xc + c0 + 32 * t + 4 * q);
    }
}

// W <- W - lr * sqrt(max(1, rows/cols)) * X in the stored orientation (rows =
// fan-out of the stored matrix); refresh bf16. With row_scale (NorMuon), row r
// of X is first multiplied by row_scale[j * x_rows + r]. Grid and thread
// mapping as muon_pack_kernel (up to four 32x32 tiles of X per workgroup,
// one float4 of each per thread, loads issued together).
__global__ void muon_update_kernel(const MuonGroup g, const float* __restrict__ x32,
                                   float* __restrict__ params, uint16_t* __restrict__ pbf, float lr,
                                   const float* __restrict__ row_scale) {
  __shared__ float tile[4][32][33];
  const int j = blockIdx.z;
  const long off = muon_mat_offset(g, j);
  const int k = j % g.per_layer;
  const bool tr = (g.transposed_mask >> k) & 1;
  const long xr = g.x_rows, xc = g.x_cols;
  const float srows = (float)(tr ? xc : xr), scols = (float)(tr ? xr : xc);
  const float scale = lr * sqrtf(fmaxf(1.f, srows / scols));
  const long xoff = (long)j * xr * xc;
  const int q = threadIdx.x & 7;
  const int ry = threadIdx.x >> 3;
  const long r0 = blockIdx.y * 32L, c0 = blockIdx.x * 128L;  // X block origin
  const int nsub = (int)min(4L, (xc - c0) / 32);               // workgroup-uniform
  const float* rsc = row_scale ? row_scale + (long)j * xr + r0 : nullptr;
  float* w = params + off;
  uint16_t* wb = pbf + off;
  long widx[4];
  float4 xv[4], wv[4];
  // X tile t: rows r0 + ry, columns c0 + 32 t + 4q .. +3.
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    widx[t] = tr ? (c0 + 32 * t + ry) * xr + r0 + 4 * q : (r0 + ry) * xc + c0 + 32 * t + 4 * q;
    if (t < nsub) {
      xv[t] = *reinterpret_cast<const float4*>(x32 + xoff + (r0 + ry) * xc + c0 + 32 * t + 4 * q);
      wv[t] = *reinterpret_cast<const float4*>(w + widx[t]);
    }
  }
  const float sr = rsc ? rsc[ry] : 1.f;
  if (tr) {
    // The stored matrix W[c][r] is written along r: stored row c0 + 32 t +
    // ry, X rows r0 + 4q .. +3, through the LDS tile.
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < nsub) {
        tile[t][ry][4 * q] = sr * xv[t].x;
        tile[t][ry][4 * q + 1] = sr * xv[t].y;
        tile[t][ry][4 * q + 2] = sr * xv[t].z;
        tile[t][ry][4 * q + 3] = sr * xv[t].w;
      }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (t < nsub) {
      float u[4];  // X values for the four stored elements widx .. widx+3
      if (!tr) {
        u[0] = sr * xv[t].x; u[1] = sr * xv[t].y; u[2] = sr * xv[t].z; u[3] = sr * xv[t].w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = tile[t][4 * q + e][ry];
      }
      float4 nv = wv[t];
      nv.x -= scale * u[0];
      nv.y -= scale * u[1];
      nv.z -= scale * u[2];
      nv.w -= scale * u[3];
      *reinterpret_cast<float4*>(w + widx[t]) = nv;
      *reinterpret_cast<uint2*>(wb + widx[t]) = make_uint2(pack_bf2(nv.x, nv.y), pack_bf2(nv.z, nv.w));
    }
}

// NorMuon ([CT50] "2. Otimizador Muon", variance reduction after the
// iteration). Statistics are per row of X, the tall orientation, i.e. per
// element of the stored matrix's longer side; the mean runs over x_cols.
// Pass 1, one wave per X row: v_mean = mean(X_r^2); the moving average
// v <- beta2 v + (1 - beta2) v_mean; step_r = 1 / sqrt(max(v, 1e-10)).
// Writes step_r to rs and the row's terms of the two norms (v_mean and
// v_mean * step_r^2) to terms[0] / terms[1] ([count, x_rows] each).
// Grid: (x_rows / 4, count); 256 threads.
__global__ void normuon_stats_kernel(const MuonGroup g, const float* __restrict__ x32,
                                     float* __restrict__ state, float beta2, float* __restrict__ rs,
                                     float* __restrict__ terms) {
  const int j = blockIdx.y;
  const long xr = g.x_rows, xc = g.x_cols;
  const long r = blockIdx.x * 4L + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const float4* row = reinterpret_cast<const float4*>(x32 + ((long)j * xr + r) * xc);
  float ss = 0.f;
  for (long c = lane; c < xc / 4; c += 64) {
    const float4 v = row[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = warp_sum(ss);
  if (lane == 0) {
    const long i = (long)j * xr + r;
    const float vmean = ss / (float)xc;
    const float v = beta2 * state[i] + (1.f - beta2) * vmean;
    state[i] = v;
    const float st = 1.f / sqrtf(fmaxf(v, 1e-10f));
    rs[i] = st;
    terms[i] = vmean;
    terms[(long)g.count * xr + i] = vmean * st * st;
  }
}

// Pass 2, one workgroup per matrix: v_norm = sqrt(sum v_mean), v_norm_new =
// sqrt(sum v_mean step^2); rs_r <- step_r * v_norm / max(v_norm_new, 1e-10).
// Each thread sums a fixed stride of rows, so the result is deterministic.
// Grid: (count); 256 threads.
__global__ void normuon_scale_kernel(const MuonGroup g, float* __restrict__ rs,
                                     const float* __restrict__ terms) {
  __shared__ float red[2][4];
  const int j = blockIdx.x;
  const long xr = g.x_rows;
  const float* a = terms + (long)j * xr;
  const float* b = terms + ((long)g.count + j) * xr;
  float sa = 0.f, sb = 0.f;
  for (long r = threadIdx.x; r < xr; r += blockDim.x) {
    sa += a[r];
    sb += b[r];
  }
  sa = warp_sum(sa);
  sb = warp_sum(sb);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = sa;
    red[1][threadIdx.x >> 6] = sb;
  }
  __syncthreads();
  const float ta = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  const float tb = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float ratio = sqrtf(ta) / fmaxf(sqrtf(tb), 1e-10f);
  for (long r = threadIdx.x; r < xr; r += blockDim.x) rs[(long)j * xr + r] *= ratio;
}

// ---------------------------------------------------------------------------
// Residual scalars and backout ([CT50] "Truques de Eficiência", items 1 and
// 3). The scalars are read from the bf16 weight copy the step computes with.
// ---------------------------------------------------------------------------
// Before block i: x_prev <- x; x <- a x + b x0 (a = resid_lambdas[i],
// b = x0_lambdas[i]). n4 float4 groups.
__global__ void resid_mix_fwd_kernel(float* __restrict__ x, const float* __restrict__ x0,
                                     float* __restrict__ x_prev, const uint16_t* __restrict__ pa,
                                     const uint16_t* __restrict__ pb, long n4) {
  const float a = bf2f(*pa), b = bf2f(*pb);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    const float4 z = reinterpret_cast<const float4*>(x0)[i];
    reinterpret_cast<float4*>(x_prev)[i] = v;
    reinterpret_cast<float4*>(x)[i] =
        make_float4(a * v.x + b * z.x, a * v.y + b * z.y, a * v.z + b * z.z, a * v.w + b * z.w);
  }
}

// y <- y + c * x over n4 float4 groups, c = scale * (bf16 scalar at pc, or 1
// when pc is null).
__global__ void axpy_f32_kernel(float* __restrict__ y, const float* __restrict__ x,
                                const uint16_t* __restrict__ pc, float scale, long n4) {
  const float c = scale * (pc ? bf2f(*pc) : 1.f);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    float4 v = reinterpret_cast<float4*>(y)[i];
    const float4 u = reinterpret_cast<const float4*>(x)[i];
    v.x += c * u.x;
    v.y += c * u.y;
    v.z += c * u.z;
    v.w += c * u.w;
    reinterpret_cast<float4*>(y)[i] = v;
  }
}

// Fixed-order block sum of two values; thread 0 writes both to out[blockIdx.x].
__device__ __forceinline__ void block_sum2(float s0, float s1, float2* out) {
  __shared__ float red[2][4];
  s0 = warp_sum(s0);
  s1 = warp_sum(s1);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = s0;
    red[1][threadIdx.x >> 6] = s1;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    out[blockIdx.x] = make_float2(red[0][0] + red[0][1] + red[0][2] + red[0][3],
                                  red[1][0] + red[1][1] + red[1][2] + red[1][3]);
}

// Backward of the mix before block i, with g = dx (gradient of the mixed
// stream): partial sums of g . x_prev (d a) and g . x0 (d b); dx0 += b g;
// dx <- a g and its bf16 copy. 256 threads per block; partials[blockIdx.x].
__global__ void __launch_bounds__(256) resid_mix_bwd_kernel(float* __restrict__ dx, uint16_t* __restrict__ dxb,
                                                            const float* __restrict__ x_prev,
                                                            const float* __restrict__ x0, float* __restrict__ dx0,
                                                            const uint16_t* __restrict__ pa,
                                                            const uint16_t* __restrict__ pb, long n4,
                                                            float2* __restrict__ partials) {
  const float a = bf2f(*pa), b = bf2f(*pb);
  float s0 = 0.f, s1 = 0.f;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    const float4 g = reinterpret_cast<const float4*>(dx)[i];
    const float4 xp = reinterpret_cast<const float4*>(x_prev)[i];
    const float4 z = reinterpret_cast<const float4*>(x0)[i];
    float4 d0 = reinterpret_cast<float4*>(dx0)[i];
    s0 += g.x * xp.x + g.y * xp.y + g.z * xp.z + g.w * xp.w;
    s1 += g.x * z.x + g.y * z.y + g.z * z.z + g.w * z.w;
    d0.x += b * g.x;
    d0.y += b * g.y;
    d0.z += b * g.z;
    d0.w += b * g.w;
    reinterpret_cast<float4*>(dx0)[i] = d0;
    const float o[4] = {a * g.x, a * g.y, a * g.z, a * g.w};
    reinterpret_cast<float4*>(dx)[i] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint2*>(dxb)[i] = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
  }
  block_sum2(s0, s1, partials);
}

// Backout, top of the backward (g = dx, gradient of the final stream):
// partial sums of g . x_backout; keep dback <- g.
__global__ void __launch_bounds__(256) backout_bwd_kernel(const float* __restrict__ dx,
                                                          const float* __restrict__ xbo, float* __restrict__ dback,
                                                          long n4, float2* __restrict__ partials) {
  float s0 = 0.f;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    const float4 g = reinterpret_cast<const float4*>(dx)[i];
    const float4 v = reinterpret_cast<const float4*>(xbo)[i];
    s0 += g.x * v.x + g.y * v.y + g.z * v.z + g.w * v.w;
    reinterpret_cast<float4*>(dback)[i] = g;
  }
  block_sum2(s0, 0.f, partials);
}

// At the backout block: dx += -c dback (c = backout_lambda) and refresh dxb.
__global__ void backout_add_kernel(float* __restrict__ dx, uint16_t* __restrict__ dxb,
                                   const float* __restrict__ dback, const uint16_t* __restrict__ pc, long n4) {
  const float c = -bf2f(*pc);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    float4 v = reinterpret_cast<float4*>(dx)[i];
    const float4 u = reinterpret_cast<const float4*>(dback)[i];
    const float o[4] = {v.x + c * u.x, v.y + c * u.y, v.z + c * u.z, v.w + c * u.w};
    reinterpret_cast<float4*>(dx)[i] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint2*>(dxb)[i] = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
  }
}

// Scalar gradients from the partials, summed in block order by one thread
// per output: out0 (+)= sign0 * sum .x, out1 (+)= sign1 * sum .y (out1 may be
// null).
__global__ void scalar_grads_kernel(const float2* __restrict__ partials, int nb, float* out0, float sign0,
                                    float* out1, float sign1, int accumulate) {
  if (threadIdx.x > 1) return;
  float* out = threadIdx.x == 0 ? out0 : out1;
  if (!out) return;
  float t = 0.f;
  for (int i = 0; i < nb; ++i) t += threadIdx.x == 0 ? partials[i].x : partials[i].y;
  t *= threadIdx.x == 0 ? sign0 : sign1;
  *out = accumulate ? *out + t : t;
}

// AdamW on a small contiguous fp32 tensor (the scalars), one element per
// thread, no alignment assumed; same update as adamw_kernel.
__global__ void adamw_small_kernel(float* __restrict__ w, uint16_t* __restrict__ wb, const float* __restrict__ g,
                                   float* __restrict__ m, float* __restrict__ v, long n, float lr, float b1,
                                   float b2, float eps, float wd, float bc1, float bc2) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gv = g[i];
  const float mv = b1 * m[i] + (1.f - b1) * gv;
  const float vv = b2 * v[i] + (1.f - b2) * (gv * gv);
  m[i] = mv;
  v[i] = vv;
  const float wv = w[i] - lr * wd * w[i] - lr * (mv / bc1) / (sqrtf(vv / bc2) + eps);
  w[i] = wv;
  wb[i] = (uint16_t)f2bf(wv);
}

// Smear ([CT50] "Truques de Eficiência", item 2): y_t = x_t + gate_t x_(t-1),
// gate_t = lambda * sigmoid(w . x_t[0:24]), x_(-1) = 0 at a sequence's first
// token. One wave per row (token); rows are b * T + t.
constexpr int SMEAR_CH = 24;

__global__ void __launch_bounds__(256) smear_fwd_kernel(const float* __restrict__ xe, float* __restrict__ x,
                                                        float* __restrict__ a_out, const uint16_t* __restrict__ pw,
                                                        const uint16_t* __restrict__ plam, long N, int T, int d) {
  const long row = blockIdx.x * 4L + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const int t = (int)(row % T);
  const float4* xr = reinterpret_cast<const float4*>(xe + row * d);
  float part = 0.f;
  if (lane < SMEAR_CH / 4) {
    const float4 v = xr[lane];
    part = v.x * bf2f(pw[4 * lane]) + v.y * bf2f(pw[4 * lane + 1]) + v.z * bf2f(pw[4 * lane + 2]) +
           v.w * bf2f(pw[4 * lane + 3]);
  }
  const float a = warp_sum(part);
  const float g = t > 0 ? bf2f(*plam) / (1.f + __expf(-a)) : 0.f;
  const float4* pr = reinterpret_cast<const float4*>(xe + (row - (t > 0 ? 1 : 0)) * d);
  float4* yr = reinterpret_cast<float4*>(x + row * d);
  for (int c = lane; c < d / 4; c += 64) {
    const float4 v = xr[c], u = pr[c];
    yr[c] = make_float4(v.x + g * u.x, v.y + g * u.y, v.z + g * u.z, v.w + g * u.w);
  }
  if (lane == 0) a_out[row] = a;
}

// Backward, with dy the gradient of the smeared stream: per row,
// s_t = dy_t . x_(t-1), c_t = lambda sig(a_t) (1 - sig(a_t)) s_t,
// dx_t = dy_t + gate_(t+1) dy_(t+1) + c_t w (on channels 0..23). Block
// partials of d lambda = sum sig(a_t) s_t and d w = sum c_t x_t[0:24] go to
// partials[blockIdx.x][25]. Grid-stride over rows, 4 waves per block.
__global__ void __launch_bounds__(256) smear_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ xe,
                                                        const float* __restrict__ a_in, float* __restrict__ dxo,
                                                        const uint16_t* __restrict__ pw,
                                                        const uint16_t* __restrict__ plam, long N, int T, int d,
                                                        float* __restrict__ partials) {
  __shared__ float red[4][SMEAR_CH + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float lam = bf2f(*plam);
  float acc_l = 0.f;
  float acc_w[4] = {0.f, 0.f, 0.f, 0.f};  // channels 4 lane .. 4 lane + 3 (lanes < 6)
  for (long row = blockIdx.x * 4L + wave; row < N; row += gridDim.x * 4L) {
    const int t = (int)(row % T);
    const float4* g0 = reinterpret_cast<const float4*>(dy + row * d);
    float s = 0.f;
    if (t > 0) {
      const float4* xp = reinterpret_cast<const float4*>(xe + (row - 1) * d);
      for (int c = lane; c < d / 4; c += 64) {
        const float4 u = g0[c], v = xp[c];
        s += u.x * v.x + u.y * v.y + u.z * v.z + u.w * v.w;
      }
    }
    s = warp_sum(s);
    const float sig = 1.f / (1.f + __expf(-a_in[row]));
    const float cc = lam * sig * (1.f - sig) * s;
    const bool has_next = t + 1 < T && row + 1 < N;
    const float gn = has_next ? lam / (1.f + __expf(-a_in[row + 1])) : 0.f;
    const float4* g1 = reinterpret_cast<const float4*>(dy + (row + (has_next ? 1 : 0)) * d);
    float4* out = reinterpret_cast<float4*>(dxo + row * d);
    for (int c = lane; c < d / 4; c += 64) {
      const float4 u = g0[c], v = g1[c];
      float4 o = make_float4(u.x + gn * v.x, u.y + gn * v.y, u.z + gn * v.z, u.w + gn * v.w);
      if (c < SMEAR_CH / 4) {
        o.x += cc * bf2f(pw[4 * c]);
        o.y += cc * bf2f(pw[4 * c + 1]);
        o.z += cc * bf2f(pw[4 * c + 2]);
        o.w += cc * bf2f(pw[4 * c + 3]);
      }
      out[c] = o;
    }
    acc_l += sig * s;
    if (lane < SMEAR_CH / 4) {
      const float4 xv = reinterpret_cast<const float4*>(xe + row * d)[lane];
      acc_w[0] += cc * xv.x;
      acc_w[1] += cc * xv.y;
      acc_w[2] += cc * xv.z;
      acc_w[3] += cc * xv.w;
    }
  }
  // Every lane of a wave holds the same acc_l (s and sig are wave-uniform).
  if (lane == 0) red[wave][SMEAR_CH] = acc_l;
  if (lane < SMEAR_CH / 4)
    for (int k = 0; k < 4; ++k) red[wave][4 * lane + k] = acc_w[k];
  __syncthreads();
  if (threadIdx.x < SMEAR_CH + 1)
    partials[blockIdx.x * (SMEAR_CH + 1) + threadIdx.x] =
        red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

// grads (+)= column sums of partials [nb][25]: smear_gate (24) then smear_lambda.
__global__ void smear_grads_kernel(const float* __restrict__ partials, int nb, float* gw, float* glam,
                                   int accumulate) {
  const int k = threadIdx.x;
  if (k > SMEAR_CH) return;
  float t = 0.f;
  for (int i = 0; i < nb; ++i) t += partials[i * (SMEAR_CH + 1) + k];
  float* out = k < SMEAR_CH ? gw + k : glam;
  *out = accumulate ? *out + t : t;
}

// Value embeddings ([CT50] "Embeddings de Valor (ResFormer)"): per token
// row and key/value head h, logit_h = ve_gate[h] . xn[0:32], and
// v_h += 3 sigmoid(logit_h) * ve[token][h*128 .. h*128+127]. v lives in qkv
// ([N, (H + 2 Hkv) * 128] bf16, columns d + dkv ..); xn is the block's
// normalised input (bf16 [N, d]). One wave per row; logits saved [N, Hkv].
constexpr int VE_CH = 32;

__global__ void __launch_bounds__(256) ve_fwd_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ xn,
                                                     const int32_t* __restrict__ tok,
                                                     const uint16_t* __restrict__ table,
                                                     const uint16_t* __restrict__ gate, float* __restrict__ logits,
                                                     long N, int d, int Hkv, int V) {
  const long row = blockIdx.x * 4L + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const int dkv = Hkv * 128;
  const float xj = lane < VE_CH ? bf2f(xn[row * d + lane]) : 0.f;
  const int t = tok[row];
  const bool ok = t >= 0 && t < V;
  uint16_t* v = qkv + row * (long)(d + 2 * dkv) + d + dkv;
  const uint16_t* e = table + (long)(ok ? t : 0) * dkv;
  for (int h = 0; h < Hkv; ++h) {
    const float lg = warp_sum(lane < VE_CH ? bf2f(gate[h * VE_CH + lane]) * xj : 0.f);
    if (lane == 0) logits[row * Hkv + h] = lg;
    const float g = ok ? 3.f / (1.f + __expf(-lg)) : 0.f;
    // 128 elements of head h: 16 chunks of 8, lanes 0..15.
    if (lane < 16) {
      const int c = h * 128 + 8 * lane;
      float a[8], b[8];
      unpack8(*reinterpret_cast<const uint4*>(v + c), a);
      unpack8(*reinterpret_cast<const uint4*>(e + c), b);
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] += g * b[k];
      *reinterpret_cast<uint4*>(v + c) = pack8(a);
    }
  }
}

// Backward with dv the gradient of v (in dqkv): per row and head,
// s_h = dv_h . ve_h, dlogit_h = 3 sig (1 - sig) s_h (saved [N, Hkv]);
// block partials of d ve_gate[h][j] = sum dlogit_h xn[j] go to
// partials[blockIdx.x][Hkv*32]. (The table gradient, the rows 3 sig dv_h
// summed per token, is the ordered scatter below.)
// Grid-stride over rows, one wave per row, 4 waves per block.
__global__ void __launch_bounds__(256) ve_bwd_kernel(const uint16_t* __restrict__ dqkv,
                                                     const uint16_t* __restrict__ xn,
                                                     const int32_t* __restrict__ tok,
                                                     const uint16_t* __restrict__ table,
                                                     const float* __restrict__ logits,
                                                     float* __restrict__ dlogit, float* __restrict__ partials,
                                                     long N, int d, int Hkv, int V) {
  __shared__ float red[4][16 * VE_CH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int dkv = Hkv * 128;
  float acc[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) acc[h] = 0.f;
  for (long row = blockIdx.x * 4L + wave; row < N; row += gridDim.x * 4L) {
    const int t = tok[row];
    const bool ok = t >= 0 && t < V;
    const uint16_t* dv = dqkv + row * (long)(d + 2 * dkv) + d + dkv;
    const uint16_t* e = table + (long)(ok ? t : 0) * dkv;
    const float xj = lane < VE_CH ? bf2f(xn[row * d + lane]) : 0.f;
#pragma unroll
    for (int h = 0; h < 16; ++h) {  // unrolled so that acc[h] stays in registers
      if (h >= Hkv) break;
      const float lg = logits[row * Hkv + h];
      const float sig = 1.f / (1.f + __expf(-lg));
      float part = 0.f;
      if (lane < 16) {
        const int c = h * 128 + 8 * lane;
        float a[8], b[8];
        unpack8(*reinterpret_cast<const uint4*>(dv + c), a);
        unpack8(*reinterpret_cast<const uint4*>(e + c), b);
#pragma unroll
        for (int k = 0; k < 8; ++k) part += a[k] * b[k];
      }
      const float sh = warp_sum(part);
      const float dl = ok ? 3.f * sig * (1.f - sig) * sh : 0.f;
      if (lane == 0) dlogit[row * Hkv + h] = dl;
      acc[h] += dl * xj;
    }
  }
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < Hkv && lane < VE_CH) red[wave][h * VE_CH + lane] = acc[h];
  __syncthreads();
  for (int i = threadIdx.x; i < Hkv * VE_CH; i += blockDim.x)
    partials[(long)blockIdx.x * Hkv * VE_CH + i] = red[0][i] + red[1][i] + red[2][i] + red[3][i];
}

// dxn[row][j] += sum_h dlogit[row][h] * ve_gate[h][j], j < 32.
__global__ void ve_dxn_kernel(float* __restrict__ dxn, const float* __restrict__ dlogit,
                              const uint16_t* __restrict__ gate, long N, int d, int Hkv) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (i >= N * VE_CH) return;
  const long row = i / VE_CH;
  const int j = (int)(i - row * VE_CH);
  float a = 0.f;
  for (int h = 0; h < Hkv; ++h) a += dlogit[row * Hkv + h] * bf2f(gate[h * VE_CH + j]);
  dxn[row * d + j] += a;
}

// grads (+)= column sums of partials [nb][n] in block order.
__global__ void column_sums_kernel(const float* __restrict__ partials, int nb, int n, float* out, int accumulate) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  float t = 0.f;
  for (int i = 0; i < nb; ++i) t += partials[(long)i * n + k];
  out[k] = accumulate ? out[k] + t : t;
}

// AdamW on one contiguous fp32 tensor and its moments ([CT50] "2. Otimizador
// Muon": embeddings and lm_head are in the AdamW group). Decoupled decay scaled
// by lr and taken from the weights before the step; bias corrections
// bc1 = 1 - beta1^t, bc2 = 1 - beta2^t come from the host. Tensor y of the
// grid's y dimension is at w + woff[y], with moments at state + y * n.
struct AdamwArgs {
  float* w;
  uint16_t* wb;
  const float* g;
  float* m;
  float* v;
  long woff[2];
  long n;
  float lr, b1, b2, eps, wd, bc1, bc2;
};

__global__ void adamw_kernel(const AdamwArgs a) {
  const long base = a.woff[blockIdx.y];
  float* __restrict__ w = a.w + base;
  uint16_t* __restrict__ wb = a.wb + base;
  const float* __restrict__ g = a.g + base;
  float* __restrict__ m = a.m + (long)blockIdx.y * a.n;
  float* __restrict__ v = a.v + (long)blockIdx.y * a.n;
  const long n4 = a.n / 4;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    const float4 gg = reinterpret_cast<const float4*>(g)[i];
    float4 mm = reinterpret_cast<float4*>(m)[i];
    float4 vv = reinterpret_cast<float4*>(v)[i];
    float4 ww = reinterpret_cast<float4*>(w)[i];
    float gv[4] = {gg.x, gg.y, gg.z, gg.w};
    float mv[4] = {mm.x, mm.y, mm.z, mm.w};
    float vv4[4] = {vv.x, vv.y, vv.z, vv.w};
    float wv[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mv[e] = a.b1 * mv[e] + (1.f - a.b1) * gv[e];
      vv4[e] = a.b2 * vv4[e] + (1.f - a.b2) * (gv[e] * gv[e]);
      const float mhat = mv[e] / a.bc1;
      const float vhat = vv4[e] / a.bc2;
      wv[e] = wv[e] - a.lr * a.wd * wv[e] - a.lr * mhat / (sqrtf(vhat) + a.eps);
    }
    reinterpret_cast<float4*>(m)[i] = make_float4(mv[0], mv[1], mv[2], mv[3]);
    reinterpret_cast<float4*>(v)[i] = make_float4(vv4[0], vv4[1], vv4[2], vv4[3]);
    reinterpret_cast<float4*>(w)[i] = make_float4(wv[0], wv[1], wv[2], wv[3]);
    reinterpret_cast<uint2*>(wb)[i] = make_uint2(pack_bf2(wv[0], wv[1]), pack_bf2(wv[2], wv[3]));
  }
}

// Sum of squares of each of `count` contiguous matrices of n elements.
__global__ void sumsq_kernel(const float* __restrict__ x, long n, float* __restrict__ partials) {
  __shared__ float red[4];
  const int j = blockIdx.y;
  const float* p = x + (long)j * n;
  float ss = 0.f;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    ss += p[i] * p[i];
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[(long)j * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ void ns_normalize_kernel(float* __restrict__ x32, uint16_t* __restrict__ xb, long n,
                                    const float* __restrict__ partials, int nb) {
  const int j = blockIdx.y;
  const float inv = 1.f / (sqrtf(sum_partials(partials, j, nb)) + 1e-7f);
  const long base = (long)j * n;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    x0_store(x32[base + i] * inv, x32, xb, base + i);
}

inline int grid_for(long work, int per_block, int cap = 16384) {
  long b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (int)b;
}

}  // namespace

hipError_t launch_fill_u32(void* p, uint32_t value, long n_words, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n_words, 256)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), value, n_words);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* cs, int T, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3((T * 64 + 255) / 256), dim3(256), 0, s, cs, T);
  return hipGetLastError();
}

hipError_t launch_embed_fwd(const int32_t* tok, const uint16_t* wte, float* x, int* err, long N,
                            int d, int V, hipStream_t s) {
  hipLaunchKernelGGL(embed_fwd_kernel, dim3(grid_for(N * (d / 8), 256)), dim3(256), 0, s, tok, wte, x,
                     err, N, d, V);
  return hipGetLastError();
}

namespace {
template <class Src>
hipError_t launch_scatter(const Src& src, const int32_t* idx, long N, int V, int W, float* out, int accumulate,
                          const ScatterWs& ws, hipStream_t s) {
  if (N <= 0) return accumulate ? hipSuccess : launch_fill_u32(out, 0, (long)V * W, s);
  if (W % 4 != 0 || V >= (1 << 24)) return hipErrorInvalidValue;
  const int G = (int)((N + SC_G - 1) / SC_G);
  if (G > kScatterMaxGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scatter_runs_kernel<Src>, dim3(G), dim3(SC_G), 0, s, src, idx, N, V, W / 4, ws.part,
                     ws.run_ids, ws.nruns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scatter_merge_kernel, dim3((V + SC_R - 1) / SC_R), dim3(256), (size_t)SC_R * G * sizeof(int), s,
                     static_cast<const float*>(ws.part), static_cast<const int32_t*>(ws.run_ids),
                     static_cast<const int32_t*>(ws.nruns), G, V, W / 4, out, accumulate);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_embed_bwd(const int32_t* tok, const float* dx, float* dwte, long N, int d, int V, int accumulate,
                            const ScatterWs& ws, hipStream_t s) {
  return launch_scatter(ScatterSrcF32{dx, (long)d}, tok, N, V, d, dwte, accumulate, ws, s);
}

hipError_t launch_ve_table_bwd(const uint16_t* dqkv, long ld, const float* logits, int Hkv, const int32_t* tok,
                               long N, int V, float* dtable, int accumulate, const ScatterWs& ws, hipStream_t s) {
  return launch_scatter(ScatterSrcVe{dqkv, ld, logits, Hkv}, tok, N, V, Hkv * 128, dtable, accumulate, ws, s);
}

hipError_t launch_rmsnorm_fwd(const float* x, uint16_t* xn, float* rstd, long N, int d,
                              hipStream_t s) {
  const dim3 grid((unsigned)((N + 3) / 4));
  switch ((d / 8 + 63) / 64) {
    case 1: hipLaunchKernelGGL(rmsnorm_fwd_reg_kernel<1>, grid, dim3(256), 0, s, x, xn, rstd, N, d); break;
    case 2: hipLaunchKernelGGL(rmsnorm_fwd_reg_kernel<2>, grid, dim3(256), 0, s, x, xn, rstd, N, d); break;
    case 3: hipLaunchKernelGGL(rmsnorm_fwd_reg_kernel<3>, grid, dim3(256), 0, s, x, xn, rstd, N, d); break;
    case 4: hipLaunchKernelGGL(rmsnorm_fwd_reg_kernel<4>, grid, dim3(256), 0, s, x, xn, rstd, N, d); break;
    default: hipLaunchKernelGGL(rmsnorm_fwd_kernel, grid, dim3(256), 0, s, x, xn, rstd, N, d); break;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const float* dxn, const uint16_t* xn, const float* rstd, float* dx,
                              uint16_t* dx_bf16, long N, int d, int accumulate, hipStream_t s) {
  const dim3 grid((unsigned)((N + 3) / 4));
#define RMSB(C) hipLaunchKernelGGL(rmsnorm_bwd_reg_kernel<C>, grid, dim3(256), 0, s, dxn, xn, rstd, dx, dx_bf16, \
                                   N, d, accumulate)
  switch ((d / 8 + 63) / 64) {
    case 1: RMSB(1); break;
    case 2: RMSB(2); break;
    case 3: RMSB(3); break;
    case 4: RMSB(4); break;
    default:
      hipLaunchKernelGGL(rmsnorm_bwd_kernel, grid, dim3(256), 0, s, dxn, xn, rstd, dx, dx_bf16, N, d,
                         accumulate);
      break;
  }
#undef RMSB
  return hipGetLastError();
}



hipError_t launch_count_targets(const int32_t* tgt, long N, int V, int* counter, int* err,
                                hipStream_t s) {
  hipLaunchKernelGGL(count_targets_kernel, dim3(grid_for(N, 256, 1024)), dim3(256), 0, s, tgt, N, V,
                     counter, err);
  return hipGetLastError();
}

hipError_t launch_ce_softmax(uint16_t* logits, const int32_t* tgt, float* loss_rows, long rows,
                             int V, const int* n_valid, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(ce_softmax_kernel, dim3((unsigned)rows), dim3(256), 0, s, logits, tgt, loss_rows,
                     V, n_valid);
  return hipGetLastError();
}

hipError_t launch_loss_reduce(const float* loss_rows, long N, const int* n_valid, float* loss,
                              hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, s, loss_rows, N, n_valid, loss);
  return hipGetLastError();
}

hipError_t launch_muon_momentum(const MuonGroup& g, const float* grads, float* mom, float mu,
                                float* partials, int blocks_per_mat, hipStream_t s) {
  hipLaunchKernelGGL(muon_momentum_kernel, dim3(blocks_per_mat, g.count), dim3(256), 0, s, g, grads,
                     mom, mu, partials);
  return hipGetLastError();
}

hipError_t launch_muon_pack(const MuonGroup& g, const float* mom, const float* partials,
                            int blocks_per_mat, float* x32, uint16_t* xb, hipStream_t s) {
  dim3 grid((unsigned)((g.x_cols + 127) / 128), (unsigned)(g.x_rows / 32), g.count);
  hipLaunchKernelGGL(muon_pack_kernel, grid, dim3(256), 0, s, g, mom, partials, blocks_per_mat, x32, xb);
  return hipGetLastError();
}

hipError_t launch_muon_update(const MuonGroup& g, const float* x32, float* params,
                              uint16_t* params_bf16, float lr, hipStream_t s) {
  dim3 grid((unsigned)((g.x_cols + 127) / 128), (unsigned)(g.x_rows / 32), g.count);
  hipLaunchKernelGGL(muon_update_kernel, grid, dim3(256), 0, s, g, x32, params, params_bf16, lr,
                     static_cast<const float*>(nullptr));
  return hipGetLastError();
}

hipError_t launch_normuon(const MuonGroup& g, const float* x32, float* state, float beta2, float* rs,
                          float* terms, hipStream_t s) {
  hipLaunchKernelGGL(normuon_stats_kernel, dim3((unsigned)(g.x_rows / 4), g.count), dim3(256), 0, s, g, x32,
                     state, beta2, rs, terms);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(normuon_scale_kernel, dim3(g.count), dim3(256), 0, s, g, rs,
                     static_cast<const float*>(terms));
  return hipGetLastError();
}

hipError_t launch_muon_update_scaled(const MuonGroup& g, const float* x32, float* params,
                                     uint16_t* params_bf16, float lr, const float* row_scale, hipStream_t s) {
  dim3 grid((unsigned)((g.x_cols + 127) / 128), (unsigned)(g.x_rows / 32), g.count);
  hipLaunchKernelGGL(muon_update_kernel, grid, dim3(256), 0, s, g, x32, params, params_bf16, lr, row_scale);
  return hipGetLastError();
}

hipError_t launch_adamw(float* w, uint16_t* wb, const float* g, float* m, float* v, long off0, long off1,
                        long n, float lr, float b1, float b2, float eps, float wd, float bc1, float bc2,
                        hipStream_t s) {
  AdamwArgs a;
  a.w = w; a.wb = wb; a.g = g; a.m = m; a.v = v;
  a.woff[0] = off0; a.woff[1] = off1;
  a.n = n;
  a.lr = lr; a.b1 = b1; a.b2 = b2; a.eps = eps; a.wd = wd; a.bc1 = bc1; a.bc2 = bc2;
  hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(n / 4, 256, 2048), 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ns_prepare(float* x32, uint16_t* xb, int count, long n, float* partials,
                             int blocks_per_mat, hipStream_t s) {
  hipLaunchKernelGGL(sumsq_kernel, dim3(blocks_per_mat, count), dim3(256), 0, s, x32, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ns_normalize_kernel, dim3(grid_for(n, 256, 1024), count), dim3(256), 0, s, x32, xb, n,
                     partials, blocks_per_mat);
  return hipGetLastError();
}

// ---- residual scalars and backout
namespace {
constexpr int kRedBlocks = 1024;  // blocks of the two-value reductions (partials buffer size)
}
int resid_partials_count() { return kRedBlocks; }

hipError_t launch_resid_mix_fwd(float* x, const float* x0, float* x_prev, const uint16_t* pa, const uint16_t* pb,
                                long n, hipStream_t s) {
  hipLaunchKernelGGL(resid_mix_fwd_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, x, x0, x_prev, pa, pb,
                     n / 4);
  return hipGetLastError();
}

hipError_t launch_axpy_f32(float* y, const float* x, const uint16_t* pc, float scale, long n, hipStream_t s) {
  hipLaunchKernelGGL(axpy_f32_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, y, x, pc, scale, n / 4);
  return hipGetLastError();
}

hipError_t launch_resid_mix_bwd(float* dx, uint16_t* dxb, const float* x_prev, const float* x0, float* dx0,
                                const uint16_t* pa, const uint16_t* pb, long n, float2* partials, float* ga,
                                float* gb, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(resid_mix_bwd_kernel, dim3(kRedBlocks), dim3(256), 0, s, dx, dxb, x_prev, x0, dx0, pa, pb,
                     n / 4, partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scalar_grads_kernel, dim3(1), dim3(64), 0, s, static_cast<const float2*>(partials),
                     kRedBlocks, ga, 1.f, gb, 1.f, accumulate);
  return hipGetLastError();
}

hipError_t launch_backout_bwd(const float* dx, const float* xbo, float* dback, long n, float2* partials,
                              float* gc, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(backout_bwd_kernel, dim3(kRedBlocks), dim3(256), 0, s, dx, xbo, dback, n / 4, partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scalar_grads_kernel, dim3(1), dim3(64), 0, s, static_cast<const float2*>(partials),
                     kRedBlocks, gc, -1.f, static_cast<float*>(nullptr), 0.f, accumulate);
  return hipGetLastError();
}

hipError_t launch_backout_add(float* dx, uint16_t* dxb, const float* dback, const uint16_t* pc, long n,
                              hipStream_t s) {
  hipLaunchKernelGGL(backout_add_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, s, dx, dxb, dback, pc, n / 4);
  return hipGetLastError();
}

hipError_t launch_adamw_small(float* w, uint16_t* wb, const float* g, float* m, float* v, long n, float lr,
                              float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(adamw_small_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w, wb, g, m, v, n, lr,
                     b1, b2, eps, wd, bc1, bc2);
  return hipGetLastError();
}

// ---- smear
namespace {
constexpr int kSmearBlocks = 256;
}
int smear_partials_floats() { return kSmearBlocks * (SMEAR_CH + 1); }

hipError_t launch_smear_fwd(const float* xe, float* x, float* a, const uint16_t* pw, const uint16_t* plam, long N,
                            int T, int d, hipStream_t s) {
  hipLaunchKernelGGL(smear_fwd_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, xe, x, a, pw, plam, N, T, d);
  return hipGetLastError();
}

hipError_t launch_smear_bwd(const float* dy, const float* xe, const float* a, float* dxo, const uint16_t* pw,
                            const uint16_t* plam, long N, int T, int d, float* partials, float* gw, float* glam,
                            int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(smear_bwd_kernel, dim3(kSmearBlocks), dim3(256), 0, s, dy, xe, a, dxo, pw, plam, N, T, d,
                     partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(smear_grads_kernel, dim3(1), dim3(64), 0, s, static_cast<const float*>(partials), kSmearBlocks,
                     gw, glam, accumulate);
  return hipGetLastError();
}

// ---- value embeddings
namespace {
constexpr int kVeBlocks = 256;
}
int ve_partials_floats(int Hkv) { return kVeBlocks * Hkv * VE_CH; }

hipError_t launch_ve_fwd(uint16_t* qkv, const uint16_t* xn, const int32_t* tok, const uint16_t* table,
                         const uint16_t* gate, float* logits, long N, int d, int Hkv, int V, hipStream_t s) {
  if (Hkv > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ve_fwd_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, qkv, xn, tok, table, gate,
                     logits, N, d, Hkv, V);
  return hipGetLastError();
}

hipError_t launch_ve_bwd(const uint16_t* dqkv, const uint16_t* xn, const int32_t* tok, const uint16_t* table,
                         const uint16_t* gate, const float* logits, float* dtable, float* dlogit, float* partials,
                         float* dgate, float* dxn, long N, int d, int Hkv, int V, int accumulate,
                         const ScatterWs& ws, hipStream_t s) {
  if (Hkv > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ve_bwd_kernel, dim3(kVeBlocks), dim3(256), 0, s, dqkv, xn, tok, table, logits, dlogit, partials,
                     N, d, Hkv, V);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = Hkv * VE_CH;
  hipLaunchKernelGGL(column_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(partials), kVeBlocks, n, dgate, accumulate);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ve_dxn_kernel, dim3((unsigned)((N * VE_CH + 255) / 256)), dim3(256), 0, s, dxn,
                     static_cast<const float*>(dlogit), gate, N, d, Hkv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long dkv = (long)Hkv * 128;
  return launch_ve_table_bwd(dqkv + d + dkv, d + 2 * dkv, logits, Hkv, tok, N, V, dtable, accumulate, ws, s);
}

hipError_t launch_adamw_range(float* w, uint16_t* wb, const float* g, float* m, float* v, long n, float lr,
                              float b1, float b2, float eps, float wd, float bc1, float bc2, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 != 0) return hipErrorInvalidValue;
  AdamwArgs a;
  a.w = w; a.wb = wb; a.g = g; a.m = m; a.v = v;
  a.woff[0] = 0; a.woff[1] = 0;
  a.n = n;
  a.lr = lr; a.b1 = b1; a.b2 = b2; a.eps = eps; a.wd = wd; a.bc1 = bc1; a.bc2 = bc2;
  hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(n / 4, 256, 2048), 1), dim3(256), 0, s, a);
  return hipGetLastError();
}
