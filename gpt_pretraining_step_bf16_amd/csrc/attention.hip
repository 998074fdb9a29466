// Causal flash attention forward and backward for gfx950, head size 128.
//
// [CT50] "1. Modelo GPT" and "5. Flash Attention Unificado": causal softmax
// attention computed by a fused flash-attention kernel (the page's FA3 is
// written for Hopper; this is a gfx950 design).
//
// Layout: q, k, v live in one packed buffer qkv [B*T, 3*H*128] bf16 (q heads,
// then k heads, then v heads; 128 columns per head), o is [B*T, H*128].
//
// Forward (per workgroup: 128 queries of one (b, h); 4 waves x 32 queries):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = 32 keys from LDS, B = the wave's 32
//    queries held in registers). A lane then holds one query and 32 of the 64
//    keys of a block, so the online-softmax max/sum are in-lane, plus one
//    exchange with lane ^ 32.
//  * O^T += V^T P^T: P^T is already in the B-operand layout (the 8 k-slots
//    of a lane are two groups of 4 consecutive keys), V^T comes from LDS
//    where V is stored transposed as [dim][key] in 8-byte units of 4 keys,
//    XOR-swizzled by dim so 16 consecutive dims hit distinct banks. The
//    accumulator O^T keeps one query per lane, so the rescale is in-lane too.
//  * K/V blocks of 64 keys are double-buffered in LDS (2 x 32 KB).
//  * Softmax runs in the log2 domain: scores are scaled by log2(e)/sqrt(128),
//    exp2 is used, and the saved normaliser lse2 is log2-based.
//
// Backward (deterministic, no atomics):
//  * delta = rowsum(dO * O) per (b, h, t).
//  * dK/dV kernel: a workgroup owns 128 keys, walks query blocks of 64 from
//    the diagonal; recomputes S = Q K^T and dP = dO V^T with the keys as the
//    lane index, then dV^T += dO^T P and dK^T += Q^T dS with Q and dO staged
//    in LDS both row-major and transposed.
//  * dQ kernel: a workgroup owns 128 queries, walks key blocks up to the
//    diagonal; recomputes S^T and dP^T with the queries as the lane index,
//    then dQ^T += K^T dS^T with K^T staged in LDS.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int HD = 128;
constexpr int QB = 128;   // queries per forward / dQ workgroup
constexpr int KB = 64;    // keys per K/V block
constexpr int NTHR = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Row-major [rows][128] tile in 16-byte chunks (16 per row), swizzled so the
// 16 lanes a 256-byte LDS cycle serves (16 rows, same logical chunk) hit 16
// distinct chunk positions.
__device__ __forceinline__ int rswz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }
// Transposed [128 dims][64 rows] tile in 8-byte units of 4 rows (16 per dim),
// with the unit position rotated by the dim so that consecutive dims reading
// the same logical unit land on different banks (measured best of the
// row/dim-parity variants).
__device__ __forceinline__ int tswz(int dim, int unit) { return dim * 16 + (unit ^ (dim & 15)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load a [64 rows][128] bf16 block (rows r0.. of a strided buffer) as 4 rows x
// 8 columns per thread: rows 4*(t%16)+i, columns 8*(t/16)..+7.
__device__ __forceinline__ void load_rows4x8(const uint16_t* __restrict__ base, long ld, int r0,
                                             int nrows, int tid, uint4 (&r)[4]) {
  const int kg = tid & 15;
  const int dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + 4 * kg + i;
    if (row < nrows) {
      r[i] = *reinterpret_cast<const uint4*>(base + (long)row * ld + dc * 8);
    } else {
      r[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t w4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Store the 4x8 block transposed: unit (dim 8dc+j, rows 4kg..4kg+3).
__device__ __forceinline__ void store_t4x8(uint2* __restrict__ lt, int tid, const uint4 (&r)[4]) {
  const int kg = tid & 15;
  const int dc = tid >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int sh = (j & 1) * 16;
    const uint32_t e0 = (w4(r[0], j >> 1) >> sh) & 0xffffu;
    const uint32_t e1 = (w4(r[1], j >> 1) >> sh) & 0xffffu;
    const uint32_t e2 = (w4(r[2], j >> 1) >> sh) & 0xffffu;
    const uint32_t e3 = (w4(r[3], j >> 1) >> sh) & 0xffffu;
    lt[tswz(dc * 8 + j, kg)] = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
  }
}

// Store the 4x8 block row-major.
__device__ __forceinline__ void store_r4x8(uint4* __restrict__ lr, int tid, const uint4 (&r)[4]) {
  const int kg = tid & 15;
  const int dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) lr[rswz(4 * kg + i, dc)] = r[i];
}

// A-operand fragment from a transposed tile: dim `dim`, k-slots = rows
// {base4, base4+1, base4+2, base4+3, base4+8, ..., base4+11} where
// base4 = 32t + 16(s%2) + 4h (rows relative to the tile).
__device__ __forceinline__ bf16x8 tfrag(const uint2* __restrict__ lt, int dim, int unit) {
  const uint2 a = lt[tswz(dim, unit)];
  const uint2 b = lt[tswz(dim, unit + 2)];
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

// Pack accumulator registers v0..v0+7 of a 32x32 tile into a bf16 B fragment.
__device__ __forceinline__ bf16x8 pack_frag(const f32x16& x, int v0) {
  return as_bf16x8(make_uint4(pack_bf2(x[v0 + 0], x[v0 + 1]), pack_bf2(x[v0 + 2], x[v0 + 3]),
                              pack_bf2(x[v0 + 4], x[v0 + 5]), pack_bf2(x[v0 + 6], x[v0 + 7])));
}

// ===========================================================================
// Forward
// ===========================================================================
__global__ void __launch_bounds__(NTHR, 2)
    attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out,
                    float* __restrict__ lse2, int T, int H) {
  __shared__ uint4 ks[2][KB * 16];
  __shared__ uint2 vt[2][HD * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int nqb = (T + QB - 1) / QB;
  const int qblk = nqb - 1 - blockIdx.x;  // heaviest blocks first
  const int bh = blockIdx.y;
  const int b = bh / H;
  const int h = bh - b * H;
  const int d = H * HD;
  const long ld = 3L * d;
  const uint16_t* qbase = qkv + (long)b * T * ld + h * HD;
  const uint16_t* kbase = qbase + d;
  const uint16_t* vbase = qbase + 2 * d;

  const int q0 = qblk * QB + wave * 32;
  const int qpos = q0 + (lane & 31);
  const float sc = GPT_LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)

  // Q fragments (B operand): query qpos, dims 16ks + 8hl .. +7.
  uint4 qf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qf[k] = qpos < T ? *reinterpret_cast<const uint4*>(qbase + (long)qpos * ld + 16 * k + 8 * hl)
                     : make_uint4(0, 0, 0, 0);
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int qmax = min(T - 1, qblk * QB + QB - 1);
  const int nkb = qmax / KB + 1;

  uint4 kr[4], vr[4];
  auto load_kv = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NTHR * i;
      const int key = kb * KB + (c >> 4);
      kr[i] = key < T ? *reinterpret_cast<const uint4*>(kbase + (long)key * ld + (c & 15) * 8)
                      : make_uint4(0, 0, 0, 0);
    }
    load_rows4x8(vbase, ld, kb * KB, T, tid, vr);
  };
  auto store_kv = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NTHR * i;
      ks[st][rswz(c >> 4, c & 15)] = kr[i];
    }
    store_t4x8(vt[st], tid, vr);
  };

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nkb) load_kv(kb + 1);
    if (kb * KB <= q0 + 31) {  // some key of this block is visible to the wave
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[t][v] = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const bf16x8 a = as_bf16x8(ks[st][rswz(32 * t + (lane & 31), 2 * k + hl)]);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qf[k]), s[t], 0, 0, 0);
        }
      }
      // s[t][v]: key kb*64 + 32t + 8(v/4) + 4hl + v%4, query qpos.
      float mloc = -INFINITY;
      // Masking is needed only where the block reaches past the wave's first
      // query (causal diagonal) or past the end of the sequence.
      const bool need_mask = (kb * KB + KB - 1 > q0) || (kb * KB + KB > T);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb * KB + 32 * t + 8 * (v >> 2) + 4 * hl + (v & 3);
            float x = s[t][v] * sc;
            if (key > qpos || key >= T) x = -INFINITY;
            s[t][v] = x;
            mloc = fmaxf(mloc, x);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = s[t][v] * sc;
            s[t][v] = x;
            mloc = fmaxf(mloc, x);
          }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_ref);
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = fast_exp2(s[t][v] - m_ref);
          s[t][v] = pv;
          lsum += pv;
        }
      lsum += __shfl_xor(lsum, 32, 64);
      l_run = alpha * l_run + lsum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
      bf16x8 pf[4];
#pragma unroll
      for (int sidx = 0; sidx < 4; ++sidx) pf[sidx] = pack_frag(s[sidx >> 1], 8 * (sidx & 1));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dim = 32 * dt + (lane & 31);
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx) {
          const int unit = 8 * (sidx >> 1) + 4 * (sidx & 1) + hl;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(vt[st], dim, unit), pf[sidx], o[dt], 0,
                                                          0, 0);
        }
      }
    }
    if (kb + 1 < nkb) store_kv(st ^ 1);
    __syncthreads();
  }

  if (qpos < T) {
    const float inv = 1.f / l_run;
    uint16_t* orow = out + ((long)b * T + qpos) * d + h * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * dt + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(orow + dim) =
            make_uint2(pack_bf2(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv),
                       pack_bf2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv));
      }
    if (hl == 0) lse2[(long)bh * T + qpos] = m_run + log2f(l_run);
  }
}

// ===========================================================================
// Backward: delta = rowsum(dO * O)
// ===========================================================================
__global__ void attn_bwd_delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
                                      float* __restrict__ delta, int T, int H, long rows) {
  const int lane = threadIdx.x & 63;
  const long idx = blockIdx.x * 4L + (threadIdx.x >> 6);  // (row, head)
  if (idx >= rows * H) return;
  const long row = idx / H;
  const int h = (int)(idx - row * H);
  const long off = row * (long)H * HD + h * HD + 2 * lane;
  const uint32_t a = *reinterpret_cast<const uint32_t*>(o + off);
  const uint32_t g = *reinterpret_cast<const uint32_t*>(dO + off);
  float s = bf_lo(a) * bf_lo(g) + bf_hi(a) * bf_hi(g);
  s = warp_sum(s);
  if (lane == 0) {
    const long b = row / T;
    const long t = row - b * T;
    delta[(b * H + h) * T + t] = s;
  }
}

// ===========================================================================
// Backward: dK, dV
// ===========================================================================
constexpr int KBW = 128;  // keys per dK/dV workgroup
constexpr int QBW = 64;   // queries per block walked

__global__ void __launch_bounds__(NTHR, 1)
    attn_bwd_dkdv_kernel(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dO,
                         const float* __restrict__ lse2, const float* __restrict__ delta,
                         uint16_t* __restrict__ dqkv, int T, int H) {
  __shared__ uint4 qs[2][QBW * 16];
  __shared__ uint4 dos[2][QBW * 16];
  __shared__ uint2 qt[2][HD * 16];
  __shared__ uint2 dot_[2][HD * 16];
  __shared__ __attribute__((aligned(16))) float ls[2][QBW];
  __shared__ __attribute__((aligned(16))) float ds_[2][QBW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int kblk = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H;
  const int h = bh - b * H;
  const int d = H * HD;
  const long ld = 3L * d;
  const uint16_t* qbase = qkv + (long)b * T * ld + h * HD;
  const uint16_t* kbase = qbase + d;
  const uint16_t* vbase = qbase + 2 * d;
  const uint16_t* dobase = dO + (long)b * T * d + h * HD;
  const float* lrow = lse2 + (long)bh * T;
  const float* drow = delta + (long)bh * T;
  const float sc = GPT_LOG2E * 0.08838834764831845f;

  const int k0 = kblk * KBW + wave * 32;
  const int kpos = k0 + (lane & 31);

  // K and V fragments as B operands: key kpos, dims 16k + 8hl .. +7.
  uint4 kf[8], vf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool ok = kpos < T;
    kf[k] = ok ? *reinterpret_cast<const uint4*>(kbase + (long)kpos * ld + 16 * k + 8 * hl)
               : make_uint4(0, 0, 0, 0);
    vf[k] = ok ? *reinterpret_cast<const uint4*>(vbase + (long)kpos * ld + 16 * k + 8 * hl)
               : make_uint4(0, 0, 0, 0);
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dk[i][v] = 0.f;
      dv[i][v] = 0.f;
    }

  const int qb_first = (kblk * KBW) / QBW;
  const int qb_end = (T + QBW - 1) / QBW;

  uint4 qr[4], gr[4];
  float lv = 0.f, dvv = 0.f;
  auto load_q = [&](int qb) {
    load_rows4x8(qbase, ld, qb * QBW, T, tid, qr);
    load_rows4x8(dobase, d, qb * QBW, T, tid, gr);
    if (tid < QBW) {
      const int q = qb * QBW + tid;
      lv = q < T ? lrow[q] : 0.f;
      dvv = q < T ? drow[q] : 0.f;
    }
  };
  auto store_q = [&](int st) {
    store_r4x8(qs[st], tid, qr);
    store_t4x8(qt[st], tid, qr);
    store_r4x8(dos[st], tid, gr);
    store_t4x8(dot_[st], tid, gr);
    if (tid < QBW) {
      ls[st][tid] = lv;
      ds_[st][tid] = dvv;
    }
  };

  if (qb_first < qb_end) {
    load_q(qb_first);
    store_q(0);
  }
  __syncthreads();

  for (int qb = qb_first; qb < qb_end; ++qb) {
    const int st = (qb - qb_first) & 1;
    if (qb + 1 < qb_end) load_q(qb + 1);
    if (qb * QBW + QBW - 1 >= k0 && k0 < T) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[t][v] = 0.f;
          dp[t][v] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int row = 32 * t + (lane & 31);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qs[st][rswz(row, 2 * k + hl)]),
                                                         as_bf16x8(kf[k]), s[t], 0, 0, 0);
          dp[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(dos[st][rswz(row, 2 * k + hl)]),
                                                          as_bf16x8(vf[k]), dp[t], 0, 0, 0);
        }
      }
      // s[t][v]: query qb*64 + 32t + 8(v/4) + 4hl + v%4, key kpos.
      // Mask where some query of the block precedes a key of the wave, or the
      // block runs past the end of the sequence.
      const bool need_mask = (qb * QBW < k0 + 31) || (qb * QBW + QBW > T);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * t + 8 * g + 4 * hl;
          const float4 l4 = *reinterpret_cast<const float4*>(&ls[st][ql]);
          const float4 d4 = *reinterpret_cast<const float4*>(&ds_[st][ql]);
          const float lq[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qb * QBW + ql + r;
            const int v = 4 * g + r;
            float p = fast_exp2(fmaf(s[t][v], sc, -lq[r]));
            if (need_mask && (kpos > q || q >= T)) p = 0.f;
            s[t][v] = p;
            dp[t][v] = p * (dp[t][v] - dq[r]);
          }
        }
      bf16x8 pf[4], dsf[4];
#pragma unroll
      for (int sidx = 0; sidx < 4; ++sidx) {
        pf[sidx] = pack_frag(s[sidx >> 1], 8 * (sidx & 1));
        dsf[sidx] = pack_frag(dp[sidx >> 1], 8 * (sidx & 1));
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dim = 32 * dt + (lane & 31);
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx) {
          const int unit = 8 * (sidx >> 1) + 4 * (sidx & 1) + hl;
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(dot_[st], dim, unit), pf[sidx], dv[dt],
                                                           0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(qt[st], dim, unit), dsf[sidx], dk[dt],
                                                           0, 0, 0);
        }
      }
    }
    if (qb + 1 < qb_end) store_q(st ^ 1);
    __syncthreads();
  }

  if (kpos < T) {
    const float scale = 0.08838834764831845f;
    uint16_t* krow = dqkv + ((long)b * T + kpos) * ld + d + h * HD;
    uint16_t* vrow = krow + d;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * dt + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(krow + dim) =
            make_uint2(pack_bf2(dk[dt][4 * g + 0] * scale, dk[dt][4 * g + 1] * scale),
                       pack_bf2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale));
        *reinterpret_cast<uint2*>(vrow + dim) =
            make_uint2(pack_bf2(dv[dt][4 * g + 0], dv[dt][4 * g + 1]),
                       pack_bf2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]));
      }
  }
}

// ===========================================================================
// Backward: dQ
// ===========================================================================
__global__ void __launch_bounds__(NTHR, 1)
    attn_bwd_dq_kernel(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dO,
                       const float* __restrict__ lse2, const float* __restrict__ delta,
                       uint16_t* __restrict__ dqkv, int T, int H) {
  __shared__ uint4 ks[2][KB * 16];
  __shared__ uint4 vs[2][KB * 16];
  __shared__ uint2 kt[2][HD * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int nqb = (T + QB - 1) / QB;
  const int qblk = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H;
  const int h = bh - b * H;
  const int d = H * HD;
  const long ld = 3L * d;
  const uint16_t* qbase = qkv + (long)b * T * ld + h * HD;
  const uint16_t* kbase = qbase + d;
  const uint16_t* vbase = qbase + 2 * d;
  const uint16_t* dobase = dO + (long)b * T * d + h * HD;
  const float sc = GPT_LOG2E * 0.08838834764831845f;

  const int q0 = qblk * QB + wave * 32;
  const int qpos = q0 + (lane & 31);
  const bool qok = qpos < T;

  uint4 qf[8], gf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qf[k] = qok ? *reinterpret_cast<const uint4*>(qbase + (long)qpos * ld + 16 * k + 8 * hl)
                : make_uint4(0, 0, 0, 0);
    gf[k] = qok ? *reinterpret_cast<const uint4*>(dobase + (long)qpos * d + 16 * k + 8 * hl)
                : make_uint4(0, 0, 0, 0);
  }
  const float lq = qok ? lse2[(long)bh * T + qpos] : 0.f;
  const float dq_ = qok ? delta[(long)bh * T + qpos] : 0.f;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  const int qmax = min(T - 1, qblk * QB + QB - 1);
  const int nkb = qmax / KB + 1;

  uint4 kr[4], vr[4];
  auto load_kv = [&](int kb) {
    load_rows4x8(kbase, ld, kb * KB, T, tid, kr);
    load_rows4x8(vbase, ld, kb * KB, T, tid, vr);
  };
  auto store_kv = [&](int st) {
    store_r4x8(ks[st], tid, kr);
    store_t4x8(kt[st], tid, kr);
    store_r4x8(vs[st], tid, vr);
  };

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nkb) load_kv(kb + 1);
    if (kb * KB <= q0 + 31) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[t][v] = 0.f;
          dp[t][v] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int row = 32 * t + (lane & 31);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ks[st][rswz(row, 2 * k + hl)]),
                                                         as_bf16x8(qf[k]), s[t], 0, 0, 0);
          dp[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vs[st][rswz(row, 2 * k + hl)]),
                                                          as_bf16x8(gf[k]), dp[t], 0, 0, 0);
        }
      }
      // s[t][v]: key kb*64 + 32t + 8(v/4) + 4hl + v%4, query qpos.
      const bool need_mask = (kb * KB + KB - 1 > q0) || (kb * KB + KB > T) || (q0 + 32 > T);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * KB + 32 * t + 8 * (v >> 2) + 4 * hl + (v & 3);
          float p = fast_exp2(fmaf(s[t][v], sc, -lq));
          if (need_mask && (key > qpos || key >= T || !qok)) p = 0.f;
          dp[t][v] = p * (dp[t][v] - dq_);
        }
      bf16x8 dsf[4];
#pragma unroll
      for (int sidx = 0; sidx < 4; ++sidx) dsf[sidx] = pack_frag(dp[sidx >> 1], 8 * (sidx & 1));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dim = 32 * dt + (lane & 31);
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx) {
          const int unit = 8 * (sidx >> 1) + 4 * (sidx & 1) + hl;
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag(kt[st], dim, unit), dsf[sidx],
                                                            acc[dt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) store_kv(st ^ 1);
    __syncthreads();
  }

  if (qok) {
    const float scale = 0.08838834764831845f;
    uint16_t* qrow = dqkv + ((long)b * T + qpos) * ld + h * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * dt + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(qrow + dim) =
            make_uint2(pack_bf2(acc[dt][4 * g + 0] * scale, acc[dt][4 * g + 1] * scale),
                       pack_bf2(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale));
      }
  }
}

}  // namespace

hipError_t launch_attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse2, int B, int T, int H,
                                hipStream_t s) {
  if (B <= 0 || T <= 0 || H <= 0) return hipSuccess;
  dim3 grid((T + QB - 1) / QB, B * H);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(NTHR), 0, s, qkv, o, lse2, T, H);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse2,
                                const uint16_t* dO, uint16_t* dqkv, float* delta, int B, int T,
                                int H, hipStream_t s) {
  if (B <= 0 || T <= 0 || H <= 0) return hipSuccess;
  const long rows = (long)B * T;
  hipLaunchKernelGGL(attn_bwd_delta_kernel, dim3((unsigned)((rows * H + 3) / 4)), dim3(256), 0, s, o,
                     dO, delta, T, H, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((T + KBW - 1) / KBW, B * H), dim3(NTHR), 0, s, qkv,
                     dO, lse2, delta, dqkv, T, H);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((T + QB - 1) / QB, B * H), dim3(NTHR), 0, s, qkv, dO,
                     lse2, delta, dqkv, T, H);
  return hipGetLastError();
}
