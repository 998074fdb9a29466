// Causal flash attention forward and backward for gfx950, head size 128.
//
// [CT50] "1. Modelo GPT" and "5. Flash Attention Unificado": causal softmax
// attention computed by a fused flash-attention kernel (the page's FA3 is
// written for Hopper; this is a gfx950 design), optionally with a window W
// (short/long window attention): key j is visible to query i when
// i - W <= j <= i. W >= T - 1 is the plain causal mask. Tiles wholly outside
// the band are skipped, not masked.
//
// Layout: q, k, v live in one packed buffer qkv [B*T, (H + 2*Hkv)*128] bf16
// (H query heads, then Hkv key heads, then Hkv value heads; 128 columns per
// head), o is [B*T, H*128]. With Hkv < H (grouped-query attention, [CT50]
// "1. Modelo GPT": fewer KV heads) query head h reads key/value head
// h / (H / Hkv); the dK/dV kernel sums over the query heads of its group.
//
// Every K, V, Q or dO tile that more than one wave reads goes global -> LDS
// by direct loads (global_load_lds_dwordx4), row-major [64 rows][128] with
// the 16-byte chunk c of row r at position c ^ swz(r), swz swapping the two
// 2-bit fields of r % 16: 16 consecutive rows of one chunk, and 4 consecutive
// rows of 4 consecutive chunks, each land on 16 distinct bank groups, which
// makes both read kinds below free of bank conflicts. MFMA operands come
// out of that one copy two ways: row fragments (32 rows x 8 dims per lane
// half) by ds_read_b128, and transposed fragments (32 dims x 4+4 rows) by
// ds_read_b64_tr_b16. No wave transposes through registers.
//
// All products are v_mfma_f32_32x32x16_bf16. A 32x32 accumulator lane holds
// one column (lane % 32) and the 16 rows 8g + 4(lane / 32) + r, g, r < 4; a
// pair of row groups (g = 2m, 2m+1) is exactly the k-slot order of a
// transposed fragment read at rows 16m + 4(lane / 32) + {0..3, 8..11}, so a
// packed accumulator feeds the next product as a B operand with no shuffle.
//
// Forward (workgroup: 128 queries of one (b, h); 4 waves x 32 queries):
//  * S^T = K Q^T (A = K rows from LDS, B = the wave's queries in registers):
//    a lane holds one query, so the online-softmax state is per lane, plus
//    one exchange with lane ^ 32 for the block max.
//  * O^T += V^T P^T (A = V transposed from LDS, B = P^T packed in place).
//  * Softmax in the log2 domain with the scale folded into one FMA. The
//    reference max is only moved (and O, l rescaled) when a block exceeds it
//    by more than 8 in log2 units; probabilities then stay below 2^8, so
//    nothing overflows and the normalised result is unchanged.
//
// Backward (deterministic, no atomics), two kernels in this order:
//  * dQ: a workgroup owns 128 queries (Q, dO in registers) and walks 64-key
//    tiles up to the diagonal: S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T (A = K transposed). It first forms
//    delta = rowsum(dO * O) for its queries and writes it out.
//  * dK/dV: a workgroup owns 128 keys (32 per wave, K and V in registers) and
//    walks 64-query tiles of Q and dO from the diagonal: S = Q K^T and
//    dP = dO V^T (A = Q, dO rows), then dV^T += dO^T P and dK^T += Q^T dS
//    (A = dO, Q transposed), using the delta written by dQ.
#include <type_traits>

#include "common.h"
#include "attention.h"
#include "kernels.h"
#include "lds_dma.h"

namespace {

constexpr int HD = 128;

// A burst of MFMAs (with the fragment reads that feed it) at raised wave
// priority. The dQ kernel holds two waves per SIMD (two workgroups per CU);
// while one issues its MFMAs, the other's softmax and dS VALU work fills the
// gaps instead of taking their issue slots (d20, same GPU: attention
// backward 37.9-38.2 -> 37.4-37.8 ms per step). The forward kernel and the
// GEMM measured 1% slower with the same.
__device__ __forceinline__ void mfma_prio_begin() {
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void mfma_prio_end() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}
constexpr int QB = 128;   // queries per forward / dQ workgroup
constexpr int KB = 64;    // keys per K/V tile
constexpr int KBW = 128;  // keys per dK/dV workgroup
constexpr int QBW = 64;   // queries per Q/dO tile of the dK/dV kernel
constexpr int NTHR = 256;
constexpr int TILE = 64 * HD * 2;  // bytes of one [64][128] bf16 tile

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Chunk swizzle of row r (only r % 16 matters; tile fragments start at rows % 16 == 0).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Per-lane byte offsets, within a tile, of the fragments a lane reads.
struct FragAddr {
  uint32_t row[8];    // row fragment of k-step k: row lane % 32, chunk 2k + lane / 32
  uint32_t tr[4][2];  // transposed fragment of dim tile dt, read r (rows +8r)
};

__device__ __forceinline__ void frag_addr(int lane, FragAddr& a) {
  const int hl = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int k = 0; k < 8; ++k) a.row[k] = r * 256 + (((2 * k + hl) ^ swz(r)) << 4);
  // Transposed read: group g = lane / 16, group-lane p = 4 j + q addresses row
  // base + 8 rr + 4 (g >> 1) + j at dims 32 dt + 16 (g & 1) + 4 q .. +3; the
  // lane receives dim 32 dt + 16 (g & 1) + p at the four rows of its group.
  const int g = lane >> 4, p = lane & 15, j = p >> 2, q = p & 3;
  const int c0 = 2 * (g & 1) + (q >> 1);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int x = 8 * rr + 4 * (g >> 1) + j;  // row within the 16-row group (base % 16 == 0)
      a.tr[dt][rr] = x * 256 + (((4 * dt + c0) ^ swz(x)) << 4) + (q & 1) * 8;
    }
}

// Row fragment: rows rbase + lane % 32 (rbase % 16 == 0), dims 16k + 8 (lane / 32) .. +7.
__device__ __forceinline__ bf16x8 row_frag(const char* tile, const FragAddr& a, int rbase, int k) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(tile + rbase * 256 + a.row[k]));
}

// Transposed fragment: dims 32 dt + lane % 32; k-slots rows
// rbase + 4 (lane / 32) + {0..3} and rbase + 8 + 4 (lane / 32) + {0..3} (rbase % 16 == 0).
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, const FragAddr& a, int rbase, int dt) {
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_V4S(tile + rbase * 256 + a.tr[dt][0]));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_V4S(tile + rbase * 256 + a.tr[dt][1]));
  const uint2 x = __builtin_bit_cast(uint2, lo);
  const uint2 y = __builtin_bit_cast(uint2, hi);
  return as_bf16x8(make_uint4(x.x, x.y, y.x, y.y));
}

// Direct load of rows r0 .. r0+63 (row stride ld elements, rows past nrows - 1
// read row nrows - 1) into a swizzled LDS tile; wave w issues 1 KB blocks
// 4w .. 4w+3 (4 rows each).
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ base, long ld, int r0, int nrows,
                                         char* tile, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = 4 * wave + i;
    const int row = 4 * blk + (lane >> 4);
    const int chunk = (lane & 15) ^ swz(row);
    const int gr = min(r0 + row, nrows - 1);
    dma16(base + (long)gr * ld + chunk * 8, lds_addr(tile + blk * 1024));
  }
}

// Per-lane byte offsets of the four 1 KB blocks a wave loads from a row-major
// source with row stride ld elements (rows 16 wave + 4 i + lane / 16).
struct TileDma {
  uint32_t off[4];
};

__device__ __forceinline__ void tile_dma_init(TileDma& t, long ld, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ swz(row);
    t.off[i] = (uint32_t)(((long)row * ld + chunk * 8) * 2);
  }
}

// dma_tile with a scalar base and precomputed offsets when all 64 rows exist.
__device__ __forceinline__ void dma_tile_fast(const uint16_t* __restrict__ base, long ld, int r0, int nrows,
                                              char* tile, int wave, int lane, const TileDma& t) {
  if (r0 + 64 <= nrows) {
    const uint16_t* sb = base + (long)r0 * ld;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_sv(sb, t.off[i], lds_addr(tile + (4 * wave + i) * 1024));
  } else {
    dma_tile(base, ld, r0, nrows, tile, wave, lane);
  }
}

// 64 floats v[r0 .. r0+63] (indices past n - 1 read v[n - 1]) into LDS.
__device__ __forceinline__ void dma_vec64(const float* __restrict__ v, int r0, int n, float* dst,
                                          int lane) {
  dma4(v + min(r0 + lane, n - 1), lds_addr(dst));
}

__device__ __forceinline__ bf16x8 pack_frag(const f32x16& x, int v0) {
  return as_bf16x8(make_uint4(pack_bf2(x[v0 + 0], x[v0 + 1]), pack_bf2(x[v0 + 2], x[v0 + 3]),
                              pack_bf2(x[v0 + 4], x[v0 + 5]), pack_bf2(x[v0 + 6], x[v0 + 7])));
}

// Work item of a (blocks_per_head x heads) grid, remapped so that the blocks
// of one head run on the same XCD (they share its K/V or Q/dO in L2). Heads
// go in groups of HG whose blocks alternate, block index 0 of each first:
// callers map block 0 to the most work, so the short blocks of one group fill
// the gaps left by the long ones of the next instead of a head's long block
// starting last. Measured on the d20 step: groups of 8 for the forward, 4 for
// the two backward kernels (pairs: 2-4% slower; one head at a time: 6-7%).
template <int HG>
__device__ __forceinline__ void head_block(int& blk, int& bh) {
  const int nb = gridDim.x;
  const int nh = gridDim.y;
  const int total = nb * nh;
  int lin = blockIdx.x + nb * blockIdx.y;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int grp = lin / (HG * nb);
  const int r = lin - grp * HG * nb;
  const int gs = min(HG, nh - HG * grp);  // fewer for the last heads
  blk = r / gs;
  bh = HG * grp + (r - blk * gs);
}

// ===========================================================================
// Forward
// ===========================================================================
__global__ void __launch_bounds__(NTHR, 2)
    attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out,
                    float* __restrict__ lse2, int T, int H, int Hkv, int W) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  int xb, bh;
  head_block<8>(xb, bh);
  const int nqb = (T + QB - 1) / QB;
  const int qblk = nqb - 1 - xb;  // heaviest blocks first
  const int b = bh / H;
  const int h = bh - b * H;
  const int d = H * HD;
  const int dkv = Hkv * HD;
  const long ld = (long)d + 2L * dkv;
  const uint16_t* qbase = qkv + (long)b * T * ld + h * HD;
  const uint16_t* kbase = qkv + (long)b * T * ld + d + (h / (H / Hkv)) * HD;
  const uint16_t* vbase = kbase + dkv;
  const int q0 = qblk * QB + wave * 32;
  const int qpos = q0 + (lane & 31);
  const float sc = GPT_LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)
  // Rescale only when the block max exceeds the reference by 8 in log2 units.
  const float lazy = 8.f / sc;

  FragAddr fa;
  frag_addr(lane, fa);

  // Q fragments (B operand): query qpos, dims 16k + 8hl .. +7.
  uint4 qf[8];
  {
    const uint16_t* qrow = qbase + (long)min(qpos, T - 1) * ld + 8 * hl;
#pragma unroll
    for (int k = 0; k < 8; ++k) qf[k] = *reinterpret_cast<const uint4*>(qrow + 16 * k);
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_ref = -INFINITY;  // raw-score reference max (the same in both lane halves)
  float l_run = 0.f;        // this lane half's share of the normaliser

  const int qmax = min(T - 1, qblk * QB + QB - 1);
  const int nkb = qmax / KB + 1;
  const int kb_lo = max(0, qblk * QB - W) / KB;  // first tile inside the window of the block

  TileDma td;
  tile_dma_init(td, ld, wave, lane);
  // Keys visible to this lane's query: kwin .. kwin + kspan, i.e.
  // qpos - W .. min(qpos, T - 1).
  const int kwin = qpos - W;
  const uint32_t kspan = (uint32_t)(min(qpos, T - 1) - kwin);

  auto issue = [&](int kb, int st) {
    char* ks = smem + st * 2 * TILE;
    dma_tile_fast(kbase, ld, kb * KB, T, ks, wave, lane, td);
    dma_tile_fast(vbase, ld, kb * KB, T, ks + TILE, wave, lane, td);
  };

  auto block = [&](int kb, int st) {
    const char* ks = smem + st * 2 * TILE;
    const char* vs = ks + TILE;
    // No key of this block is visible to the wave: past its last query, or
    // before the window of its first query.
    if (kb * KB > q0 + 31 || kb * KB + KB - 1 < q0 - W) return;
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[t][v] = 0.f;
    // K fragments are read one step ahead of their MFMA.
    bf16x8 fk[16];
    fk[0] = row_frag(ks, fa, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) fk[i + 1] = row_frag(ks, fa, 32 * ((i + 1) >> 3), (i + 1) & 7);
      s[i >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[i], as_bf16x8(qf[i & 7]), s[i >> 3], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // s[t][v]: key kb*64 + 32t + 8(v/4) + 4hl + v%4, query qpos (raw q.k).
    const bool need_mask = (kb * KB + KB - 1 > q0) || (kb * KB + KB > T) || (kb * KB < q0 + 31 - W);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * KB + 32 * t + 8 * (v >> 2) + 4 * hl + (v & 3);
          if ((uint32_t)(key - kwin) > kspan) s[t][v] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[t][v]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    if (__builtin_amdgcn_ballot_w64(mloc > m_ref + lazy) != 0) {
      const float m_new = fmaxf(m_ref, mloc);
      const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * sc);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
      m_ref = m_new;
    }
    const float msc = m_ref == -INFINITY ? 0.f : m_ref * sc;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = fast_exp2(fmaf(s[t][v], sc, -msc));
        s[t][v] = pv;
        l_run += pv;
      }
    bf16x8 pf[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) pf[si] = pack_frag(s[si >> 1], 8 * (si & 1));
    // V^T fragments of dim tile dt+1 are read during the MFMAs of dt.
    bf16x8 av[2][4];
#pragma unroll
    for (int si = 0; si < 4; ++si) av[0][si] = tr_frag(vs, fa, 16 * si, 0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int cb = dt & 1;
      if (dt + 1 < 4) {
#pragma unroll
        for (int si = 0; si < 4; ++si) av[cb ^ 1][si] = tr_frag(vs, fa, 16 * si, dt + 1);
      }
#pragma unroll
      for (int si = 0; si < 4; ++si)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cb][si], pf[si], o[dt], 0, 0, 0);
    }
  };

  issue(kb_lo, 0);
  VMCNT_BARRIER(0);
  for (int kb = kb_lo; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) issue(kb + 1, 1);
    block(kb, 0);
    VMCNT_BARRIER(0);
    if (kb + 1 < nkb) {
      if (kb + 2 < nkb) issue(kb + 2, 0);
      block(kb + 1, 1);
      VMCNT_BARRIER(0);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qpos < T) {
    const float inv = 1.f / l_tot;
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
    if (hl == 0) lse2[(long)bh * T + qpos] = m_ref * sc + log2f(l_tot);
  }
}

// QK-norm + RoPE backward ([CT50] "1. Modelo GPT": q and k are normalised per
// head, then rotated) on a head's gradient dy held in the accumulator layout:
// the lane holds dims 32 dt + 8 g + 4 hl + r (element 4 g + r of a[dt]) of one
// row, lane ^ 32 the other half, so a RoPE pair (j, j + 64) is a[dt], a[dt + 2]
// of one lane. y = rope(norm(x)) is the saved bf16 head, given as the row
// fragments the kernel already holds (yf[k]: dims 16 k + 8 hl .. +7), rstd its
// saved norm scale, cs the (cos, sin) row of the position. With n = rope^-1(y),
// dn = rope^-1(dy): dx = rstd (dn - n mean(dy y)) (the rotation keeps dot
// products). The result replaces a; `scale` multiplies dy first.
__device__ __forceinline__ void qknorm_rope_bwd_acc(f32x16 (&a)[4], float scale, const uint4 (&yf)[8], float rstd,
                                                    const float* __restrict__ cs, int hl) {
  // Dims 32 dt + 8 g + 4 hl + r sit in yf[2 dt + g / 2] of lane half g % 2,
  // words (x, y) for hl = 0 and (z, w) for hl = 1: half of them come from the
  // lane ^ 32, which sends the pair this lane needs.
  // yw[dt][v / 2]: the bf16 pair of dims 32 dt + 8 g + 4 hl + 2 h + {0, 1}
  // (v = 4 g + 2 h), kept packed to spare registers.
  uint32_t yw[4][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t own0 = hl ? yf[k].z : yf[k].x, own1 = hl ? yf[k].w : yf[k].y;
    const uint32_t give0 = hl ? yf[k].x : yf[k].z, give1 = hl ? yf[k].y : yf[k].w;
    const uint32_t got0 = (uint32_t)__shfl_xor((int)give0, 32, 64);
    const uint32_t got1 = (uint32_t)__shfl_xor((int)give1, 32, 64);
    const int dt = k >> 1;
    const int w0 = 4 * (k & 1);  // g = 2 (k & 1) (lane half 0's) and g + 1 (lane half 1's)
    yw[dt][w0 + 0] = hl ? got0 : own0;
    yw[dt][w0 + 1] = hl ? got1 : own1;
    yw[dt][w0 + 2] = hl ? own0 : got0;
    yw[dt][w0 + 3] = hl ? own1 : got1;
  }
  float dot = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[dt][4 * g + r] *= scale;
        dot += a[dt][4 * g + r] * ((r & 1) ? bf_hi(yw[dt][2 * g + (r >> 1)]) : bf_lo(yw[dt][2 * g + (r >> 1)]));
      }
    }
  dot += __shfl_xor(dot, 32, 64);
  dot *= 1.f / 128.f;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4* cp = reinterpret_cast<const float4*>(cs + 2 * (32 * dt + 8 * g + 4 * hl));
      const float4 c01 = cp[0], c23 = cp[1];
      const float cv[4] = {c01.x, c01.z, c23.x, c23.z};
      const float sv[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * g + r;
        const float g1 = a[dt][v], g2 = a[dt + 2][v];
        const uint32_t w1 = yw[dt][2 * g + (r >> 1)], w2 = yw[dt + 2][2 * g + (r >> 1)];
        const float y1 = (r & 1) ? bf_hi(w1) : bf_lo(w1), y2 = (r & 1) ? bf_hi(w2) : bf_lo(w2);
        const float dn1 = g1 * cv[r] + g2 * sv[r], dn2 = g2 * cv[r] - g1 * sv[r];
        const float n1 = y1 * cv[r] + y2 * sv[r], n2 = y2 * cv[r] - y1 * sv[r];
        a[dt][v] = rstd * (dn1 - n1 * dot);
        a[dt + 2][v] = rstd * (dn2 - n2 * dot);
      }
    }
}

// ===========================================================================
// Backward: dK, dV
// ===========================================================================
constexpr int DKDV_STAGE = 2 * TILE + 2 * QBW * 4;  // Q tile, dO tile, lse, delta
constexpr int DKDV_NST = 4;                         // stages of the Q/dO ring

// Software-pipelined over the query tiles: while the softmax / dS VALU work
// of tile n runs, the MFMAs of S and dP for tile n+1 are issued from the same
// wave, then dV and dK of tile n; the Q/dO ring holds tiles n .. n+2. Every
// wave walks every tile of the workgroup (tiles entirely before a wave's keys
// are masked to zero), so all waves keep one schedule. Each wave issues the
// same number of direct loads per tile (waves 2 and 3 load a dummy row), so a
// single vmcnt(0) + barrier per tile orders the ring.
__global__ void __launch_bounds__(NTHR, 1)
    attn_bwd_dkdv_kernel(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dO,
                         const float* __restrict__ lse2, const float* __restrict__ delta,
                         uint16_t* __restrict__ dqkv, const float* __restrict__ rstd_qk,
                         const float* __restrict__ cs, int T, int H, int Hkv, int W) {
  __shared__ __attribute__((aligned(1024))) char smem[DKDV_NST * DKDV_STAGE + 256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  int kblk, bkv;
  head_block<4>(kblk, bkv);  // bkv = b * Hkv + key/value head
  const int b = bkv / Hkv;
  const int hk = bkv - b * Hkv;
  const int G = H / Hkv;  // query heads per key/value head
  const int d = H * HD;
  const int dkv = Hkv * HD;
  const long ld = (long)d + 2L * dkv;
  const uint16_t* kbase = qkv + (long)b * T * ld + d + hk * HD;
  const uint16_t* vbase = kbase + dkv;
  // Query head g of the group: its q columns, dO columns, lse and delta rows.
  auto qbase = [&](int g) { return qkv + (long)b * T * ld + (hk * G + g) * HD; };
  auto dobase = [&](int g) { return dO + (long)b * T * d + (hk * G + g) * HD; };
  auto lrow = [&](int g) { return lse2 + ((long)b * H + hk * G + g) * T; };
  auto drow = [&](int g) { return delta + ((long)b * H + hk * G + g) * T; };
  const float sc = GPT_LOG2E * 0.08838834764831845f;

  const int k0 = kblk * KBW + wave * 32;
  const int kpos = k0 + (lane & 31);

  FragAddr fa;
  frag_addr(lane, fa);

  // K and V fragments as B operands: key kpos, dims 16k + 8hl .. +7.
  uint4 kf[8], vf[8];
  {
    const long kr = (long)min(kpos, T - 1) * ld + 8 * hl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      kf[k] = *reinterpret_cast<const uint4*>(kbase + kr + 16 * k);
      vf[k] = *reinterpret_cast<const uint4*>(vbase + kr + 16 * k);
    }
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dk[i][v] = 0.f;
      dv[i][v] = 0.f;
    }

  // Query tiles from the block's first key to the last query that sees its
  // last key (query i sees key j for j <= i <= j + W).
  const int qb_first = (kblk * KBW) / QBW;
  const int qb_end = min((T + QBW - 1) / QBW, (min(T - 1, kblk * KBW + KBW - 1 + W)) / QBW + 1);
  const int nqt = qb_end - qb_first;  // query tiles per query head
  const int ntile = G * nqt;          // tile n: head n / nqt, query tile n % nqt
  const int qlim = min(T - 1 - kpos, W);  // last visible query - kpos (negative past T)

  TileDma tq, tg;
  tile_dma_init(tq, ld, wave, lane);
  tile_dma_init(tg, d, wave, lane);
  float* dummy = reinterpret_cast<float*>(smem + DKDV_NST * DKDV_STAGE);

  auto stage = [&](int st) { return smem + st * DKDV_STAGE; };
  auto issue = [&](int n, int st) {
    char* base = stage(st);
    const int g = n / nqt;
    const int q0 = (qb_first + n - g * nqt) * QBW;
    dma_tile_fast(qbase(g), ld, q0, T, base, wave, lane, tq);
    dma_tile_fast(dobase(g), d, q0, T, base + TILE, wave, lane, tg);
    float* dst = wave == 0 ? reinterpret_cast<float*>(base + 2 * TILE)
               : wave == 1 ? reinterpret_cast<float*>(base + 2 * TILE + QBW * 4)
                           : dummy;
    dma_vec64(wave == 1 ? drow(g) : lrow(g), q0, T, dst, lane);
  };

  // Work unit: one 32-query half t of a 64-query tile.
  // S = Q K^T and dP = dO V^T of half t of the tile in stage st. Fragments are
  // read two k-steps ahead of their MFMAs (sched_group_barrier pins the
  // order), so LDS latency hides under the previous MFMAs.
  auto sdp = [&](int st, int t, f32x16& s, f32x16& dp) {
    const char* qs = stage(st);
    const char* gs = qs + TILE;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = 0.f;
      dp[v] = 0.f;
    }
    bf16x8 fq[8], fg[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      fq[k] = row_frag(qs, fa, 32 * t, k);
      fg[k] = row_frag(gs, fa, 32 * t, k);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + 2 < 8) {
        fq[k + 2] = row_frag(qs, fa, 32 * t, k + 2);
        fg[k + 2] = row_frag(gs, fa, 32 * t, k + 2);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[k], as_bf16x8(kf[k]), s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fg[k], as_bf16x8(vf[k]), dp, 0, 0, 0);
    }
    // mask 0x100: DS read, 0x008: MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // dV^T += dO^T P and dK^T += Q^T dS for half t of the tile in stage st;
  // the transposed fragments of dim tile dt+1 are read during the MFMAs of dt.
  auto dvdk = [&](int st, int t, const bf16x8 (&pf)[2], const bf16x8 (&dsf)[2]) {
    const char* qs = stage(st);
    const char* gs = qs + TILE;
    bf16x8 ag[2][2], aq[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      ag[0][u] = tr_frag(gs, fa, 32 * t + 16 * u, 0);
      aq[0][u] = tr_frag(qs, fa, 32 * t + 16 * u, 0);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int cb = dt & 1;
      if (dt + 1 < 4) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          ag[cb ^ 1][u] = tr_frag(gs, fa, 32 * t + 16 * u, dt + 1);
          aq[cb ^ 1][u] = tr_frag(qs, fa, 32 * t + 16 * u, dt + 1);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag[cb][u], pf[u], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cb][u], dsf[u], dk[dt], 0, 0, 0);
      }
    }
    // Each tr_frag is two DS reads.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // P and dS of half t of tile n (stage st), packed as B operands, fused with
  // sdp(st2, t2): the two are independent, so each k-step's S / dP MFMAs are
  // followed in program order by the softmax of two of this lane's 16 values
  // and the MFMAs run while the VALU work issues (8.8% off the backward at
  // d20 against the softmax as one block). The last tile computes a
  // throw-away S / dP of the stage after it.
  // MASK (a compile-time tag): whether any (query, key) pair of the half is
  // outside the causal band or past T; halves wholly inside skip the test.
  auto softmax_sdp = [&](auto mask_tag, int n, int st, int t, f32x16& s, f32x16& dp, bf16x8 (&pf)[2],
                         bf16x8 (&dsf)[2], int st2, int t2, f32x16& s2, f32x16& dp2)
                         __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float* ls = reinterpret_cast<const float*>(stage(st) + 2 * TILE);
    const float* ds = ls + QBW;
    const int qb = qb_first + n % nqt;
    const uint32_t lim = (uint32_t)qlim;
    float lq[16], dq[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ql = 32 * t + 8 * g + 4 * hl;
      const float4 l4 = *reinterpret_cast<const float4*>(ls + ql);
      const float4 d4 = *reinterpret_cast<const float4*>(ds + ql);
      lq[4 * g] = l4.x; lq[4 * g + 1] = l4.y; lq[4 * g + 2] = l4.z; lq[4 * g + 3] = l4.w;
      dq[4 * g] = d4.x; dq[4 * g + 1] = d4.y; dq[4 * g + 2] = d4.z; dq[4 * g + 3] = d4.w;
    }
    const int qrow = qb * QBW + 32 * t + 4 * hl - kpos;  // q - kpos for v = 0
    auto one = [&](int v) {
      // s[v]: query qb*64 + 32t + 8(v/4) + 4hl + v%4, key kpos.
      float p = fast_exp2(fmaf(s[v], sc, -lq[v]));
      if constexpr (MASK) p = (uint32_t)(qrow + 8 * (v >> 2) + (v & 3)) > lim ? 0.f : p;
      s[v] = p;
      dp[v] = p * (dp[v] - dq[v]);
    };
    const char* qs = stage(st2);
    const char* gs = qs + TILE;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s2[v] = 0.f;
      dp2[v] = 0.f;
    }
    bf16x8 fq[8], fg[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      fq[k] = row_frag(qs, fa, 32 * t2, k);
      fg[k] = row_frag(gs, fa, 32 * t2, k);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + 2 < 8) {
        fq[k + 2] = row_frag(qs, fa, 32 * t2, k + 2);
        fg[k + 2] = row_frag(gs, fa, 32 * t2, k + 2);
      }
      s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[k], as_bf16x8(kf[k]), s2, 0, 0, 0);
      dp2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fg[k], as_bf16x8(vf[k]), dp2, 0, 0, 0);
      one(2 * k);
      one(2 * k + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    pf[0] = pack_frag(s, 0);
    pf[1] = pack_frag(s, 8);
    dsf[0] = pack_frag(dp, 0);
    dsf[1] = pack_frag(dp, 8);
  };

  // Pipeline over halves: the S / dP MFMAs of the next half are issued while
  // the softmax of the current half runs (set A holds halves t = 0, set B
  // halves t = 1). Tile n lives in stage n % 4; tile n+2 is loaded during
  // tile n into the stage of tile n-2.
  f32x16 sa, da, sb, db;
  if (ntile > 0) {
    issue(0, 0);
    if (ntile > 1) issue(1, 1);
    VMCNT_BARRIER(0);
    sdp(0, 0, sa, da);
  }
  for (int n = 0; n < ntile; ++n) {
    const int st = n & (DKDV_NST - 1);
    if (n > 0) VMCNT_BARRIER(0);  // tile n+1 is in LDS; every wave is past tile n-1
    if (n + 2 < ntile) issue(n + 2, (n + 2) & (DKDV_NST - 1));
    bf16x8 pf[2], dsf[2];
    // Half t of tile n needs the mask when a pair of it is outside the band.
    auto need_mask = [&](int t) {
      const int q0 = (qb_first + n % nqt) * QBW + 32 * t;
      return (q0 < k0 + 31) || (q0 + 32 > T) || (q0 + 31 > k0 + W);
    };
    auto half = [&](int t, f32x16& s, f32x16& dp, int st2, int t2, f32x16& s2, f32x16& dp2)
        __attribute__((always_inline)) {
      if (need_mask(t))
        softmax_sdp(std::true_type{}, n, st, t, s, dp, pf, dsf, st2, t2, s2, dp2);
      else
        softmax_sdp(std::false_type{}, n, st, t, s, dp, pf, dsf, st2, t2, s2, dp2);
    };
    half(0, sa, da, st, 1, sb, db);
    dvdk(st, 0, pf, dsf);
    half(1, sb, db, (n + 1) & (DKDV_NST - 1), 0, sa, da);
    dvdk(st, 1, pf, dsf);
  }

  if (kpos < T) {
    float scale = 0.08838834764831845f;
    if (rstd_qk) {  // k's QK-norm + RoPE backward (wave-uniform)
      int kp = kpos;  // opaque copy: addresses computed here, not before the loop
      asm volatile("" : "+v"(kp));
      const long row = (long)b * T + kp;
      qknorm_rope_bwd_acc(dk, scale, kf, rstd_qk[row * (H + Hkv) + H + hk], cs + 2L * kp * 64, hl);
      scale = 1.f;
    }
    uint16_t* krow = dqkv + ((long)b * T + kpos) * ld + d + hk * HD;
    uint16_t* vrow = krow + dkv;
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
__global__ void __launch_bounds__(NTHR, 2)
    attn_bwd_dq_kernel(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ o,
                       const uint16_t* __restrict__ dO, const float* __restrict__ lse2,
                       float* __restrict__ delta, uint16_t* __restrict__ dqkv,
                       const float* __restrict__ rstd_qk, const float* __restrict__ cs, int T, int H, int Hkv,
                       int W) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  int xb, bh;
  head_block<4>(xb, bh);
  const int nqb = (T + QB - 1) / QB;
  const int qblk = nqb - 1 - xb;
  const int b = bh / H;
  const int h = bh - b * H;
  const int d = H * HD;
  const int dkv = Hkv * HD;
  const long ld = (long)d + 2L * dkv;
  const uint16_t* qbase = qkv + (long)b * T * ld + h * HD;
  const uint16_t* kbase = qkv + (long)b * T * ld + d + (h / (H / Hkv)) * HD;
  const uint16_t* vbase = kbase + dkv;
  const uint16_t* dobase = dO + (long)b * T * d + h * HD;
  const float sc = GPT_LOG2E * 0.08838834764831845f;

  const int q0 = qblk * QB + wave * 32;
  const int qpos = q0 + (lane & 31);
  const bool qok = qpos < T;
  const int qc = min(qpos, T - 1);

  FragAddr fa;
  frag_addr(lane, fa);

  uint4 qf[8], gf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qf[k] = *reinterpret_cast<const uint4*>(qbase + (long)qc * ld + 16 * k + 8 * hl);
    gf[k] = *reinterpret_cast<const uint4*>(dobase + (long)qc * d + 16 * k + 8 * hl);
  }
  const float lq = lse2[(long)bh * T + qc];
  // delta = rowsum(dO * O) of this lane's query (the lane holds half the
  // dims, lane ^ 32 the other half); also written out for the dK/dV kernel.
  float dq_ = 0.f;
  {
    const uint16_t* orow = o + ((long)b * T + qc) * d + h * HD + 8 * hl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 ov = *reinterpret_cast<const uint4*>(orow + 16 * k);
      const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
      const uint32_t gw[4] = {gf[k].x, gf[k].y, gf[k].z, gf[k].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) dq_ += bf_lo(ow[w]) * bf_lo(gw[w]) + bf_hi(ow[w]) * bf_hi(gw[w]);
    }
    dq_ += __shfl_xor(dq_, 32, 64);
    if (hl == 0 && qok) delta[(long)bh * T + qpos] = dq_;
  }

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  const int qmax = min(T - 1, qblk * QB + QB - 1);
  const int nkb = qmax / KB + 1;
  const int kb_lo = max(0, qblk * QB - W) / KB;

  TileDma td;
  tile_dma_init(td, ld, wave, lane);
  // Visible keys: kwin .. kwin + kspan, i.e. qpos - W .. min(qpos, T - 1)
  // (lanes past T are discarded).
  const int kwin = qpos - W;
  const uint32_t kspan = (uint32_t)(min(qpos, T - 1) - kwin);

  auto issue = [&](int kb, int st) {
    char* ks = smem + st * 2 * TILE;
    dma_tile_fast(kbase, ld, kb * KB, T, ks, wave, lane, td);
    dma_tile_fast(vbase, ld, kb * KB, T, ks + TILE, wave, lane, td);
  };

  auto block = [&](int kb, int st) {
    const char* ks = smem + st * 2 * TILE;
    const char* vs = ks + TILE;
    if (kb * KB > q0 + 31 || kb * KB + KB - 1 < q0 - W) return;
    const bool need_mask =
        (kb * KB + KB - 1 > q0) || (kb * KB + KB > T) || (q0 + 32 > T) || (kb * KB < q0 + 31 - W);
    // One 32-key half of the tile at a time (keeps two accumulators live, not
    // four); fragments are read one k-step (or one dim tile) ahead.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 sv, dp;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = 0.f;
        dp[v] = 0.f;
      }
      bf16x8 fk[8], fv[8];
      mfma_prio_begin();
      fk[0] = row_frag(ks, fa, 32 * t, 0);
      fv[0] = row_frag(vs, fa, 32 * t, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k + 1 < 8) {
          fk[k + 1] = row_frag(ks, fa, 32 * t, k + 1);
          fv[k + 1] = row_frag(vs, fa, 32 * t, k + 1);
        }
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[k], as_bf16x8(qf[k]), sv, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[k], as_bf16x8(gf[k]), dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int k = 0; k < 7; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      mfma_prio_end();
      // sv[v]: key kb*64 + 32t + 8(v/4) + 4hl + v%4, query qpos.
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * KB + 32 * t + 8 * (v >> 2) + 4 * hl + (v & 3);
        float p = fast_exp2(fmaf(sv[v], sc, -lq));
        if (need_mask && (uint32_t)(key - kwin) > kspan) p = 0.f;
        dp[v] = p * (dp[v] - dq_);
      }
      const bf16x8 ds0 = pack_frag(dp, 0);
      const bf16x8 ds1 = pack_frag(dp, 8);
      bf16x8 ak[2][2];
      mfma_prio_begin();
      ak[0][0] = tr_frag(ks, fa, 32 * t, 0);
      ak[0][1] = tr_frag(ks, fa, 32 * t + 16, 0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int cb = dt & 1;
        if (dt + 1 < 4) {
          ak[cb ^ 1][0] = tr_frag(ks, fa, 32 * t, dt + 1);
          ak[cb ^ 1][1] = tr_frag(ks, fa, 32 * t + 16, dt + 1);
        }
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[cb][0], ds0, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[cb][1], ds1, acc[dt], 0, 0, 0);
      }
      mfma_prio_end();
    }
  };

  issue(kb_lo, 0);
  VMCNT_BARRIER(0);
  for (int kb = kb_lo; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) issue(kb + 1, 1);
    block(kb, 0);
    VMCNT_BARRIER(0);
    if (kb + 1 < nkb) {
      if (kb + 2 < nkb) issue(kb + 2, 0);
      block(kb + 1, 1);
      VMCNT_BARRIER(0);
    }
  }

  if (qok) {
    float scale = 0.08838834764831845f;
    if (rstd_qk) {  // q's QK-norm + RoPE backward (wave-uniform)
      // An opaque copy of qpos keeps the compiler from computing these
      // addresses before the loop (they would be live across it).
      int qp = qpos;
      asm volatile("" : "+v"(qp));
      const long row = (long)b * T + qp;
      qknorm_rope_bwd_acc(acc, scale, qf, rstd_qk[row * (H + Hkv) + h], cs + 2L * qp * 64, hl);
      scale = 1.f;
    }
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

hipError_t launch_attention_fwd_window(const uint16_t* qkv, uint16_t* o, float* lse2, int B, int T, int H,
                                       int Hkv, int window, hipStream_t s) {
  if (B <= 0 || T <= 0 || H <= 0) return hipSuccess;
  if (Hkv <= 0 || H % Hkv != 0) return hipErrorInvalidValue;
  const int W = (window < 0 || window > T) ? T : window;
  dim3 grid((T + QB - 1) / QB, B * H);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(NTHR), 0, s, qkv, o, lse2, T, H, Hkv, W);
  return hipGetLastError();
}

hipError_t launch_attention_bwd_window(const uint16_t* qkv, const uint16_t* o, const float* lse2,
                                       const uint16_t* dO, uint16_t* dqkv, float* delta, int B, int T, int H,
                                       int Hkv, int window, hipStream_t s, const float* rstd_qk,
                                       const float* cs) {
  if (B <= 0 || T <= 0 || H <= 0) return hipSuccess;
  if (Hkv <= 0 || H % Hkv != 0) return hipErrorInvalidValue;
  const int W = (window < 0 || window > T) ? T : window;
  // dQ first: it also writes delta = rowsum(dO * O), which dK/dV reads.
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((T + QB - 1) / QB, B * H), dim3(NTHR), 0, s, qkv, o, dO,
                     lse2, delta, dqkv, rstd_qk, cs, T, H, Hkv, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((T + KBW - 1) / KBW, B * Hkv), dim3(NTHR), 0, s, qkv,
                     dO, lse2, delta, dqkv, rstd_qk, cs, T, H, Hkv, W);
  return hipGetLastError();
}
