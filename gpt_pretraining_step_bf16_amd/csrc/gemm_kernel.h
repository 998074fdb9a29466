// bf16 MFMA GEMM kernel for gfx950 (device code; instantiated per operand
// layout in gemm_*.hip): every dense contraction of the step (QKV, O, MLP
// and head projections forward and backward, weight gradients, Newton-Schulz).
// The EPI_H_* instantiations (Newton-Schulz after its first iteration) take
// fp16 operands through v_mfma_f32_32x32x16_f16, the same shape and rate;
// the operand path (loads, LDS layout, fragment reads) is type-blind.
//
// Design
//  * Macro tile 256 x 256, 256 threads = 4 wave64s in a 2 x 2 grid, each wave
//    owning a 128 x 128 sub-tile as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles
//    (256 fp32 accumulators per lane, held in AGPRs).
//  * Operands go from HBM straight into LDS with 16-byte global_load_lds
//    (no register staging), through a 4-stage ring of 32-wide k-blocks
//    (4 x 32 KB): three k-blocks are in flight while one is consumed, which
//    covers the load latency that a one-block register prefetch left exposed.
//  * Each operand keeps its memory layout in LDS. A K-contiguous operand is
//    staged [row][32 k] (64 B rows) and read with ds_read_b128. A K-strided
//    operand (activations read along tokens for weight gradients, weights
//    read along their out dimension) is staged [32 k][256 rows] (512 B rows)
//    and read with ds_read_b64_tr_b16, the gfx950 transposing LDS read, which
//    hands each lane the same 8-element k-run a K-contiguous read would.
//    16-byte chunks are XOR-swizzled per row so fragment reads are
//    bank-conflict free; the swizzle is applied by choosing which global
//    chunk each lane fetches (lane l of a direct load lands at base + 16 l).
//  * Fragments of the next 16-wide k-step are read before the MFMAs of the
//    current one (sched_barrier keeps that order), so LDS latency hides
//    under 16 MFMAs.
//  * Partial tiles: rows past M / N load clamped (valid) addresses and are
//    never stored; a k-block past the end of K is zeroed in LDS before use.
//  * The MFMA computes the transposed tile (B fragment as the A input), so a
//    lane holds 4 consecutive output columns, stored straight from the
//    accumulators (8-byte bf16 / 16-byte fp32 stores).
//  * Workgroup ids are remapped so consecutive tiles run on one XCD (ids are
//    dealt round-robin over the 8 XCDs), then grouped 4 tile-rows at a time so
//    an XCD's tiles share A rows and B columns in its L2.
#pragma once

#include <type_traits>

#include "common.h"
#include "lds_dma.h"
#include "gemm.h"

namespace gemm_impl {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BKD = 32;                 // k per stage
constexpr int NST = 4;                  // stages in the ring
constexpr int NTHR = 256;
constexpr int OP_BYTES = BM * BKD * 2;  // one operand's stage: 16 KB
constexpr int STAGE_BYTES = 2 * OP_BYTES;

// Byte offset of (row r, 16-byte k-chunk c) in a K-contiguous stage [256][32].
__device__ __forceinline__ int koff(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
// Byte offset of (k-row kr, 16-byte row-chunk c) in a K-strided stage [32][256].
__device__ __forceinline__ int toff(int kr, int c) { return kr * 512 + ((c ^ ((kr & 3) << 2)) << 4); }

// Work item of this workgroup: output tile (tm, tn) and batch / split index z.
// Workgroups are dealt round-robin over the 8 XCDs in launch order, so the
// linear launch index is remapped to give consecutive work items (the tiles of
// one matrix, then those of the next) to one XCD, whose L2 then holds their
// shared operand panels; within a matrix, tiles go 4 tile-rows at a time along
// N. A symmetric output enumerates its upper triangle tm <= tn.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn, int& z) {
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int per = gridDim.x;
  const int total = per * gridDim.y;
  int lin = blockIdx.x + per * blockIdx.y;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  z = lin / per;
  int t = lin - z * per;
  if (p.sym) {
    tm = 0;
    while (t >= tiles_m - tm) {
      t -= tiles_m - tm;
      ++tm;
    }
    tn = tm + t;
  } else {
    constexpr int GM = 4;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_group = t - group * GM * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
  }
}

// Work item `lin` of `total` (per tiles per batch / split): output tile
// (tm, tn) and batch / split index z, with the same XCD-aware remap as
// tile_coords (a persistent workgroup on XCD x walks lin = x, x + G, ... with
// G a multiple of 8).
__device__ __forceinline__ void tile_coords_lin(const GemmArgs& p, int lin, int per, int total, int tiles_m,
                                                int tiles_n, int& tm, int& tn, int& z) {
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  z = lin / per;
  int t = lin - z * per;
  if (p.sym) {
    tm = 0;
    while (t >= tiles_m - tm) {
      t -= tiles_m - tm;
      ++tm;
    }
    tn = tm + t;
  } else {
    constexpr int GM = 4;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_group = t - group * GM * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
  }
}

// Issue 1 KB block `blk` (0..15) of one operand's k-block [k0, k0 + 32) into
// the LDS stage buffer at byte address lds_op (wave-uniform); the 4 waves
// issue blocks 4 wave .. 4 wave + 3. Rows and k past the operand are clamped.
template <bool KMAJ>
__device__ __forceinline__ void issue_one(const uint16_t* __restrict__ base, long ld, int row0,
                                          int rows, int k0, int kend, uint32_t lds_op, int blk,
                                          int lane) {
  {
    const uint16_t* src;
    if (KMAJ) {
      // 1 KB = rows 16 blk .. +15, 64 B each; lane l -> row 16 blk + l/4, slot l%4.
      const int r = 16 * blk + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      const int gr = min(row0 + r, rows - 1);
      const int kk = min(k0 + 8 * c, kend - 8);
      src = base + (long)gr * ld + kk;
    } else {
      // 1 KB = k-rows 2 blk, 2 blk + 1, 512 B each; lane l -> k-row 2 blk + l/32, slot l%32.
      const int kr = 2 * blk + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      const int gk = min(k0 + kr, kend - 1);
      const int gm = min(row0 + 8 * c, rows - 8);
      src = base + (long)gk * ld + gm;
    }
    dma16(src, lds_op + blk * 1024);
  }
}

// Per-lane byte offsets, relative to a full k-block's scalar base, of the
// four 1 KB blocks wave `wave` loads (same layout as issue_one).
template <bool KMAJ>
__device__ __forceinline__ void block_offsets(long ld, int wave, int lane, uint32_t (&off)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int blk = 4 * wave + j;
    if (KMAJ) {
      const int r = 16 * blk + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      off[j] = (uint32_t)(((long)r * ld + 8 * c) * 2);
    } else {
      const int kr = 2 * blk + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      off[j] = (uint32_t)(((long)kr * ld + 8 * c) * 2);
    }
  }
}

// Zero the k-range [kvalid, 32) of one operand's stage (tail k-block).
template <bool KMAJ>
__device__ __forceinline__ void zero_tail(char* lds_op, int kvalid, int tid) {
  if (KMAJ) {
    // 256 rows x 4 chunks; chunk c holds k 8c..8c+7.
    for (int i = tid; i < BM * 4; i += NTHR) {
      const int r = i >> 2, c = i & 3;
      if (8 * c >= kvalid) *reinterpret_cast<uint4*>(lds_op + koff(r, c)) = make_uint4(0, 0, 0, 0);
    }
  } else {
    for (int i = tid; i < BKD * 32; i += NTHR) {
      const int kr = i >> 5, c = i & 31;
      if (kr >= kvalid) *reinterpret_cast<uint4*>(lds_op + toff(kr, c)) = make_uint4(0, 0, 0, 0);
    }
  }
}

// 32 x 16 fragment (rows rb + lane%32, k-step ks of the stage) as 8 bf16.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const char* lds_op, int rb, int ks, int lane) {
  if (KMAJ) {
    const int r = rb + (lane & 31);
    const int c = 2 * ks + (lane >> 5);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds_op + koff(r, c)));
  } else {
    // Group g = lane/16 covers rows rb + 16 (g & 1) .. +15 and k 16 ks + 8 (g >> 1) .. +7.
    // Group-lane p addresses k-row (base + p/4) at row offset 4 (p % 4); two reads
    // (k base and k base + 4) give the lane's 8 k values for its row.
    const int g = lane >> 4, p = lane & 15;
    const int m = rb + 16 * (g & 1) + 4 * (p & 3);
    const int kr = 16 * ks + 8 * (g >> 1) + (p >> 2);
    const int c = m >> 3, within = (m & 7) * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_V4S(lds_op + toff(kr, c) + within));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_V4S(lds_op + toff(kr + 4, c) + within));
    const uint2 a = __builtin_bit_cast(uint2, lo);
    const uint2 b = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
  }
}

// Wait until at most `n` of this wave's direct loads are outstanding (they
// complete in issue order), then barrier. Both are compiler memory barriers,
// so no LDS access moves across them.
__device__ __forceinline__ void ring_sync(int n) {
  if (n >= 16) {
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else if (n >= 8) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void store_bf16x4(void* p, float v0, float v1, float v2, float v3) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
}

// hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void store_hilo4(void* ph, void* pl, const float* v) {
  float hi[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = bf2f(f2bf(v[r]));
    lo[r] = v[r] - hi[r];
  }
  store_bf16x4(ph, hi[0], hi[1], hi[2], hi[3]);
  store_bf16x4(pl, lo[0], lo[1], lo[2], lo[3]);
}

__device__ __forceinline__ void load_bf16x4(const void* p, float* v) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = bf_lo(u.x);
  v[1] = bf_hi(u.x);
  v[2] = bf_lo(u.y);
  v[3] = bf_hi(u.y);
}

// Whether an epilogue reads memory besides the accumulators.
template <int E>
constexpr bool epi_reads() {
  return E == EPI_F32_ACC || E == EPI_RESID_BF16 || E == EPI_DRELU2_BF16 || E == EPI_NS_POLY ||
         E == EPI_NS_UPDATE || E == EPI_H_NS_POLY || E == EPI_H_NS_UPDATE || E == EPI_H_NS_LAST;
}

// Whether the operands are fp16 (the EPI_H_* epilogues) rather than bf16.
template <int E>
constexpr bool f16_operands() {
  return E == EPI_H_GRAM || E == EPI_H_NS_POLY || E == EPI_H_NS_UPDATE || E == EPI_H_NS_LAST;
}

// One 32 x 32 x 16 MFMA of the instantiation's operand type (the fragments
// hold the operands' 16-bit patterns either way).
template <int E>
__device__ __forceinline__ f32x16 mfma16(const bf16x8& b, const bf16x8& a, const f32x16& c) {
  if constexpr (f16_operands<E>())
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
}

// Per-lane output pointers of one wave's tile: element (row m, column n) of
// C / C2 / C3 / D / D2 for the lane's rows m = mb + 32 i and columns
// n = nb + 32 j + 8 g + r (mb, nb the lane's first row and column).
struct EpiPtrs {
  float* cf;            // C as fp32 (F32, F32_ACC, SPLITK)
  uint16_t* cb;         // C as bf16 (fp16 for EPI_NS_UPDATE and EPI_H_*)
  uint16_t* c2;         // lo half of hi/lo outputs
  float* c3;            // fp32 X (NS_UPDATE; D layout)
  bool c3ok;            // C3 given (NS_UPDATE may leave it null)
  const uint16_t* db;   // D as bf16
  const uint16_t* d2;   // D2 as bf16
  const float* df;      // D as fp32
  uint16_t* cbt;        // transposed C / C2 of a symmetric output: element (n, m)
  uint16_t* c2t;        //   at cbt[(n - nb) * ldc + (m - mb)]
  bool tr;              // also store the tile transposed (off-diagonal symmetric tile)
  long ldc, ldd;
  float alpha, beta;
};

// What the epilogue of group (i, j, g) reads, in one 16-byte slot.
template <int E>
__device__ __forceinline__ uint4 epi_load(const EpiPtrs& e, int i, int j, int g) {
  const long co = 32L * i * e.ldc + 32 * j + 8 * g;
  const long dof = 32L * i * e.ldd + 32 * j + 8 * g;
  uint4 r = make_uint4(0, 0, 0, 0);
  if constexpr (E == EPI_F32_ACC) {
    if (e.beta != 0.f) r = *reinterpret_cast<const uint4*>(e.cf + co);
  } else if constexpr (E == EPI_RESID_BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(e.cb + co);
    r.x = u.x;
    r.y = u.y;
  } else if constexpr (E == EPI_DRELU2_BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(e.db + dof);
    r.x = u.x;
    r.y = u.y;
  } else if constexpr (E == EPI_NS_POLY) {
    const uint2 h = *reinterpret_cast<const uint2*>(e.db + dof);
    const uint2 l = *reinterpret_cast<const uint2*>(e.d2 + dof);
    r = make_uint4(h.x, h.y, l.x, l.y);
  } else if constexpr (E == EPI_H_NS_POLY || E == EPI_H_NS_UPDATE || E == EPI_H_NS_LAST) {
    const uint2 u = *reinterpret_cast<const uint2*>(e.db + dof);
    r.x = u.x;
    r.y = u.y;
  } else if constexpr (E == EPI_NS_UPDATE) {
    r = *reinterpret_cast<const uint4*>(e.df + dof);
  }
  return r;
}

// Transposed hi/lo store of group (i, j, g) of a symmetric output:
// C(n + r, m) for the lane's row m and columns n .. n+3 (consecutive lanes
// hold consecutive m, so each store coalesces across the wave).
__device__ __forceinline__ void store_hilo4_t(const EpiPtrs& e, int i, int j, int g, const float* w) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const long o = (long)(32 * j + 8 * g + r) * e.ldc + 32 * i;
    const uint32_t h = f2bf(w[r]);
    e.cbt[o] = (uint16_t)h;
    e.c2t[o] = (uint16_t)f2bf(w[r] - bf2f(h));
  }
}

__device__ __forceinline__ void store_h4(void* p, const float* w) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_h2(w[0], w[1]), pack_h2(w[2], w[3]));
}

// Transposed fp16 store of group (i, j, g) of a symmetric output (as
// store_hilo4_t, one output).
__device__ __forceinline__ void store_h4_t(const EpiPtrs& e, int i, int j, int g, const float* w) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const long o = (long)(32 * j + 8 * g + r) * e.ldc + 32 * i;
    e.cbt[o] = __builtin_bit_cast(uint16_t, (_Float16)w[r]);
  }
}

// Epilogue of group (i, j, g) for a compile-time mode; v are the four
// accumulators, `in` what epi_load returned.
template <int E>
__device__ __forceinline__ void epi4(const EpiPtrs& e, int i, int j, int g, const float* v, const uint4& in) {
  const long co = 32L * i * e.ldc + 32 * j + 8 * g;
  const long dof = 32L * i * e.ldd + 32 * j + 8 * g;
  if constexpr (E == EPI_F32 || E == EPI_SPLITK) {
    *reinterpret_cast<float4*>(e.cf + co) =
        make_float4(e.alpha * v[0], e.alpha * v[1], e.alpha * v[2], e.alpha * v[3]);
  } else if constexpr (E == EPI_F32_ACC) {
    const float4 o = __builtin_bit_cast(float4, in);
    *reinterpret_cast<float4*>(e.cf + co) =
        make_float4(e.beta * o.x + e.alpha * v[0], e.beta * o.y + e.alpha * v[1],
                    e.beta * o.z + e.alpha * v[2], e.beta * o.w + e.alpha * v[3]);
  } else if constexpr (E == EPI_BF16) {
    store_bf16x4(e.cb + co, e.alpha * v[0], e.alpha * v[1], e.alpha * v[2], e.alpha * v[3]);
  } else if constexpr (E == EPI_RELU_BF16) {
    store_bf16x4(e.cb + co, fmaxf(v[0], 0.f), fmaxf(v[1], 0.f), fmaxf(v[2], 0.f), fmaxf(v[3], 0.f));
  } else if constexpr (E == EPI_RESID_BF16) {
    store_bf16x4(e.cb + co, bf_lo(in.x) + v[0], bf_hi(in.x) + v[1], bf_lo(in.y) + v[2], bf_hi(in.y) + v[3]);
  } else if constexpr (E == EPI_DRELU2_BF16) {
    // d relu(u)^2 / du = 2 relu(u) = 2 sqrt(h), h = relu(u)^2 as stored
    // (v_sqrt_f32 directly: its ~1 ulp is far below the bf16 output's).
    store_bf16x4(e.cb + co, 2.f * v[0] * __builtin_amdgcn_sqrtf(bf_lo(in.x)),
                 2.f * v[1] * __builtin_amdgcn_sqrtf(bf_hi(in.x)), 2.f * v[2] * __builtin_amdgcn_sqrtf(bf_lo(in.y)),
                 2.f * v[3] * __builtin_amdgcn_sqrtf(bf_hi(in.y)));
  } else if constexpr (E == EPI_RELU2_BF16) {
    const float r0 = fmaxf(v[0], 0.f), r1 = fmaxf(v[1], 0.f), r2 = fmaxf(v[2], 0.f), r3 = fmaxf(v[3], 0.f);
    store_bf16x4(e.cb + co, r0 * r0, r1 * r1, r2 * r2, r3 * r3);
  } else if constexpr (E == EPI_HILO) {
    float w[4] = {e.alpha * v[0], e.alpha * v[1], e.alpha * v[2], e.alpha * v[3]};
    store_hilo4(e.cb + co, e.c2 + co, w);
    if (e.tr) store_hilo4_t(e, i, j, g, w);
  } else if constexpr (E == EPI_NS_POLY) {
    const float h[4] = {bf_lo(in.x), bf_hi(in.x), bf_lo(in.y), bf_hi(in.y)};
    const float l[4] = {bf_lo(in.z), bf_hi(in.z), bf_lo(in.w), bf_hi(in.w)};
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = e.alpha * v[r] + e.beta * (h[r] + l[r]);
    store_hilo4(e.cb + co, e.c2 + co, w);
    if (e.tr) store_hilo4_t(e, i, j, g, w);
  } else if constexpr (E == EPI_NS_UPDATE) {
    const float4 x = __builtin_bit_cast(float4, in);
    float w[4] = {e.alpha * v[0] + e.beta * x.x, e.alpha * v[1] + e.beta * x.y,
                  e.alpha * v[2] + e.beta * x.z, e.alpha * v[3] + e.beta * x.w};
    if (e.c3ok) *reinterpret_cast<float4*>(e.c3 + dof) = make_float4(w[0], w[1], w[2], w[3]);
    store_h4(e.cb + co, w);
  } else if constexpr (E == EPI_H_NS_UPDATE || E == EPI_H_NS_LAST) {
    const float w[4] = {e.alpha * v[0] + e.beta * h_lo(in.x), e.alpha * v[1] + e.beta * h_hi(in.x),
                        e.alpha * v[2] + e.beta * h_lo(in.y), e.alpha * v[3] + e.beta * h_hi(in.y)};
    if constexpr (E == EPI_H_NS_UPDATE)
      store_h4(e.cb + co, w);
    else
      *reinterpret_cast<float4*>(e.c3 + dof) = make_float4(w[0], w[1], w[2], w[3]);
  } else if constexpr (E == EPI_H_GRAM) {
    const float w[4] = {e.alpha * v[0], e.alpha * v[1], e.alpha * v[2], e.alpha * v[3]};
    store_h4(e.cb + co, w);
    if (e.tr) store_h4_t(e, i, j, g, w);
  } else if constexpr (E == EPI_H_NS_POLY) {
    const float w[4] = {e.alpha * v[0] + e.beta * h_lo(in.x), e.alpha * v[1] + e.beta * h_hi(in.x),
                        e.alpha * v[2] + e.beta * h_lo(in.y), e.alpha * v[3] + e.beta * h_hi(in.y)};
    store_h4(e.cb + co, w);
    if (e.tr) store_h4_t(e, i, j, g, w);
  }
}

// Store a finished 256 x 256 tile straight from the accumulators.
// acc[i][j][4g + r] is C(m, n) with m = m0 + wm*128 + i*32 + lane%32 and
// n = n0 + wn*128 + j*32 + 8g + 4*(lane/32) + r.
// Epilogues that read memory load a whole 32-row block's inputs at once and
// issue the next block's loads before the current block's stores (the
// blocks touch disjoint rows), so load latency is paid about once per block
// instead of once per group. Interior tiles skip the bounds checks.
template <int E, int NJ>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const f32x16 (&acc)[4][NJ], int bi, int si,
                                           int m0, int n0, int row_off, int col_off, int lane) {
  const int mb = m0 + row_off + (lane & 31);
  const int nb = n0 + col_off + 4 * (lane >> 5);
  const long co = (long)bi * p.sc + (long)mb * p.ldc + nb;
  const long dof = (long)bi * p.sd + (long)mb * p.ldd + nb;
  EpiPtrs e;
  e.cf = reinterpret_cast<float*>(p.c) + co + (E == EPI_SPLITK ? (long)si * p.s_split : 0L);
  e.cb = reinterpret_cast<uint16_t*>(p.c) + co;
  e.c2 = reinterpret_cast<uint16_t*>(p.c2) + co;
  e.c3ok = p.c3 != nullptr;
  e.c3 = e.c3ok ? reinterpret_cast<float*>(p.c3) + dof : nullptr;
  e.db = reinterpret_cast<const uint16_t*>(p.d) + dof;
  e.d2 = reinterpret_cast<const uint16_t*>(p.d2) + dof;
  e.df = reinterpret_cast<const float*>(p.d) + dof;
  const long cot = (long)bi * p.sc + (long)nb * p.ldc + mb;
  e.cbt = reinterpret_cast<uint16_t*>(p.c) + cot;
  e.c2t = reinterpret_cast<uint16_t*>(p.c2) + cot;
  e.tr = p.sym && (m0 != n0);
  e.ldc = p.ldc;
  e.ldd = p.ldd;
  e.alpha = (E == EPI_SPLITK) ? 1.f : p.alpha;
  e.beta = p.beta;
  const int M = p.M, N = p.N;
  // Straight-line code for interior tiles: with no branches between them the
  // loads and stores keep exact wait counts instead of a full drain per group.
  auto run = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    auto ok = [&](int i, int j, int g) { return FULL || (mb + 32 * i < M && nb + 32 * j + 8 * g < N); };
    uint4 in[2][NJ][4];
    auto load_block = [&](int i, uint4 (&dst)[NJ][4]) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) dst[j][g] = ok(i, j, g) ? epi_load<E>(e, i, j, g) : make_uint4(0, 0, 0, 0);
    };
    // 16-byte inputs (fp32 or hi/lo pairs) load block by block; 8-byte ones
    // also prefetch the next block (registers allow it).
    constexpr bool WIDE = E == EPI_F32_ACC || E == EPI_NS_POLY || E == EPI_NS_UPDATE;
    if constexpr (epi_reads<E>()) load_block(0, in[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (epi_reads<E>()) {
        if (i + 1 < 4 && !WIDE) load_block(i + 1, in[(i + 1) & 1]);
        if (i > 0 && WIDE) load_block(i, in[i & 1]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (ok(i, j, g)) {
            const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]};
            epi4<E>(e, i, j, g, v, in[i & 1][j][g]);
          }
        }
    }
  };
  if ((m0 + BM <= M) && (n0 + BN <= N))
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ---------------------------------------------------------------------------
// Epilogue through LDS for bf16 outputs of the ping-pong kernel (128 x 64 per
// wave). The accumulator layout gives a lane 4 consecutive columns of one row,
// so direct bf16 stores write 16 bytes per row per instruction. Instead, per
// 32-row block, each wave applies the element-wise math, writes the bf16
// 32 x 64 block into a private LDS region (rows padded to 144 bytes, which
// keeps the writes free of bank conflicts), reads it back row-contiguous and
// stores whole 128-byte row segments (8 lanes per row). Edge tiles check
// every row segment against M and N (N a multiple of 4).
// ---------------------------------------------------------------------------
template <int E>
constexpr bool lds_epi() {
  return E == EPI_BF16 || E == EPI_RELU_BF16 || E == EPI_RELU2_BF16;
}
constexpr int STG_RS = 144;  // padded row stride of a staging block (bytes)

template <int E, bool FULL>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& p, const f32x16 (&acc)[4][2], int bi, int m0,
                                               int n0, int row_off, int col_off, int lane, int wave, char* smem) {
  const int rows_left = p.M - (m0 + row_off), cols_left = p.N - (n0 + col_off);
  char* wreg = smem + wave * (32 * STG_RS);
  const int r = lane & 31, hl = lane >> 5;
  const long ldc = p.ldc;
  uint16_t* cb = reinterpret_cast<uint16_t*>(p.c) + (long)bi * p.sc + (long)(m0 + row_off) * ldc + (n0 + col_off);
  const float alpha = p.alpha;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // (Scheduling barriers keep each block's registers from being hoisted
    // across blocks.)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * j + 8 * g + 4 * hl;
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float v = acc[i][j][4 * g + t];
          if constexpr (E == EPI_BF16) {
            o[t] = alpha * v;
          } else if constexpr (E == EPI_RELU_BF16) {
            o[t] = fmaxf(v, 0.f);
          } else {
            const float u = fmaxf(v, 0.f);
            o[t] = u * u;
          }
        }
        *reinterpret_cast<uint2*>(wreg + r * STG_RS + col * 2) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 8 * q + (lane >> 3), cc = lane & 7;
      const uint4 val = *reinterpret_cast<const uint4*>(wreg + rr * STG_RS + cc * 16);
      uint16_t* dst = cb + (long)(32 * i + rr) * ldc + cc * 8;
      if (FULL || (32 * i + rr < rows_left && cc * 8 + 8 <= cols_left)) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else if (32 * i + rr < rows_left && cc * 8 + 4 <= cols_left) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(val.x, val.y);
      }
    }
  }
}

// QKV projection epilogue with QK-norm and RoPE ([CT50] "1. Modelo GPT": q and
// k normalised per head, then rotated): the two waves of one group that hold
// a head's dims 0..63 and 64..127 (waves w, w ^ 1, the same 128 rows) each
// stage their 32 x 64 block as bf16, plus every row's fp32 sum of squares
// over its 64 columns; after a workgroup barrier each lane takes 8 columns of
// a row from both blocks (its RoPE pairs (j, j + 64)), normalises with the
// summed squares and rotates; a second barrier frees the staging for the
// next block. A lane's rows within the group are lane / 8 + 8 k (k = 4 i + q),
// so when the sequence length is a multiple of 256 (a tile never spans two
// sequences) the (cos, sin) of its pairs advance from row to row by a
// rotation by 8 positions (table row 8); otherwise they are read per row.
// Heads at or past qk_heads (v) are stored as they are.
template <bool FULL>
__device__ __forceinline__ void store_tile_qkn(const GemmArgs& p, const f32x16 (&acc)[4][2], int m0, int n0,
                                               int row_off, int col_off, int lane, int wave, char* smem) {
  const int rows_left = p.M - (m0 + row_off), cols_left = p.N - (n0 + col_off);
  // Two sets of staging regions, alternating by block, so one barrier per
  // block suffices: a region is rewritten two blocks later, after the
  // partner has passed the next block's barrier (its reads done).
  constexpr int SET = 8 * 32 * STG_RS + 8 * 32 * 4;  // 8 staging blocks + row sums
  const int r = lane & 31, hl = lane >> 5, cc = lane & 7;
  const long ldc = p.ldc;
  uint16_t* cb = reinterpret_cast<uint16_t*>(p.c) + (long)(m0 + row_off) * ldc + (n0 + col_off);
  const int head = (n0 + col_off) >> 7;
  const bool normed = head < p.qk_heads;             // wave-uniform, same for both waves of the head
  const bool lo_half = ((col_off >> 6) & 1) == 0;    // this wave holds dims 0..63 (else 64..127)
  const int T = p.qk_T;
  const bool rec = (T & 255) == 0;
  const long grow0 = (long)m0 + row_off + (lane >> 3);  // the lane's first row
  float cv[8], sv[8], c8[8], s8[8];
  auto load_cs = [&](long t, float (&c)[8], float (&sn)[8]) {
    const float4* q = reinterpret_cast<const float4*>(p.qk_cs + 2 * (t * 64 + 8 * cc));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = q[k];
      c[2 * k] = v.x;
      sn[2 * k] = v.y;
      c[2 * k + 1] = v.z;
      sn[2 * k + 1] = v.w;
    }
  };
  if (normed) {
    load_cs(grow0 % T, cv, sv);
    if (rec) load_cs(8, c8, s8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    char* set = smem + (i & 1) * SET;
    char* wreg = set + wave * (32 * STG_RS);
    const char* preg = set + (wave ^ 1) * (32 * STG_RS);
    float* part = reinterpret_cast<float*>(set + 8 * 32 * STG_RS);  // [wave][row]
    __builtin_amdgcn_sched_barrier(0);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * j + 8 * g + 4 * hl;
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          o[t] = acc[i][j][4 * g + t];
          ss += o[t] * o[t];
        }
        *reinterpret_cast<uint2*>(wreg + r * STG_RS + col * 2) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      }
    ss += __shfl_xor(ss, 32, 64);
    if (hl == 0) part[wave * 32 + r] = ss;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma nounroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 8 * q + (lane >> 3);
      uint4 val = *reinterpret_cast<const uint4*>(wreg + rr * STG_RS + cc * 16);
      if (normed) {
        const long grow = grow0 + 32 * i + 8 * q;
        if (!rec && (i | q)) load_cs(grow % T, cv, sv);
        const uint4 oth = *reinterpret_cast<const uint4*>(preg + rr * STG_RS + cc * 16);
        const float rs = rsqrtf((part[wave * 32 + rr] + part[(wave ^ 1) * 32 + rr]) * (1.f / 128.f) + 1e-6f);
        const uint32_t ow[4] = {val.x, val.y, val.z, val.w};
        const uint32_t pw[4] = {oth.x, oth.y, oth.z, oth.w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = rs * ((e & 1) ? bf_hi(ow[e >> 1]) : bf_lo(ow[e >> 1]));  // this wave's dim
          const float b = rs * ((e & 1) ? bf_hi(pw[e >> 1]) : bf_lo(pw[e >> 1]));  // the pair's other dim
          // pair (x1, x2) = (dim j, dim j + 64): (x1 c - x2 s, x1 s + x2 c)
          y[e] = lo_half ? a * cv[e] - b * sv[e] : b * sv[e] + a * cv[e];
        }
        val = make_uint4(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]), pack_bf2(y[4], y[5]), pack_bf2(y[6], y[7]));
        if (lo_half && cc == 0 && (FULL || 32 * i + rr < rows_left))
          p.qk_rstd[grow * p.qk_heads + head] = rs;
        if (rec) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float cn = cv[e] * c8[e] - sv[e] * s8[e];
            sv[e] = sv[e] * c8[e] + cv[e] * s8[e];
            cv[e] = cn;
          }
        }
      }
      uint16_t* dst = cb + (long)(32 * i + rr) * ldc + cc * 8;
      if (FULL || (32 * i + rr < rows_left && cc * 8 + 8 <= cols_left)) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else if (32 * i + rr < rows_left && cc * 8 + 4 <= cols_left) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(val.x, val.y);
      }
    }
  }
  // The caller's barrier (before the next tile's direct loads) ends the last
  // block's reads.
}
static_assert(2 * (8 * 32 * STG_RS + 8 * 32 * 4) <= NST * STAGE_BYTES, "QK-norm staging must fit in the ring");

// The same staging for the epilogues that read an operand: the fp32 residual
// add (read-modify-write of fp32 C), the ReLU^2 backward (reads bf16 D) and
// the Newton-Schulz updates (first iteration: reads fp32 X, writes fp32 X and
// its fp16 copy; later ones: fp16 X in, fp16 X out; the last iteration's fp32
// output takes the register path). Per 32-row block: the block's inputs (old C, or D) are read
// row-contiguous into the wave's LDS region; each lane combines its
// accumulators with the inputs at its own positions, in place; the results
// leave row-contiguous (256-byte fp32 or 128-byte bf16 row segments). The
// next block's inputs are loaded while the current block is processed.
// Global accesses go through buffer instructions on the wave's tile base:
// one per-lane 32-bit offset for the whole epilogue, the row-group offset
// in a scalar register. fp32 rows are padded to 272 bytes in LDS.
template <int E>
constexpr bool lds_epi_io() {
  // (Plain fp32 outputs and split-K partials measured no faster staged: their
  // GEMMs have long K, and the register path already writes 16 bytes a lane.)
  return E == EPI_F32_ACC || E == EPI_DRELU2_BF16 || E == EPI_NS_UPDATE || E == EPI_H_NS_UPDATE;
}
constexpr int STG_RS_F = 272;  // padded row stride of an fp32 staging block (bytes)
static_assert(8 * 32 * STG_RS_F <= NST * STAGE_BYTES, "staging regions must fit in the ring");

// Orders this wave's LDS accesses as written: lanes read what other lanes of
// the wave wrote, which the compiler cannot see.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Raw buffer resource over a wave-uniform base (range 2 GiB; gfx9 dword 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           0x7fffffff, 0x00020000);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// A buffer store of more than 8 bytes reads its data VGPRs after it issues;
// a VALU write to those VGPRs right behind it can reach some lanes first (fp32
// rows were stored holding the fp16 bits that the following conversion wrote
// into the same registers). The compiler inserts the wait states only for
// stores whose soffset is not a register, and the staged epilogues pass the
// row offset in an SGPR, so a store whose registers a VALU may reuse is
// fenced off alone and followed by the wait written out here.
__device__ __forceinline__ void wide_store_wait() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

template <int E, bool FULL>
__device__ __forceinline__ void store_tile_lds_io(const GemmArgs& p, const f32x16 (&acc)[4][2], int bi,
                                                  int m0, int n0, int row_off, int col_off, int lane, int wave,
                                                  char* smem) {
  const int rows_left = p.M - (m0 + row_off), cols_left = p.N - (n0 + col_off);
  char* wreg = smem + wave * (32 * STG_RS_F);
  const int r = lane & 31, hl = lane >> 5;
  const int ldc = (int)p.ldc;
  const long cbase = (long)bi * p.sc + (long)(m0 + row_off) * p.ldc + (n0 + col_off);
  if constexpr (E == EPI_DRELU2_BF16 || E == EPI_H_NS_UPDATE) {
    // 16-bit D in, 16-bit C out (ReLU^2 backward: bf16; Newton-Schulz update
    // v = alpha acc + beta X: fp16). 8 lanes per 128-byte segment, 8 rows per
    // instruction.
    constexpr int RS = STG_RS;
    const int ldd = (int)p.ldd;
    const float alpha = p.alpha, beta = p.beta;
    const auto drs =
        wave_rsrc(reinterpret_cast<const uint16_t*>(p.d) + (long)bi * p.sd + (long)(m0 + row_off) * p.ldd + (n0 + col_off));
    const auto crs = wave_rsrc(reinterpret_cast<uint16_t*>(p.c) + cbase);
    const int rq = lane >> 3, cc = lane & 7;
    const int dvo = (rq * ldd + cc * 8) * 2, cvo = (rq * ldc + cc * 8) * 2;
    u32x4_t din[4];
    auto load_d = [&](int i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * i + 8 * q + rq;
        const int so = (32 * i + 8 * q) * ldd * 2;
        if (FULL || (row < rows_left && cc * 8 + 8 <= cols_left)) {
          din[q] = __builtin_amdgcn_raw_buffer_load_b128(drs, dvo, so, 0);
        } else if (row < rows_left && cc * 8 + 4 <= cols_left) {
          const u32x2_t u = __builtin_amdgcn_raw_buffer_load_b64(drs, dvo, so, 0);
          din[q] = u32x4_t{u.x, u.y, 0u, 0u};
        } else {
          din[q] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    load_d(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4_t*>(wreg + (8 * q + rq) * RS + cc * 16) = din[q];
      if (i + 1 < 4) load_d(i + 1);
      wave_lds_order();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          char* a = wreg + r * RS + (32 * j + 8 * g + 4 * hl) * 2;
          const uint2 h = *reinterpret_cast<const uint2*>(a);
          const f32x16& v = acc[i][j];
          if constexpr (E == EPI_DRELU2_BF16) {
            // d relu(u)^2 / du = 2 relu(u) = 2 sqrt(h), h = relu(u)^2 as stored.
            *reinterpret_cast<uint2*>(a) =
                make_uint2(pack_bf2(2.f * v[4 * g] * __builtin_amdgcn_sqrtf(bf_lo(h.x)),
                                    2.f * v[4 * g + 1] * __builtin_amdgcn_sqrtf(bf_hi(h.x))),
                           pack_bf2(2.f * v[4 * g + 2] * __builtin_amdgcn_sqrtf(bf_lo(h.y)),
                                    2.f * v[4 * g + 3] * __builtin_amdgcn_sqrtf(bf_hi(h.y))));
          } else {
            *reinterpret_cast<uint2*>(a) =
                make_uint2(pack_h2(alpha * v[4 * g] + beta * h_lo(h.x), alpha * v[4 * g + 1] + beta * h_hi(h.x)),
                           pack_h2(alpha * v[4 * g + 2] + beta * h_lo(h.y), alpha * v[4 * g + 3] + beta * h_hi(h.y)));
          }
        }
      wave_lds_order();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * i + 8 * q + rq;
        const int so = (32 * i + 8 * q) * ldc * 2;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(wreg + (8 * q + rq) * RS + cc * 16);
        if (FULL || (row < rows_left && cc * 8 + 8 <= cols_left)) {
          __builtin_amdgcn_raw_buffer_store_b128(val, crs, cvo, so, 0);
        } else if (row < rows_left && cc * 8 + 4 <= cols_left) {
          __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{val.x, val.y}, crs, cvo, so, 0);
        }
      }
      wave_lds_order();
    }
  } else if constexpr (E == EPI_NS_UPDATE) {
    // v = alpha acc + beta D; fp32 v to C3 (stride ldd), fp16 v to C (stride
    // ldc). fp32 rows: 16 lanes per 256-byte segment.
    constexpr int RS = STG_RS_F;
    const int ldd = (int)p.ldd;
    const long dbase = (long)bi * p.sd + (long)(m0 + row_off) * p.ldd + (n0 + col_off);
    const auto drs = wave_rsrc(reinterpret_cast<const float*>(p.d) + dbase);
    // C3 may be null: then only the fp16 copy is written (a run with more
    // iterations reads X from it).
    const bool with_x32 = p.c3 != nullptr;
    const auto x3 = wave_rsrc(reinterpret_cast<float*>(p.c3) + dbase);
    const auto hrs = wave_rsrc(reinterpret_cast<uint16_t*>(p.c) + cbase);
    const float alpha = p.alpha, beta = p.beta;
    const int rq = lane >> 4, cc = lane & 15;
    const int dvo = (rq * ldd + cc * 4) * 4, hvo = (rq * ldc + cc * 4) * 2;
    auto ok = [&](int row) { return FULL || (row < rows_left && cc * 4 < cols_left); };
    u32x4_t din[8];
    auto load_d = [&](int i) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 32 * i + 4 * q + rq;
        din[q] = ok(row) ? __builtin_amdgcn_raw_buffer_load_b128(drs, dvo, (32 * i + 4 * q) * ldd * 4, 0)
                         : u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    load_d(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4_t*>(wreg + (4 * q + rq) * RS + cc * 16) = din[q];
      if (i + 1 < 4) load_d(i + 1);
      wave_lds_order();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float* a = reinterpret_cast<float*>(wreg + r * RS + (32 * j + 8 * g + 4 * hl) * 4);
          const f32x16& v = acc[i][j];
          const float4 x = *reinterpret_cast<const float4*>(a);
          *reinterpret_cast<float4*>(a) =
              make_float4(alpha * v[4 * g] + beta * x.x, alpha * v[4 * g + 1] + beta * x.y,
                          alpha * v[4 * g + 2] + beta * x.z, alpha * v[4 * g + 3] + beta * x.w);
        }
      wave_lds_order();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 32 * i + 4 * q + rq;
        const float4 w = *reinterpret_cast<const float4*>(wreg + (4 * q + rq) * RS + cc * 16);
        if (ok(row)) {
          const u32x2_t h = u32x2_t{pack_h2(w.x, w.y), pack_h2(w.z, w.w)};
          if (with_x32) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), x3, dvo,
                                                   (32 * i + 4 * q) * ldd * 4, 0);
            wide_store_wait();
          }
          __builtin_amdgcn_raw_buffer_store_b64(h, hrs, hvo, (32 * i + 4 * q) * ldc * 2, 0);
        }
      }
      wave_lds_order();
    }
  } else {
    // fp32 rows: 16 lanes per 256-byte segment, 4 rows per instruction.
    constexpr int RS = STG_RS_F;
    const auto crs = wave_rsrc(reinterpret_cast<float*>(p.c) + cbase);
    const float alpha = p.alpha;
    const float beta = p.beta;
    const bool reads = (E == EPI_F32_ACC) && beta != 0.f;
    const int rq = lane >> 4, cc = lane & 15;
    const int cvo = (rq * ldc + cc * 4) * 4;
    auto ok = [&](int row) { return FULL || (row < rows_left && cc * 4 < cols_left); };
    u32x4_t cin[8];
    auto load_c = [&](int i) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 32 * i + 4 * q + rq;
        cin[q] = ok(row) ? __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, (32 * i + 4 * q) * ldc * 4, 0)
                         : u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    if constexpr (E == EPI_F32_ACC) {
      if (reads) load_c(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (E == EPI_F32_ACC) {
        if (reads) {
#pragma unroll
          for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4_t*>(wreg + (4 * q + rq) * RS + cc * 16) = cin[q];
          if (i + 1 < 4) load_c(i + 1);
        }
      }
      wave_lds_order();
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float* a = reinterpret_cast<float*>(wreg + r * RS + (32 * j + 8 * g + 4 * hl) * 4);
          const f32x16& v = acc[i][j];
          float4 o = make_float4(alpha * v[4 * g], alpha * v[4 * g + 1], alpha * v[4 * g + 2], alpha * v[4 * g + 3]);
          if constexpr (E == EPI_F32_ACC) {
            if (reads) {
              const float4 c = *reinterpret_cast<const float4*>(a);
              o = make_float4(beta * c.x + o.x, beta * c.y + o.y, beta * c.z + o.z, beta * c.w + o.w);
            }
          }
          *reinterpret_cast<float4*>(a) = o;
        }
      wave_lds_order();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 32 * i + 4 * q + rq;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(wreg + (4 * q + rq) * RS + cc * 16);
        if (ok(row)) __builtin_amdgcn_raw_buffer_store_b128(val, crs, cvo, (32 * i + 4 * q) * ldc * 4, 0);
      }
      wave_lds_order();
    }
  }
}

template <bool AK, bool BK_, int EPI>
__global__ void __launch_bounds__(NTHR, 1) gemm_bf16_kernel(const GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  int tm, tn, z;
  tile_coords(p, tm, tn, z);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int bi = z / p.splits;
  const int si = z - bi * p.splits;
  const int kbeg = si * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  const int kiters = (kend - kbeg + BKD - 1) / BKD;
  const int nk = kiters;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto stage_a = [&](int it) { return smem + (it % NST) * STAGE_BYTES; };
  // LDS byte address of the ring, taken once; direct-load destinations are
  // formed from it with scalar arithmetic only.
  const uint32_t lds0 = lds_addr(smem);
  auto stage_l = [&](int it) { return lds0 + (uint32_t)((it % NST) * STAGE_BYTES); };

  // A k-block inside both operands (every tile of the d20 shapes) loads with
  // a scalar base and per-lane offsets computed once; edge tiles and a
  // partial last k-block take the clamping path.
  uint32_t offa[4], offb[4];
  block_offsets<AK>(p.lda, wave, lane, offa);
  block_offsets<BK_>(p.ldb, wave, lane, offb);
  const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
  struct KBlk {
    const uint16_t* a;  // operand bases of the block's batch
    const uint16_t* b;
    const uint16_t* sa;  // scalar bases of the block (fast path)
    const uint16_t* sb;
    int k0;
    bool fast;
  };
  auto kblk = [&](int it) {
    KBlk kb;
    kb.k0 = kbeg + it * BKD;
    kb.a = p.a + (long)bi * p.sa;
    kb.b = p.b + (long)bi * p.sb;
    kb.sa = AK ? kb.a + (long)m0 * p.lda + kb.k0 : kb.a + (long)kb.k0 * p.lda + m0;
    kb.sb = BK_ ? kb.b + (long)n0 * p.ldb + kb.k0 : kb.b + (long)kb.k0 * p.ldb + n0;
    kb.fast = interior && (kb.k0 + BKD <= kend);
    return kb;
  };
  // Load q (0..3: A blocks, 4..7: B blocks) of this wave's share of kb into
  // the stage at lds_st (kb.fast is wave-uniform: a scalar branch).
  auto load_q = [&](const KBlk& kb, uint32_t lds_st, int q) {
    if (q < 4) {
      if (kb.fast)
        dma16_sv(kb.sa, offa[q], lds_st + (wave * 4 + q) * 1024);
      else
        issue_one<AK>(kb.a, p.lda, m0, p.M, kb.k0, kend, lds_st, wave * 4 + q, lane);
    } else {
      if (kb.fast)
        dma16_sv(kb.sb, offb[q - 4], lds_st + OP_BYTES + (wave * 4 + q - 4) * 1024);
      else
        issue_one<BK_>(kb.b, p.ldb, n0, p.N, kb.k0, kend, lds_st + OP_BYTES, wave * 4 + q - 4, lane);
    }
  };
  auto issue = [&](int it) {
    const KBlk kb = kblk(it);
#pragma unroll
    for (int q = 0; q < 8; ++q) load_q(kb, stage_l(it), q);
  };

  struct Frags {
    bf16x8 a[4], b[4];
  };
  auto read_frags = [&](int it, int ks, Frags& f) {
    const char* st = stage_a(it);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = read_frag<AK>(st, wm * 128 + i * 32, ks, lane);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.b[j] = read_frag<BK_>(st + OP_BYTES, wn * 128 + j * 32, ks, lane);
    }
  };
  auto mfma_step = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mfma16<EPI>(f.b[j], f.a[i], acc[i][j]);
  };

  // Interleave a k-step's 16 MFMAs with the NR LDS reads of the next
  // fragments (NR = 8 / 12 / 16 by operand layout), so that fewer than 16
  // reads are ever outstanding (the LDS counter tracks 15) and their latency
  // hides under the MFMAs.
  constexpr int NR = (AK ? 4 : 8) + (BK_ ? 4 : 8);
  auto interleave = [&]() {
    // mask 0x100: one DS read; mask 0x008: MFMAs.
    if constexpr (NR == 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    } else if constexpr (NR == 12) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  };
  // Zero the part of k-block `it` past the end of K (tail block only).
  auto tail_fix = [&](int it) {
    const int seg = it / kiters;
    const int kvalid = kend - (kbeg + (it - seg * kiters) * BKD);
    if (kvalid < BKD) {
      zero_tail<AK>(stage_a(it), kvalid, tid);
      zero_tail<BK_>(stage_a(it) + OP_BYTES, kvalid, tid);
      __syncthreads();
    }
  };
  // Number of k-blocks issued after block j once blocks 0..last are issued.
  auto pending_after = [&](int j, int last) { return max(0, min(nk - 1, last) - j) * 8; };

  // Ring of NST k-blocks, one barrier per iteration, placed mid-iteration:
  //   iteration it: MFMAs of k-step 0 of block it (reads of its k-step 1
  //   interleaved) | wait for block it+1, barrier, issue block it+NST-1 into
  //   the slot of block it-1 | MFMAs of k-step 1 of block it (reads of k-step
  //   0 of block it+1 interleaved).
  // Every read of block it-1 precedes the previous barrier, so its slot is
  // free; block it+1 is visible to all waves after this barrier.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s);
  Frags f0, f1;
  if (nk > 0) {
    ring_sync(pending_after(0, NST - 2));
    tail_fix(0);
    read_frags(0, 0, f0);
  }
  for (int it = 0; it < nk; ++it) {
    read_frags(it, 1, f1);
    mfma_step(f0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < nk) {
      ring_sync(pending_after(it + 1, it + NST - 2));
      tail_fix(it + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase B in 8 chunks: one direct load (4 of A, then 4 of B), one
    // fragment of block it+1 and two MFMAs on k-step 1 of block it per
    // chunk, so the in-order wave never stalls on a burst of loads while the
    // MFMA pipe drains. Past the last block the fragment reads hit a stale
    // slot and are unused.
    const bool more = it + NST - 1 < nk;
    const KBlk kb = kblk(more ? it + NST - 1 : 0);
    const uint32_t nst = stage_l(it + NST - 1);
    const char* rst = stage_a(it + 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (more) load_q(kb, nst, q);
      if (q < 4) {
        f0.a[q] = read_frag<AK>(rst, wm * 128 + q * 32, 0, lane);
      } else {
        f0.b[q - 4] = read_frag<BK_>(rst + OP_BYTES, wn * 128 + (q - 4) * 32, 0, lane);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * q + u;
        acc[t >> 2][t & 3] = mfma16<EPI>(f1.b[t & 3], f1.a[t >> 2], acc[t >> 2][t & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  store_tile<EPI, 4>(p, acc, bi, si, m0, n0, wm * 128, wn * 128, lane);
}

// ---------------------------------------------------------------------------
// Ping-pong variant: 8 waves in two groups of 4 (one wave of each group per
// SIMD). Group g owns rows 128 g .. 128 g + 127 of the 256 x 256 tile; wave
// w of a group owns 64 columns (4 x 2 MFMA tiles, 128 accumulators). The
// groups alternate phases: while one group runs a burst of 16 MFMAs on
// fragments already in registers, the other reads its fragments of the next
// k-block from LDS and issues its half of a later k-block's direct loads
// (group 0 the A operand, group 1 the B operand). Each SIMD thus always has
// one wave issuing only MFMAs and one wave issuing only memory instructions.
//   phase 2j:   group 0 reads k-block j (+ loads A of j+2); group 1 computes j-1
//   phase 2j+1: group 0 computes j;  group 1 reads j (+ loads B of j+2)
// A barrier closes every phase after vmcnt(4) (vmcnt(0) once no further
// batch follows): each wave keeps only its most recent batch of 4 direct
// loads in flight, so a k-block is complete before its first read, and its
// slot (k-block j-2 in a 4-stage ring) was last read two phases earlier.
// K (and each split's k range) must be a multiple of 32: there is no tail
// k-block.
// A wave's four direct loads of a k-block go out in one asm block from one
// scalar pointer that advances by a k-block per issue (no per-load address
// arithmetic, division or branch in the loop); only edge tiles take the
// clamped per-load path.
// The kernel is persistent: one workgroup per CU walks the (batch / split,
// tile) work items with stride gridDim.x, so a tile's epilogue stores drain
// while the next tile's first k-blocks load, instead of each workgroup
// draining its stores before the next one may start. Epilogues that write
// bf16 without reading an input go through LDS (store_tile_lds) so that
// every store instruction writes whole 128-byte row segments.
// ---------------------------------------------------------------------------
constexpr int PP_THR = 512;

template <bool AK, bool BK_, int EPI>
__global__ void __launch_bounds__(PP_THR, 1) gemm_pp_kernel(const GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int w4 = wave & 3;

  // Work items: (batch / split, tile) pairs, walked with stride gridDim.x.
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int per = p.sym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  const int total = per * p.batch * p.splits;

  const uint32_t lds0 = lds_addr(smem);
  auto stage_a = [&](int it) { return smem + (it % NST) * STAGE_BYTES; };
  auto stage_l = [&](int it) { return lds0 + (uint32_t)((it % NST) * STAGE_BYTES); };

  uint32_t off[4];
  if (grp == 0)
    block_offsets<AK>(p.lda, w4, lane, off);
  else
    block_offsets<BK_>(p.ldb, w4, lane, off);
  const bool opA = grp == 0;
  const long ld = opA ? p.lda : p.ldb;
  const bool kmaj = opA ? AK : BK_;
  const long kstep = kmaj ? (long)BKD : (long)BKD * ld;
  const uint32_t op_off = opA ? 0u : (uint32_t)OP_BYTES;

  // Per-tile state.
  int m0, n0, bi, si, kbeg, kend, kiters, nk;
  bool interior;
  const uint16_t* nxt;
  int nxt_k;
  auto tile_ptr = [&]() {
    const int rc0 = opA ? m0 : n0;
    const uint16_t* b = opA ? p.a + (long)bi * p.sa : p.b + (long)bi * p.sb;
    return b + (kmaj ? (long)rc0 * ld + kbeg : (long)kbeg * ld + rc0);
  };
  auto setup = [&](int lin) {
    int tm, tn, z;
    tile_coords_lin(p, lin, per, total, tiles_m, tiles_n, tm, tn, z);
    m0 = tm * BM;
    n0 = tn * BN;
    bi = z / p.splits;
    si = z - bi * p.splits;
    kbeg = si * p.k_chunk;
    kend = min(p.K, kbeg + p.k_chunk);
    kiters = (kend - kbeg + BKD - 1) / BKD;
    nk = kiters;
    interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    nxt = tile_ptr();
    nxt_k = 0;
  };

  // This wave's 4 blocks of its group's operand of k-block it (the next one
  // in issue order).
  // (INT: the tile is interior, a compile-time tag inside the k-loop.)
  auto dma_part_t = [&](int it, auto int_tag) __attribute__((always_inline)) {
    constexpr bool INT = decltype(int_tag)::value;
    const uint32_t st = stage_l(it) + op_off;
    if constexpr (INT) {
      dma16_sv4(nxt, off, st + (uint32_t)(w4 * 4 * 1024));
    } else {
      const int k0 = kbeg + nxt_k * BKD;
      if (opA) {
        const uint16_t* a = p.a + (long)bi * p.sa;
#pragma unroll
        for (int q = 0; q < 4; ++q) issue_one<AK>(a, p.lda, m0, p.M, k0, kend, st, w4 * 4 + q, lane);
      } else {
        const uint16_t* b = p.b + (long)bi * p.sb;
#pragma unroll
        for (int q = 0; q < 4; ++q) issue_one<BK_>(b, p.ldb, n0, p.N, k0, kend, st, w4 * 4 + q, lane);
      }
    }
    ++nxt_k;
    nxt += kstep;
  };
  auto dma_part = [&](int it) __attribute__((always_inline)) {
    if (interior)
      dma_part_t(it, std::true_type{});
    else
      dma_part_t(it, std::false_type{});
  };

  f32x16 acc[4][2];
  bf16x8 fa[2][4], fb[2][2];
  auto load_frags = [&](int it) {
    const char* st = stage_a(it);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[ks][i] = read_frag<AK>(st, 128 * grp + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[ks][j] = read_frag<BK_>(st + OP_BYTES, 64 * w4 + 32 * j, ks, lane);
    }
  };
  auto compute_ks = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = mfma16<EPI>(fb[ks][j], fa[ks][i], acc[i][j]);
  };
  auto compute = [&]() {
    compute_ks(0);
    compute_ks(1);
  };
  auto wait_bar = [&](bool more) {
    __builtin_amdgcn_sched_barrier(0);
    if (more)
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Barrier that orders LDS accesses only (stores may stay in flight).
  auto lds_bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // The k-loop, with the last two k-blocks (nothing left to load) peeled off
  // and the interior test hoisted, so the loop body has no branch.
  auto run_t = [&](auto int_tag) __attribute__((always_inline)) {
    int j = 0;
#pragma nounroll
    for (; j + 2 < nk; ++j) {
      load_frags(j);
      dma_part_t(j + 2, int_tag);
      wait_bar(true);
      compute();
      wait_bar(true);
    }
#pragma nounroll
    for (; j < nk; ++j) {
      load_frags(j);
      wait_bar(false);
      compute();
      wait_bar(false);
    }
  };
  auto run = [&]() __attribute__((always_inline)) {
    if (interior)
      run_t(std::true_type{});
    else
      run_t(std::false_type{});
  };

  int lin = blockIdx.x;
  if (lin >= total) return;
  setup(lin);
  if (nk > 0) dma_part(0);
  if (nk > 1) dma_part(1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma nounroll
  while (true) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    if (grp == 0) {
      run();
      wait_bar(false);
    } else {
      wait_bar(false);
      run();
    }
    lds_bar();  // every LDS read of this tile is done
    if constexpr (EPI == EPI_QKN_BF16) {
      if (interior)
        store_tile_qkn<true>(p, acc, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
      else
        store_tile_qkn<false>(p, acc, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
    } else if constexpr (lds_epi<EPI>()) {
      if (interior)
        store_tile_lds<EPI, true>(p, acc, bi, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
      else
        store_tile_lds<EPI, false>(p, acc, bi, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
    } else {
      if constexpr (lds_epi_io<EPI>()) {
        if (interior)
          store_tile_lds_io<EPI, true>(p, acc, bi, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
        else
          store_tile_lds_io<EPI, false>(p, acc, bi, m0, n0, 128 * grp, 64 * w4, lane, wave, smem);
      } else {
        store_tile<EPI, 2>(p, acc, bi, si, m0, n0, 128 * grp, 64 * w4, lane);
      }
    }
    const int lin_next = lin + gridDim.x;
    if (lin_next >= total) break;
    lds_bar();  // the epilogue's LDS staging is done before direct loads overwrite it
    lin = lin_next;
    setup(lin);
    if (nk > 0) dma_part(0);
    if (nk > 1) dma_part(1);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

}  // namespace gemm_impl

// Launch one instantiation: one workgroup per 256 x 256 tile and (batch,
// split). The ping-pong kernel needs whole 32-wide k-blocks; otherwise the
// single-group kernel (which zeroes a partial last k-block) runs.
inline bool gemm_pp_ok(const GemmArgs& g) {
  return g.K % gemm_impl::BKD == 0 && (g.splits == 1 || g.k_chunk % gemm_impl::BKD == 0);
}
// Persistent grid of the ping-pong kernel: one workgroup per CU (its LDS
// allows one), each walking work items with stride gridDim.x.
inline unsigned gemm_pp_grid(const dim3& work) {
  const unsigned total = work.x * work.y;
  return total < 256u ? total : 256u;
}
#define GEMM_LAUNCH(AK, BK, EPI)                                                                      \
  do {                                                                                                \
    if (gemm_pp_ok(g))                                                                                \
      hipLaunchKernelGGL((gemm_impl::gemm_pp_kernel<AK, BK, EPI>), dim3(gemm_pp_grid(grid)),              \
                         dim3(gemm_impl::PP_THR), 0, s, g);                                                 \
    else                                                                                              \
      hipLaunchKernelGGL((gemm_impl::gemm_bf16_kernel<AK, BK, EPI>), grid, dim3(gemm_impl::NTHR), 0,     \
                         s, g);                                                                       \
  } while (0)
