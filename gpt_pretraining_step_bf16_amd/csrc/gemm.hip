// bf16 MFMA GEMM for gfx950: every dense contraction of the step (QKV, O, MLP
// and head projections forward and backward, weight gradients, Newton-Schulz).
//
// Design
//  * Macro tile 256 x 256 x 64, 256 threads = 4 wave64s in a 2 x 2 grid, each
//    wave owning a 128 x 128 sub-tile as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles
//    (256 fp32 accumulators per lane). A 128 x 128 wave tile keeps LDS reads
//    at 2 x 4 KB per 16 MFMAs, half of what a 128 x 64 tile would need.
//  * Both operands are staged in LDS as [row][k] with k contiguous, 128 B per
//    row, in 16-byte chunks XOR-swizzled by (row ^ row >> 3) & 7 so that the
//    fragment reads (8 consecutive rows, same chunk) and the tile writes hit
//    distinct banks. Two stages (128 KB) double-buffer the K loop; the next
//    stage's global loads are issued before the current stage's MFMAs.
//  * An operand whose K dimension is strided in memory (activations read as
//    [tokens, features] for weight gradients, or weights read along their out
//    dimension) is loaded as 8 x 8 element blocks and transposed in registers
//    before the LDS write, so the LDS layout and the MFMA loop are the same
//    for every operand layout.
//  * The MFMA computes the transposed tile (B fragment as the A input), which
//    leaves each lane holding 4 consecutive output columns: 8-byte bf16 or
//    16-byte fp32 stores in the epilogue.
//  * Workgroup ids are remapped so consecutive tiles run on one XCD (ids are
//    dealt round-robin over the 8 XCDs), then grouped 4 tile-rows at a time so
//    an XCD's tiles share A rows and B columns in its L2.
//  * Up to three K segments with their own operand bases are summed into one
//    accumulator: Newton-Schulz uses it for hi/lo split products.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHR = 256;
constexpr int TILE_CHUNKS = BM * BK / 8;  // 16-byte chunks per operand tile

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7));
}

__device__ __forceinline__ uint32_t sq2(uint32_t w) {
  float lo = bf_lo(w), hi = bf_hi(w);
  return pack_bf2(lo * lo, hi * hi);
}
__device__ __forceinline__ uint4 sq8(uint4 v) {
  return make_uint4(sq2(v.x), sq2(v.y), sq2(v.z), sq2(v.w));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Register-staged operand tile: 8 x 16 B per thread.
template <bool KMAJ>
struct Stage {
  uint4 r[8];

  // KMAJ: element (row, k) at base[row*ld + k]. Thread t owns chunks
  //   row = t/8 + 32 i, k-chunk = t%8.
  // !KMAJ: element (row, k) at base[k*ld + row]. Thread t owns the 8x8 block
  //   rows 8*(t%32)..+7, k 8*(t/32)..+7, loaded as 8 k-rows of 8 rows each.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, long ld, int row0,
                                       int rows, int k0, int kend, int tid) {
    if (KMAJ) {
      const int kc = tid & 7;
      const int kk = k0 + kc * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const int gr = row0 + row;
        if (gr < rows && kk < kend) {
          r[i] = *reinterpret_cast<const uint4*>(base + (long)gr * ld + kk);
        } else {
          r[i] = make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      const int mb = tid & 31;
      const int kb = tid >> 5;
      const int gr = row0 + mb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = k0 + kb * 8 + i;
        if (gr < rows && kk < kend) {
          r[i] = *reinterpret_cast<const uint4*>(base + (long)kk * ld + gr);
        } else {
          r[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void square() {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = sq8(r[i]);
  }

  __device__ __forceinline__ void store(uint4* __restrict__ lds, int tid) const {
    if (KMAJ) {
      const int kc = tid & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) lds[swz((tid >> 3) + 32 * i, kc)] = r[i];
    } else {
      const int mb = tid & 31;
      const int kb = tid >> 5;
      // r[i] holds k-row i of the block (8 rows m = 8mb..8mb+7, 2 per word).
      // Output chunk j holds row m = 8mb + j over k = 0..7.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = word(r[2 * q], j >> 1);
          const uint32_t y = word(r[2 * q + 1], j >> 1);
          w[q] = (j & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
        lds[swz(mb * 8 + j, kb)] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
};

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

// Apply the epilogue to C(m, n..n+3) of batch bi, split si.
__device__ __forceinline__ void epilogue4(const GemmArgs& p, int bi, int si, int m, int n, float4 q) {
  const float v[4] = {q.x, q.y, q.z, q.w};
  const long off = (long)bi * p.sc + (long)m * p.ldc + n;
  const long doff = (long)bi * p.sd + (long)m * p.ldd + n;
  switch (p.epi) {
    case EPI_F32: {
      float* c = reinterpret_cast<float*>(p.c) + off;
      *reinterpret_cast<float4*>(c) =
          make_float4(p.alpha * v[0], p.alpha * v[1], p.alpha * v[2], p.alpha * v[3]);
    } break;
    case EPI_F32_ACC: {
      float* c = reinterpret_cast<float*>(p.c) + off;
      float4 o = *reinterpret_cast<const float4*>(c);
      o.x = p.beta * o.x + p.alpha * v[0];
      o.y = p.beta * o.y + p.alpha * v[1];
      o.z = p.beta * o.z + p.alpha * v[2];
      o.w = p.beta * o.w + p.alpha * v[3];
      *reinterpret_cast<float4*>(c) = o;
    } break;
    case EPI_BF16: {
      uint16_t* c = reinterpret_cast<uint16_t*>(p.c) + off;
      store_bf16x4(c, p.alpha * v[0], p.alpha * v[1], p.alpha * v[2], p.alpha * v[3]);
    } break;
    case EPI_RELU_BF16: {
      uint16_t* c = reinterpret_cast<uint16_t*>(p.c) + off;
      store_bf16x4(c, fmaxf(v[0], 0.f), fmaxf(v[1], 0.f), fmaxf(v[2], 0.f), fmaxf(v[3], 0.f));
    } break;
    case EPI_RESID_BF16: {
      uint16_t* c = reinterpret_cast<uint16_t*>(p.c) + off;
      float o[4];
      load_bf16x4(c, o);
      store_bf16x4(c, o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]);
    } break;
    case EPI_DRELU2_BF16: {
      uint16_t* c = reinterpret_cast<uint16_t*>(p.c) + off;
      float rr[4];
      load_bf16x4(reinterpret_cast<const uint16_t*>(p.d) + doff, rr);
      store_bf16x4(c, 2.f * v[0] * rr[0], 2.f * v[1] * rr[1], 2.f * v[2] * rr[2], 2.f * v[3] * rr[3]);
    } break;
    case EPI_SPLITK: {
      float* c = reinterpret_cast<float*>(p.c) + off + (long)si * p.s_split;
      *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
    } break;
    case EPI_HILO: {
      float w[4] = {p.alpha * v[0], p.alpha * v[1], p.alpha * v[2], p.alpha * v[3]};
      store_hilo4(reinterpret_cast<uint16_t*>(p.c) + off, reinterpret_cast<uint16_t*>(p.c2) + off, w);
    } break;
    case EPI_NS_POLY: {
      float h[4], l[4];
      load_bf16x4(reinterpret_cast<const uint16_t*>(p.d) + doff, h);
      load_bf16x4(reinterpret_cast<const uint16_t*>(p.d2) + doff, l);
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = p.alpha * v[r] + p.beta * (h[r] + l[r]);
      store_hilo4(reinterpret_cast<uint16_t*>(p.c) + off, reinterpret_cast<uint16_t*>(p.c2) + off, w);
    } break;
    case EPI_NS_UPDATE: {
      const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.d) + doff);
      float w[4] = {p.alpha * v[0] + p.beta * x.x, p.alpha * v[1] + p.beta * x.y,
                    p.alpha * v[2] + p.beta * x.z, p.alpha * v[3] + p.beta * x.w};
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.c3) + doff) =
          make_float4(w[0], w[1], w[2], w[3]);
      store_hilo4(reinterpret_cast<uint16_t*>(p.c) + off, reinterpret_cast<uint16_t*>(p.c2) + off, w);
    } break;
    default:
      break;
  }
}

template <bool AK, bool BK_, int SQ>
__global__ void __launch_bounds__(NTHR, 1) gemm_bf16_kernel(const GemmArgs p) {
  __shared__ uint4 lds[2][2][TILE_CHUNKS];  // [stage][A/B]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // Tile coordinates: XCD-aware remap, then grouped order along M.
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int group = bid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = bid - group * GM * tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int z = blockIdx.y;
  const int bi = z / p.splits;
  const int si = z - bi * p.splits;
  const int kbeg = si * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  const int kiters = (kend - kbeg + BK - 1) / BK;
  const int nk = kiters * p.nseg;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Stage<AK> sa;
  Stage<BK_> sb;

  auto load_it = [&](int it) {
    const int seg = it / kiters;
    const int k0 = kbeg + (it - seg * kiters) * BK;
    const uint16_t* a = p.a[seg] + (long)bi * p.sa;
    const uint16_t* b = p.b[seg] + (long)bi * p.sb;
    sa.load(a, p.lda, m0, p.M, k0, kend, tid);
    sb.load(b, p.ldb, n0, p.N, k0, kend, tid);
    if (SQ == 1) sa.square();
    if (SQ == 2) sb.square();
  };

  if (nk > 0) {
    load_it(0);
    sa.store(lds[0][0], tid);
    sb.store(lds[0][1], tid);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int st = it & 1;
    if (it + 1 < nk) load_it(it + 1);
    const uint4* la = lds[st][0];
    const uint4* lb = lds[st][1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      bf16x8 af[4], bfv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = as_bf16x8(la[swz(wm * 128 + i * 32 + (lane & 31), ch)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfv[j] = as_bf16x8(lb[swz(wn * 128 + j * 32 + (lane & 31), ch)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfv[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) {
      sa.store(lds[st ^ 1][0], tid);
      sb.store(lds[st ^ 1][1], tid);
    }
    __syncthreads();
  }

  // Epilogue, in 4 passes through LDS (the operand stages are free now).
  // Pass i: every wave dumps acc[i][*] (rows wm*128 + i*32 + 0..31 of the
  // tile, its 128 columns) into a [64][256 + 4] fp32 slab; then each wave
  // owns whole slab rows and applies the epilogue to 4 consecutive columns
  // per lane, so global loads and stores are row-contiguous.
  // acc[i][j][4g + r] is C(m, n) with m = wm*128 + i*32 + lane%32 and
  // n = wn*128 + j*32 + 8g + 4*(lane/32) + r (tile-relative).
  constexpr int SLAB_LD = BN + 4;
  float* slab = reinterpret_cast<float*>(&lds[0][0][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wm * 32 + (lane & 31);
        const int col = wn * 128 + j * 32 + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(slab + row * SLAB_LD + col) =
            make_float4(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]);
      }
    __syncthreads();
    for (int rr = wave; rr < 64; rr += 4) {
      const int m = m0 + (rr >> 5) * 128 + i * 32 + (rr & 31);
      const int n = n0 + lane * 4;
      if (m < p.M && n < p.N) {
        const float4 q = *reinterpret_cast<const float4*>(slab + rr * SLAB_LD + lane * 4);
        epilogue4(p, bi, si, m, n, q);
      }
    }
    __syncthreads();
  }
}

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
  g.nseg = 1;
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
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, g.batch * g.splits);
  dim3 block(NTHR);
  const int key = (g.a_kmajor ? 1 : 0) | (g.b_kmajor ? 2 : 0);
  if (g.square == 1 && key == 3) {
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, 1>), grid, block, 0, s, g);
  } else if (g.square == 2 && key == 0) {
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, 2>), grid, block, 0, s, g);
  } else if (g.square != 0) {
    return hipErrorInvalidValue;
  } else if (key == 3) {
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, 0>), grid, block, 0, s, g);
  } else if (key == 1) {
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, 0>), grid, block, 0, s, g);
  } else if (key == 0) {
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, 0>), grid, block, 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<false, true, 0>), grid, block, 0, s, g);
  }
  return hipGetLastError();
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
