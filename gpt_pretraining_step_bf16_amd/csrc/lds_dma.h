// Direct global -> LDS loads and the transposing LDS read of gfx950, shared
// by the GEMM and attention kernels.
#pragma once

#include "common.h"

typedef short v4s __attribute__((ext_vector_type(4)));
#define LDS_V4S(p) ((__attribute__((address_space(3))) v4s*)(p))

// LDS byte address of a pointer into shared memory, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p);
}

// One 16-byte-per-lane direct load: lane l's 16 bytes at gsrc land at LDS
// lds_base + 16 l. Issued from asm so that the compiler does not add a full
// vmcnt(0) drain before every transposing LDS read (it cannot tell which
// LDS bytes a direct load writes); the callers' explicit vmcnt waits and
// barriers order these loads instead. M0 carries the LDS base and is
// restored afterwards. The asm has no output registers.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds_base)
      : "memory");
}

// Same load with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset: lane l's 16 bytes at sbase + voff land at LDS lds_base + 16 l.
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// 4-byte variant: lane l's dword lands at lds_base + 4 l (active lanes only).
__device__ __forceinline__ void dma4(const void* gsrc, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds_base)
      : "memory");
}

// s_waitcnt vmcnt(N) for the immediate N, then s_barrier; both act as
// compiler memory barriers so no LDS access moves across them.
#define VMCNT_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory")

// Four 16-byte-per-lane direct loads from one wave-uniform 64-bit base with
// per-lane byte offsets v[0..3], landing in four consecutive 1 KB LDS blocks
// from lds_base. M0 is saved once and restored once; the s_add_u32 steps
// write SCC, which the clobber list declares.
__device__ __forceinline__ void dma16_sv4(const void* sbase, const uint32_t (&v)[4], uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_add_u32 m0, %6, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_add_u32 m0, %6, 0x800\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_add_u32 m0, %6, 0xc00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(sbase), "s"(lds_base)
      : "memory", "scc");
}
