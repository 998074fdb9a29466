// Launchers of the flash-attention kernels (defined in attention.hip).
// qkv is [B*T, (H + 2*Hkv)*128] bf16 (q heads, k heads, v heads); Hkv divides
// H (grouped-query attention when Hkv < H). window: key j is visible to query
// i when i - window <= j <= i; a negative window (or one of at least T) is the
// plain causal mask. lse2 and delta are [B, H, T].
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

hipError_t launch_attention_fwd_window(const uint16_t* qkv, uint16_t* o, float* lse2, int B, int T, int H,
                                       int Hkv, int window, hipStream_t s);
// With rstd_qk ([B*T, H + Hkv], the forward's QK-norm scales) and cs (the
// RoPE (cos, sin) table, [T][64] pairs), q and k in qkv are taken as
// rope(norm(x)) and the q, k parts of dqkv are gradients w.r.t. x (the QK-norm
// + RoPE backward is applied in the kernels' epilogues); null: w.r.t. q, k.
hipError_t launch_attention_bwd_window(const uint16_t* qkv, const uint16_t* o, const float* lse2,
                                       const uint16_t* dO, uint16_t* dqkv, float* delta, int B, int T, int H,
                                       int Hkv, int window, hipStream_t s, const float* rstd_qk = nullptr,
                                       const float* cs = nullptr);
