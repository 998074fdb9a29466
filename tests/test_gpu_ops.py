"""Step-level parity on the GPU: each HIP step against the oracle / its definition.

Inputs are seeded and rounded to bf16 before both sides see them, so the only
differences are the kernels' fp32 accumulation order and output rounding.
"""
import numpy as np
import pytest

from gpu_util import bf16_bits, bf16_round, bits_to_f32, dev, log, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpt_pretraining_step_bf16_amd import binding, synthetic as syn  # noqa: E402


def _rand_bf16(rng, shape, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * scale
    return bf16_bits(x).reshape(shape), bf16_round(x).reshape(shape).astype(np.float64)


# ----------------------------------------------------------------------------
# GEMM: every operand layout, several epilogues, ragged M / N / K tails
# ----------------------------------------------------------------------------
# K = 328 has a partial last k-block (single-group kernel); K = 320 has whole
# k-blocks (ping-pong kernel, with ragged M / N edge tiles).
@pytest.mark.parametrize("K", [328, 320])
@pytest.mark.parametrize("a_kmajor,b_kmajor", [(1, 1), (1, 0), (0, 1), (0, 0)])
def test_gemm_layouts_fp32_out(a_kmajor, b_kmajor, K):
    M, N, batch = 520, 264, 2
    log(f"gemm layouts a_kmajor={a_kmajor} b_kmajor={b_kmajor} M={M} N={N} K={K}")
    rng = np.random.default_rng(10 + 2 * a_kmajor + b_kmajor)
    Ab, Af = _rand_bf16(rng, (batch, M, K))
    Bb, Bf = _rand_bf16(rng, (batch, N, K))
    # Store each operand in the requested layout.
    A_store = Ab if a_kmajor else np.ascontiguousarray(Ab.transpose(0, 2, 1))
    B_store = Bb if b_kmajor else np.ascontiguousarray(Bb.transpose(0, 2, 1))
    lda = K if a_kmajor else M
    ldb = K if b_kmajor else N
    A = dev(torch, A_store)
    B = dev(torch, B_store)
    C = torch.zeros(batch, M, N, dtype=torch.float32, device="cuda")
    binding.op_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, N, binding.OUT_F32, batch=batch,
                    stride_a=M * K, stride_b=N * K, stride_c=M * N)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    ref = np.matmul(Af, Bf.transpose(0, 2, 1))
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 2e-6, err


# The smallest shapes the contract allows (multiples of 8 along the
# K-contiguous dimensions, N a multiple of 4): a single partial tile, K below
# one k-block or off the 32 grid (single-group kernel) or on it (ping-pong).
@pytest.mark.parametrize("M,N,K", [(8, 8, 8), (24, 16, 40), (40, 8, 1000), (8, 8, 64)])
@pytest.mark.parametrize("a_kmajor,b_kmajor", [(1, 1), (1, 0), (0, 1), (0, 0)])
def test_gemm_tiny_shapes(a_kmajor, b_kmajor, M, N, K):
    batch = 3
    rng = np.random.default_rng(M + N + K + 2 * a_kmajor + b_kmajor)
    Ab, Af = _rand_bf16(rng, (batch, M, K))
    Bb, Bf = _rand_bf16(rng, (batch, N, K))
    A_store = Ab if a_kmajor else np.ascontiguousarray(Ab.transpose(0, 2, 1))
    B_store = Bb if b_kmajor else np.ascontiguousarray(Bb.transpose(0, 2, 1))
    C = torch.zeros(batch, M, N, dtype=torch.float32, device="cuda")
    binding.op_gemm(M, N, K, dev(torch, A_store), K if a_kmajor else M, a_kmajor, dev(torch, B_store),
                    K if b_kmajor else N, b_kmajor, C, N, binding.OUT_F32, batch=batch, stride_a=M * K,
                    stride_b=N * K, stride_c=M * N)
    torch.cuda.synchronize()
    ref = np.matmul(Af, Bf.transpose(0, 2, 1))
    err = np.abs(C.cpu().numpy() - ref).max() / np.abs(ref).max()
    assert err < 2e-6, err


# bf16 outputs go through the LDS-staged epilogue (interior tiles, and edge
# tiles with a column count that is a multiple of 8 or only of 4), in a
# persistent launch that walks several tiles per workgroup.
# The layouts with bf16 epilogues: both operands K-major, and K-major A with a
# K-strided B (N = 260 needs a K-major B: K-strided rows must be 16-byte aligned).
@pytest.mark.parametrize("a_kmajor,b_kmajor,N", [(1, 1, 264), (1, 1, 260), (1, 0, 264)])
def test_gemm_layouts_bf16_out(a_kmajor, b_kmajor, N):
    M, K = 776, 320
    log(f"gemm bf16 out a_kmajor={a_kmajor} b_kmajor={b_kmajor} M={M} N={N} K={K}")
    rng = np.random.default_rng(40 + 2 * a_kmajor + b_kmajor + N)
    Ab, Af = _rand_bf16(rng, (M, K))
    Bb, Bf = _rand_bf16(rng, (N, K))
    A = dev(torch, Ab if a_kmajor else np.ascontiguousarray(Ab.T))
    B = dev(torch, Bb if b_kmajor else np.ascontiguousarray(Bb.T))
    C = torch.full((M, N), 0x7FC0, dtype=torch.int16, device="cuda")  # NaN fill: unwritten shows
    binding.op_gemm(M, N, K, A, K if a_kmajor else M, a_kmajor, B, K if b_kmajor else N, b_kmajor, C, N,
                    binding.OUT_BF16)
    torch.cuda.synchronize()
    got = bits_to_f32(C.cpu().numpy()).reshape(M, N)
    ref = Af @ Bf.T
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)


@pytest.mark.parametrize("a_kmajor,b_kmajor,mode", [(1, 1, "bf16"), (1, 1, "f32_acc"), (1, 1, "relu"),
                                                     (1, 0, "f32"), (0, 0, "f32"), (0, 1, "f32")])
def test_gemm_persistent_many_tiles(a_kmajor, b_kmajor, mode):
    """More 256 x 256 tiles (9 x 9 x 4 = 324, ragged last row and column)
    than workgroups (256), so workgroups walk several tiles, interior and
    edge, and each tile's epilogue runs while the next tile's first k-blocks
    load."""
    M = N = 2056
    K, batch = 320, 4
    log(f"gemm persistent a_kmajor={a_kmajor} b_kmajor={b_kmajor} mode={mode}")
    rng = np.random.default_rng(70 + 2 * a_kmajor + b_kmajor)
    Ab, Af = _rand_bf16(rng, (batch, M, K))
    Bb, Bf = _rand_bf16(rng, (batch, N, K))
    A = dev(torch, Ab if a_kmajor else np.ascontiguousarray(Ab.transpose(0, 2, 1)))
    B = dev(torch, Bb if b_kmajor else np.ascontiguousarray(Bb.transpose(0, 2, 1)))
    lda, ldb = (K if a_kmajor else M), (K if b_kmajor else N)
    ref = np.matmul(Af, Bf.transpose(0, 2, 1))
    if mode in ("bf16", "relu"):
        C = torch.full((batch, M, N), 0x7FC0, dtype=torch.int16, device="cuda")
        out = binding.OUT_BF16 if mode == "bf16" else binding.OUT_RELU_BF16
        binding.op_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, N, out, batch=batch,
                        stride_a=M * K, stride_b=N * K, stride_c=M * N)
        torch.cuda.synchronize()
        got = bits_to_f32(C.cpu().numpy()).reshape(batch, M, N)
        want = ref if mode == "bf16" else np.maximum(ref, 0.0)
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
    else:
        base = rng.standard_normal((batch, M, N)).astype(np.float32) if mode == "f32_acc" else None
        C = dev(torch, base) if base is not None else torch.full((batch, M, N), float("nan"), device="cuda")
        out = binding.OUT_F32_ACC if mode == "f32_acc" else binding.OUT_F32
        binding.op_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, N, out, batch=batch,
                        stride_a=M * K, stride_b=N * K, stride_c=M * N)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        want = ref if base is None else base + ref
        assert np.all(np.isfinite(got))
        assert np.abs(got - want).max() / np.abs(ref).max() < 2e-6


def test_gemm_epilogues():
    M, N, K = 300, 392, 256
    log(f"gemm epilogues M={M} N={N} K={K}")
    rng = np.random.default_rng(3)
    Ab, Af = _rand_bf16(rng, (M, K))
    Bb, Bf = _rand_bf16(rng, (N, K))
    ref = Af @ Bf.T
    A, B = dev(torch, Ab), dev(torch, Bb)
    # bf16 store
    C = torch.zeros(M, N, dtype=torch.int16, device="cuda")
    binding.op_gemm(M, N, K, A, K, 1, B, K, 1, C, N, binding.OUT_BF16)
    got = bits_to_f32(C.cpu().numpy()).reshape(M, N)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
    # relu
    binding.op_gemm(M, N, K, A, K, 1, B, K, 1, C, N, binding.OUT_RELU_BF16)
    got = bits_to_f32(C.cpu().numpy()).reshape(M, N)
    assert np.all(got >= 0) and np.all(np.abs(got - np.maximum(ref, 0)) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
    # bf16 residual add in place
    Rb, Rf = _rand_bf16(rng, (M, N), scale=4.0)
    C = dev(torch, Rb)
    binding.op_gemm(M, N, K, A, K, 1, B, K, 1, C, N, binding.OUT_RESID_BF16)
    got = bits_to_f32(C.cpu().numpy()).reshape(M, N)
    want = Rf + ref
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)
    # fp32 accumulate
    base = rng.standard_normal((M, N)).astype(np.float32)
    C = dev(torch, base)
    binding.op_gemm(M, N, K, A, K, 1, B, K, 1, C, N, binding.OUT_F32_ACC)
    got = C.cpu().numpy()
    assert np.abs(got - (base + ref)).max() < 1e-4


# ----------------------------------------------------------------------------
# QKV projection with QK-norm and RoPE in the GEMM epilogue
# ----------------------------------------------------------------------------
# Ragged rows (M = 400, 1.5 row tiles) and sequence lengths that are not a
# multiple of 256 take the per-row (cos, sin) path; multiples of 256 take the
# rotation-by-8-positions path; N not a multiple of 256 leaves half a column
# tile empty; one case has grouped key/value heads, one the d20 shape.
@pytest.mark.parametrize("B,T,d,H,HKV", [(2, 200, 256, 2, 2), (1, 512, 384, 3, 1), (3, 256, 128, 1, 1),
                                         (1, 2048, 1280, 10, 10)])
def test_qkv_projection_with_qk_norm_and_rope(B, T, d, H, HKV):
    log(f"qkv projection B={B} T={T} d={d} heads={H} kv_heads={HKV}")
    rng = np.random.default_rng(B * 1000 + T + d)
    NH = H + 2 * HKV
    xb, xf = _rand_bf16(rng, (B * T, d))
    wb, wf = _rand_bf16(rng, (NH * 128, d), scale=d ** -0.5)
    qkv = torch.zeros(B * T, NH * 128, dtype=torch.int16, device="cuda")
    rstd = torch.zeros(B * T, H + HKV, dtype=torch.float32, device="cuda")
    cs = torch.zeros(T * 128, dtype=torch.float32, device="cuda")
    binding.op_qkv_projection(dev(torch, xb), dev(torch, wb), qkv, rstd, cs, B, T, d, H, HKV)
    torch.cuda.synchronize()
    got = bits_to_f32(qkv.cpu().numpy()).astype(np.float64).reshape(B, T, NH, 128)
    got_r = rstd.cpu().numpy().reshape(B, T, H + HKV)
    x = (xf @ wf.T).reshape(B, T, NH, 128)
    cos, sin = oracle.rope_tables(T)
    n, r = oracle.rms_norm(x[:, :, :H + HKV])
    want_qk = np.stack([oracle.rope(n[b], cos, sin) for b in range(B)])
    # Per element: the kernel rotates bf16(x) * rstd and rounds the result, so
    # |error| <= 2^-9 (|n_j| + |n_j+64| + |out|); the bar is twice that.
    pair = np.abs(n) + np.abs(np.concatenate([n[..., 64:], n[..., :64]], axis=-1))
    err = np.abs(got[:, :, :H + HKV] - want_qk)
    assert np.all(err <= 2.0 ** -8 * (pair + np.abs(want_qk)) + 1e-6), float(err.max())
    assert rel_l2(got[:, :, :H + HKV], want_qk) < 5e-3
    assert np.all(np.abs(got_r - r[..., 0]) <= 1e-4 * np.abs(r[..., 0]))
    # v heads: the projection rounded once.
    v = x[:, :, H + HKV:]
    assert np.all(np.abs(got[:, :, H + HKV:] - v) <= 2.0 ** -8 * np.abs(v) + 1e-6)


def test_qkv_projection_rejects_bad_shapes():
    t = torch.zeros(64, dtype=torch.int16, device="cuda")
    f = torch.zeros(64, dtype=torch.float32, device="cuda")
    for args in [(1, 8, 100, 1, 1), (1, 8, 128, 3, 2), (0, 8, 128, 1, 1), (1, 8, 128, 1, 0)]:
        with pytest.raises(binding.GptError):
            binding.op_qkv_projection(t, t, t, f, f, *args)


# ----------------------------------------------------------------------------
# Attention forward / backward against the oracle (fp64 on the same bf16 inputs)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,H,W,HKV", [(2, 200, 2, -1, 2), (1, 64, 1, -1, 1), (1, 1, 1, -1, 1),
                                         (1, 333, 3, -1, 3), (1, 1024, 2, -1, 2), (1, 4096, 2, -1, 2),
                                         # windows: only the diagonal, odd sizes across tile edges,
                                         # exactly one tile, and the short window of a 4096 sequence
                                         (2, 200, 2, 0, 2), (1, 333, 3, 37, 3), (1, 300, 2, 63, 2),
                                         (1, 300, 2, 64, 2), (1, 1000, 1, 129, 1), (1, 1024, 2, 200, 2),
                                         (1, 4096, 2, 2048, 2),
                                         # grouped-query attention: groups of 2, 4 and 3 query heads
                                         (1, 333, 4, -1, 2), (2, 200, 4, 37, 1), (1, 1024, 6, -1, 2),
                                         (1, 2048, 4, 1024, 2),
                                         # more heads than one block-order group, ragged last
                                         # group, with and without the XCD remap
                                         (3, 200, 5, -1, 5), (4, 256, 5, -1, 5)])
def test_attention_fwd_bwd(B, T, H, W, HKV):
    log(f"attention B={B} T={T} H={H} window={W} kv_heads={HKV}")
    rng = np.random.default_rng(T + H)
    d, dkv = H * 128, HKV * 128
    qkv_b, qkv_f = _rand_bf16(rng, (B * T, d + 2 * dkv))
    do_b, do_f = _rand_bf16(rng, (B * T, d))
    qkv = dev(torch, qkv_b)
    o = torch.zeros(B * T, d, dtype=torch.int16, device="cuda")
    lse = torch.zeros(B * H * T, dtype=torch.float32, device="cuda")
    binding.op_attention_fwd(qkv, o, lse, B, T, H, W, kv_heads=HKV)
    dO = dev(torch, do_b)
    dqkv = torch.zeros(B * T, d + 2 * dkv, dtype=torch.int16, device="cuda")
    scratch = torch.zeros(B * H * T, dtype=torch.float32, device="cuda")
    binding.op_attention_bwd(qkv, o, lse, dO, dqkv, scratch, B, T, H, W, kv_heads=HKV)
    torch.cuda.synchronize()
    o_got = bits_to_f32(o.cpu().numpy()).reshape(B, T, H, 128)
    lse_got = lse.cpu().numpy().reshape(B, H, T)
    dqkv_got = bits_to_f32(dqkv.cpu().numpy()).reshape(B, T, d + 2 * dkv)
    for b in range(B):
        blk = qkv_f[b * T:(b + 1) * T]
        q = blk[:, :d].reshape(T, H, 128)
        k = blk[:, d:d + dkv].reshape(T, HKV, 128)
        v = blk[:, d + dkv:].reshape(T, HKV, 128)
        o_ref, p = oracle.causal_attention(q, k, v, None if W < 0 else W)
        assert rel_l2(o_got[b], o_ref) < 1e-2
        # lse: base-2 log of sum_j exp(q.k_j / sqrt(128)) over the visible j.
        kr = np.repeat(k, H // HKV, axis=1)
        s = np.einsum("ihd,jhd->hij", q, kr) / np.sqrt(128.0)
        vis = np.tril(np.ones((T, T), bool))
        if W >= 0:
            vis &= np.triu(np.ones((T, T), bool), -W)
        s = np.where(vis[None], s, -np.inf)
        m = s.max(-1, keepdims=True)
        lse_ref = (m[..., 0] + np.log(np.exp(s - m).sum(-1))) / np.log(2.0)
        assert np.abs(lse_got[b] - lse_ref).max() < 1e-3
        do = do_f[b * T:(b + 1) * T].reshape(T, H, 128)
        # The backward takes the kernel's own o (as the fused kernels do), so
        # the reference gradient is formed with the same o via rowsum(dO * o).
        dq_ref, dk_ref, dv_ref = oracle.causal_attention_bwd(do, q, k, v, p)
        got_q = dqkv_got[b, :, :d].reshape(T, H, 128)
        got_k = dqkv_got[b, :, d:d + dkv].reshape(T, HKV, 128)
        got_v = dqkv_got[b, :, d + dkv:].reshape(T, HKV, 128)
        for got, ref in ((got_q, dq_ref), (got_k, dk_ref), (got_v, dv_ref)):
            if np.linalg.norm(ref) == 0:
                # Window 0: P is the identity, so dS = 0 exactly in the oracle;
                # the kernel's dP - delta is a difference of two fp32 sums.
                assert np.abs(got).max() < 1e-3
            else:
                assert rel_l2(got, ref) < 2e-2


@pytest.mark.parametrize("B,T,H,W,HKV", [(2, 200, 2, -1, 2), (1, 512, 3, 100, 1), (1, 2048, 2, -1, 2)])
def test_attention_bwd_through_qk_norm_and_rope(B, T, H, W, HKV):
    """The step's attention backward, whose dQ and dK epilogues carry the
    QK-norm + RoPE backward, against the oracle's attention backward followed
    by rope_bwd and rms_norm_bwd, all on the GPU forward's own q, k, v (as
    the plain attention test feeds both sides the same qkv)."""
    log(f"attention bwd through qk-norm/rope B={B} T={T} H={H} window={W} kv_heads={HKV}")
    rng = np.random.default_rng(7 * T + H)
    d, dkv = H * 128, HKV * 128
    NH = H + 2 * HKV
    xb, _ = _rand_bf16(rng, (B * T, d))
    # Projections of RMS ~2.5, so that rstd ~0.4 matters in the check.
    wb, _ = _rand_bf16(rng, (NH * 128, d), scale=2.5 * d ** -0.5)
    qkv = torch.zeros(B * T, NH * 128, dtype=torch.int16, device="cuda")
    rstd = torch.zeros(B * T, H + HKV, dtype=torch.float32, device="cuda")
    cs = torch.zeros(T * 128, dtype=torch.float32, device="cuda")
    binding.op_qkv_projection(dev(torch, xb), dev(torch, wb), qkv, rstd, cs, B, T, d, H, HKV)
    o = torch.zeros(B * T, d, dtype=torch.int16, device="cuda")
    lse = torch.zeros(B * H * T, dtype=torch.float32, device="cuda")
    binding.op_attention_fwd(qkv, o, lse, B, T, H, W, kv_heads=HKV)
    do_b, do_f = _rand_bf16(rng, (B * T, d))
    dqkv = torch.zeros_like(qkv)
    scratch = torch.zeros(B * H * T, dtype=torch.float32, device="cuda")
    binding.op_attention_bwd_qknorm(qkv, o, lse, dev(torch, do_b), rstd, cs, dqkv, scratch, B, T, H, W,
                                    kv_heads=HKV)
    torch.cuda.synchronize()
    y = bits_to_f32(qkv.cpu().numpy()).astype(np.float64).reshape(B, T, NH, 128)
    r = rstd.cpu().numpy().astype(np.float64).reshape(B, T, H + HKV, 1)
    got = bits_to_f32(dqkv.cpu().numpy()).astype(np.float64).reshape(B, T, NH, 128)
    cos, sin = oracle.rope_tables(T)
    for b in range(B):
        q, k, v = y[b, :, :H], y[b, :, H:H + HKV], y[b, :, H + HKV:]
        _, p = oracle.causal_attention(q, k, v, None if W < 0 else W)
        dq, dk, dv = oracle.causal_attention_bwd(do_f[b * T:(b + 1) * T].reshape(T, H, 128), q, k, v, p)
        # Back through the rotation, then the norm (n = the unrotated saved head).
        dx = [oracle.rms_norm_bwd(oracle.rope_bwd(g, cos, sin), oracle.rope_bwd(yy, cos, sin), rr)
              for g, yy, rr in ((dq, q, r[b, :, :H]), (dk, k, r[b, :, H:]))]
        errs = (rel_l2(got[b, :, :H], dx[0]), rel_l2(got[b, :, H:H + HKV], dx[1]),
                rel_l2(got[b, :, H + HKV:], dv))
        log(f"  rel-L2 dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
        assert max(errs) < 1e-2  # measured 2.2e-3 to 2.7e-3


# ----------------------------------------------------------------------------
# Newton-Schulz against the oracle iteration
# ----------------------------------------------------------------------------
# Bars: the update tolerance (rel-L2 2e-2) on small matrices, 5e-3 at a block
# shape. The first iteration takes bf16 operands, the others fp16, all with
# fp32 accumulation, X kept in fp16 between iterations; a CPU emulation of
# those roundings puts Gaussian inputs at 3.0e-3 (256 x 256), 5.8e-3
# (384 x 128) and 1.3e-3 (1280 x 1280) from the fp64 iteration.
NS_BAR = {(384, 128): 2e-2, (256, 256): 2e-2, (1280, 1280): 5e-3, (40, 24): 2e-2, (72, 72): 2e-2,
          (200, 56): 2e-2, (96, 96): 2e-2, (136, 136): 2e-2}


# The last five shapes are multiples of 8 but not of 128 (the op's contract):
# single partial tiles, K not a multiple of 32 (the single-group kernel with
# its zeroed partial k-block) and symmetric products over ragged tiles.
@pytest.mark.parametrize("count,rows,cols", [(3, 384, 128), (2, 256, 256), (1, 1280, 1280), (2, 40, 24),
                                             (1, 72, 72), (2, 200, 56), (1, 96, 96), (1, 136, 136)])
def test_newton_schulz(count, rows, cols):
    log(f"newton-schulz count={count} rows={rows} cols={cols}")
    rng = np.random.default_rng(rows + cols)
    X = rng.standard_normal((count, rows, cols)).astype(np.float32)
    Xd = dev(torch, X)
    scratch = torch.empty(binding.ns_scratch_bytes(count, rows, cols), dtype=torch.uint8, device="cuda")
    binding.op_newton_schulz(Xd, count, rows, cols, syn.NS_COEFFS, scratch)
    torch.cuda.synchronize()
    got = Xd.cpu().numpy()
    for i in range(count):
        ref = oracle.newton_schulz(X[i].astype(np.float64), syn.NS_COEFFS)
        e = rel_l2(got[i], ref)
        log(f"  matrix {i}: rel-L2 {e:.2e}")
        assert e < NS_BAR[(rows, cols)], e


@pytest.mark.parametrize("steps", [1, 2, 3])
def test_newton_schulz_fewer_steps(steps):
    """Shorter tables: one step is the bf16 first iteration alone (its fp32
    output is the result), two end with the fp16 iteration that writes fp32,
    three pass X through fp16 once in between."""
    count, rows, cols = 2, 512, 256
    log(f"newton-schulz steps={steps} count={count} rows={rows} cols={cols}")
    rng = np.random.default_rng(17 + steps)
    X = rng.standard_normal((count, rows, cols)).astype(np.float32)
    Xd = dev(torch, X)
    scratch = torch.empty(binding.ns_scratch_bytes(count, rows, cols), dtype=torch.uint8, device="cuda")
    table = np.asarray(syn.NS_COEFFS, dtype=np.float32)[:steps]
    binding.op_newton_schulz(Xd, count, rows, cols, table, scratch)
    torch.cuda.synchronize()
    got = Xd.cpu().numpy()
    for i in range(count):
        ref = oracle.newton_schulz(X[i].astype(np.float64), syn.NS_COEFFS, steps)
        e = rel_l2(got[i], ref)
        log(f"  matrix {i}: rel-L2 {e:.2e}")
        assert e < (2e-3 if steps == 1 else 2e-2), e


@pytest.mark.parametrize("count,rows,cols", [(2, 256, 256), (1, 1280, 1280), (3, 384, 128)])
def test_newton_schulz_is_bit_reproducible(count, rows, cols):
    """Two runs on identical inputs give identical bits: every sum has a fixed
    order (no atomics, no split-dependent reduction), including the epilogues
    that read and rewrite the fp32 master X in place."""
    log(f"newton-schulz repeat count={count} rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * cols)
    X = rng.standard_normal((count, rows, cols)).astype(np.float32)
    outs = []
    for _ in range(2):
        Xd = dev(torch, X)
        scratch = torch.empty(binding.ns_scratch_bytes(count, rows, cols), dtype=torch.uint8, device="cuda")
        binding.op_newton_schulz(Xd, count, rows, cols, syn.NS_COEFFS, scratch)
        torch.cuda.synchronize()
        outs.append(Xd.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
