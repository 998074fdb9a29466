"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, plans the documented layout and rejects bad arguments on the host
before any launch."""
import ctypes as C
import os
import re

import pytest

from gpt_pretraining_step_bf16_amd import binding, synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libgptstep.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n.startswith(("gpt_", "muon_", "normuon_", "adamw_")) and n not in skip})


def test_every_declared_symbol_is_exported():
    lib = C.CDLL(binding.LIB_PATH)
    declared = _declared_functions()
    assert "gpt_fwd_bwd" in declared and "muon_step" in declared and "gpt_create" in declared
    assert "adamw_step" in declared and "normuon_step" in declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(binding.EXPORTS), set(declared) ^ set(binding.EXPORTS)


@pytest.mark.parametrize("depth,vocab", [(1, 64), (2, 2048), (3, 2048), (12, 32768), (20, 32768),
                                         (26, 32768), (32, 32768)])
def test_layout_matches_canonical_specs(depth, vocab):
    m = binding.GptModel(depth, vocab, 128)
    dm = syn.model_dims(depth)
    assert (m.d, m.heads, m.mlp, m.vocab) == (dm["d"], dm["heads"], dm["mlp"], vocab)
    specs = syn.tensor_specs(depth, vocab)
    tens = m.tensors()
    assert len(tens) == len(specs)
    off = 0
    for t, (name, rows, cols, kind, layer) in zip(tens, specs):
        assert (t["name"], t["rows"], t["cols"], t["kind"], t["layer"]) == (name, rows, cols, kind, layer)
        assert t["offset"] == off
        off += rows * cols
    assert m.num_params == off


def test_param_counts_closed_form():
    # 2·V·d (wte, lm_head) + L·12·d² (q, k, v, o: d² each; fc, proj: 4d² each)
    # at d20 (d = 1280) and d32 (d = 2048), V = 32768.
    m = binding.GptModel(20, 32768, 2048)
    assert m.num_params == 477_102_080
    m = binding.GptModel(32, 32768, 4096)
    assert m.num_params == 1_744_830_464


def test_workspace_sizes():
    m = binding.GptModel(2, 2048, 64)
    w1 = m.workspace_bytes(1, 64)
    w2 = m.workspace_bytes(2, 64)
    assert 0 < w1 < w2
    assert m.workspace_bytes(1, 65) == 0  # beyond max_seq
    assert m.workspace_bytes(0, 64) == 0
    assert m.muon_workspace_bytes() > 0


def test_create_rejects_bad_arguments():
    lib = binding.lib()
    h = C.c_void_p()
    for depth, vocab, seq in ((0, 2048, 64), (65, 2048, 64), (2, 2000, 64), (2, 2048, 0),
                              (2, 2048, 16385), (2, 32, 64)):
        assert lib.gpt_create(depth, vocab, seq, C.byref(h)) == binding.GPT_EINVAL
    assert lib.gpt_create(2, 2048, 64, None) == binding.GPT_EINVAL


def test_fwd_bwd_host_validation_precedes_any_launch():
    lib = binding.lib()
    m = binding.GptModel(2, 2048, 64)
    fake = C.c_void_p(4096)
    ws_need = m.workspace_bytes(2, 64)
    args = dict(pbf=fake, tok=fake, tgt=fake, B=2, T=64, loss=fake, grads=fake, acc=0,
                ws=C.c_void_p(1 << 20), wsb=ws_need, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.gpt_fwd_bwd(m.handle, a["pbf"], a["tok"], a["tgt"], a["B"], a["T"], a["loss"],
                               a["grads"], a["acc"], a["ws"], a["wsb"], a["stream"])

    assert call(pbf=None) == binding.GPT_EINVAL
    assert call(tok=None) == binding.GPT_EINVAL
    assert call(loss=None) == binding.GPT_EINVAL
    assert call(B=0) == binding.GPT_EINVAL
    assert call(T=65) == binding.GPT_ESHAPE
    assert call(acc=2) == binding.GPT_EINVAL
    assert call(wsb=ws_need - 1) == binding.GPT_EWORKSPACE
    assert call(ws=None) == binding.GPT_EWORKSPACE
    assert call(ws=C.c_void_p((1 << 20) + 16)) == binding.GPT_EINVAL  # not 256-byte aligned


def test_muon_and_op_validation():
    lib = binding.lib()
    m = binding.GptModel(2, 2048, 64)
    fake = C.c_void_p(4096)
    buf, _ = binding._coeffs(syn.NS_COEFFS)
    need = m.muon_workspace_bytes()
    ws = C.c_void_p(1 << 20)
    assert lib.muon_step(m.handle, fake, fake, fake, fake, 0.02, 0.95, buf, 0, ws, need, None) == binding.GPT_EINVAL
    # NULL coefficients select the built-in five-row table: more rows than it has is rejected,
    # and the workspace check still comes before any launch.
    assert lib.muon_step(m.handle, fake, fake, fake, fake, 0.02, 0.95, None, 6, ws, need, None) == binding.GPT_EINVAL
    assert lib.muon_step(m.handle, fake, fake, fake, fake, 0.02, 0.95, None, 5, ws, need - 1, None) == binding.GPT_EWORKSPACE
    assert lib.muon_step(m.handle, None, fake, fake, fake, 0.02, 0.95, None, 5, ws, need, None) == binding.GPT_EINVAL
    assert lib.muon_step(m.handle, fake, fake, fake, fake, 0.02, 0.95, buf, 5, ws, need - 1, None) == binding.GPT_EWORKSPACE
    # GEMM shape rules: N % 4, contiguous dims % 8.
    assert lib.gpt_op_gemm(64, 6, 64, 1, fake, 64, 0, 1, fake, 64, 0, 1, fake, 8, 0, 0, None) == binding.GPT_ESHAPE
    assert lib.gpt_op_gemm(64, 64, 60, 1, fake, 64, 0, 1, fake, 64, 0, 1, fake, 64, 0, 0, None) == binding.GPT_ESHAPE
    assert lib.gpt_op_gemm(64, 64, 64, 1, fake, 64, 0, 1, fake, 64, 0, 1, fake, 64, 0, 9, None) == binding.GPT_EINVAL
    assert lib.gpt_op_newton_schulz(fake, 1, 64, 128, buf, 5, ws, 1 << 30, None) == binding.GPT_ESHAPE
    assert binding.status_str(binding.GPT_ETOKEN).startswith("token")


def test_no_alloc_newton_schulz_host_checks():
    """The allocation-free Newton-Schulz entry point: its array size in the
    header equals the binding's, the documented shapes fit, larger requests
    and bad arguments are refused before any GPU call."""
    text = open(HEADER).read()
    m = re.search(r"#define GPT_NS_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NS_STATIC_SCRATCH_BYTES
    cap = binding.NS_STATIC_SCRATCH_BYTES
    assert binding.ns_scratch_bytes(2, 1280, 1280) <= cap and binding.ns_scratch_bytes(1, 5120, 1280) <= cap
    lib = binding.lib()
    buf, _ = binding._coeffs(syn.NS_COEFFS)
    fake = C.c_void_p(4096)
    assert lib.gpt_op_newton_schulz_noalloc(fake, 6, 1280, 1280, buf, 5, None) == binding.GPT_EWORKSPACE
    assert lib.gpt_op_newton_schulz_noalloc(None, 1, 256, 256, buf, 5, None) == binding.GPT_EINVAL
    assert lib.gpt_op_newton_schulz_noalloc(fake, 1, 128, 256, buf, 5, None) == binding.GPT_ESHAPE
    assert lib.gpt_op_newton_schulz_noalloc(fake, 1, 256, 256, buf, 9, None) == binding.GPT_EINVAL


def test_built_in_newton_schulz_table():
    """muon_step's table for ns_coeffs = NULL: its first two rows are the two
    triples the page prints (golden file), rows 3-5 follow the greedy minimax
    rule as the oracle re-derives it, and the whole table is the one the tests
    and the bench pass explicitly."""
    import numpy as np

    import oracle
    from test_oracle_muon import _read_triples

    table = binding.ns_default_coeffs()
    assert table.shape == (5, 3)
    printed = _read_triples(os.path.join(ROOT, "tests", "golden", "ns_coeffs_printed.txt"))
    np.testing.assert_array_equal(table[:2], np.asarray(printed, dtype=np.float32))
    derived, _ = oracle.greedy_minimax_triples(printed)
    np.testing.assert_allclose(table[2:], derived[2:], atol=2e-4)
    np.testing.assert_array_equal(table, syn.NS_COEFFS.astype(np.float32))


def test_adamw_state_and_host_validation_precede_any_launch():
    m = binding.GptModel(20, 32768, 2048)
    assert m.adamw_state_elems() == 2 * 32768 * 1280
    lib = binding.lib()
    fake = C.c_void_p(1 << 20)

    def call(p=fake, step=1, b1=0.9, b2=0.95, eps=1e-8, lr=0.01, wd=0.0):
        return lib.adamw_step(m.handle, p, fake, fake, fake, fake, lr, b1, b2, eps, wd, step, None)

    assert call(p=None) == binding.GPT_EINVAL
    assert call(step=0) == binding.GPT_EINVAL
    assert call(b1=1.0) == binding.GPT_EINVAL
    assert call(b2=-0.1) == binding.GPT_EINVAL
    assert call(eps=-1.0) == binding.GPT_EINVAL
    assert call(lr=float("nan")) == binding.GPT_EINVAL
    assert lib.adamw_step(None, fake, fake, fake, fake, fake, 0.01, 0.9, 0.95, 1e-8, 0.0, 1, None) == binding.GPT_EINVAL


def test_normuon_state_and_host_validation_precede_any_launch():
    m = binding.GptModel(20, 32768, 2048)
    # One value per element of each block matrix's longer side.
    assert m.normuon_state_elems() == 20 * (4 * 1280 + 2 * 5120)
    lib = binding.lib()
    fake = C.c_void_p(1 << 20)
    buf, _ = binding._coeffs(syn.NS_COEFFS)
    need = m.muon_workspace_bytes()

    def call(v=fake, b2=0.95, ws=C.c_void_p(1 << 20), wsb=need, steps=5):
        return lib.normuon_step(m.handle, fake, fake, fake, fake, v, 0.02, 0.95, b2, buf, steps, ws, wsb, None)

    assert call(v=None) == binding.GPT_EINVAL
    assert call(b2=1.0) == binding.GPT_EINVAL
    assert call(b2=-0.5) == binding.GPT_EINVAL
    assert call(b2=float("nan")) == binding.GPT_EINVAL
    assert call(steps=0) == binding.GPT_EINVAL
    assert call(wsb=need - 1) == binding.GPT_EWORKSPACE


def test_attention_windows_are_host_state_with_validation():
    from gpt_pretraining_step_bf16_amd.step import window_pattern

    m = binding.GptModel(6, 2048, 256)
    assert m.windows() == [-1] * 6
    pat = window_pattern(6, 256, "SSSL")
    assert pat == [128, 128, 128, -1, 128, 128]
    m.set_windows(pat)
    assert m.windows() == pat
    lib = binding.lib()
    bad = (C.c_int32 * 6)(1, 2, 3, -2, 5, 6)
    assert lib.gpt_set_attention_windows(m.handle, bad, 6) == binding.GPT_EINVAL
    short = (C.c_int32 * 5)(1, 2, 3, 4, 5)
    assert lib.gpt_set_attention_windows(m.handle, short, 5) == binding.GPT_ESHAPE
    assert m.windows() == pat  # a rejected call changes nothing
    m.set_windows(None)
    assert m.windows() == [-1] * 6
    with pytest.raises(ValueError):
        window_pattern(4, 64, "SXL")
    fake = C.c_void_p(4096)
    assert lib.gpt_op_attention_fwd(fake, fake, fake, 1, 64, 1, 1, -2, None) == binding.GPT_EINVAL
    assert lib.gpt_op_attention_fwd(fake, fake, fake, 1, 64, 4, 3, -1, None) == binding.GPT_EINVAL


@pytest.mark.parametrize("depth,kv_heads", [(4, 1), (20, 2), (20, 5), (12, 6)])
def test_gqa_layout_matches_canonical_specs(depth, kv_heads):
    m = binding.GptModel(depth, 2048, 128, kv_heads)
    assert m.kv_heads == kv_heads
    specs = syn.tensor_specs(depth, 2048, kv_heads)
    got = m.tensors()
    assert [t["name"] for t in got] == [sp[0] for sp in specs]
    off = 0
    for t, (name, rows, cols, _kind, _layer) in zip(got, specs):
        assert (t["rows"], t["cols"], t["offset"]) == (rows, cols, off), name
        off += rows * cols
    assert m.num_params == off
    d, f = m.d, m.mlp
    dkv = 128 * kv_heads
    # One value per element of each block matrix's longer side.
    assert m.normuon_state_elems() == depth * (2 * d + 2 * max(dkv, d) + f + f)
    assert m.muon_workspace_bytes() > 0 and m.workspace_bytes(2, 128) > 0


def test_gqa_create_rejects_kv_heads_that_do_not_divide():
    lib = binding.lib()
    h = C.c_void_p()
    assert lib.gpt_create_gqa(20, 2048, 128, 3, C.byref(h)) == binding.GPT_EINVAL  # 10 heads
    assert lib.gpt_create_gqa(20, 2048, 128, 11, C.byref(h)) == binding.GPT_EINVAL
    assert lib.gpt_create_gqa(20, 2048, 128, -1, C.byref(h)) == binding.GPT_EINVAL
    m = binding.GptModel(20, 2048, 128, 0)  # 0: every head
    assert m.kv_heads == m.heads == 10


@pytest.mark.parametrize("resid,backout,smear", [(True, None, False), (False, 1, False), (True, 0, True),
                                                (False, None, True)])
def test_scalar_tensors_follow_lm_head(resid, backout, smear):
    depth, vocab = 3, 2048
    m = binding.GptModel(depth, vocab, 128, None, resid, backout, smear)
    assert m.backout_layer == backout
    specs = syn.tensor_specs(depth, vocab, None, resid, backout is not None, smear)
    got = m.tensors()
    assert [(t["name"], t["rows"], t["cols"], t["kind"]) for t in got] == [sp[:4] for sp in specs]
    n_scal = (2 * depth if resid else 0) + (1 if backout is not None else 0) + (25 if smear else 0)
    assert m.adamw_state_elems() == 2 * vocab * m.d + n_scal
    assert m.num_params == sum(r * c for _, r, c, _, _ in specs)


def test_config_validation():
    lib = binding.lib()
    h = C.c_void_p()
    bad = [binding.GptConfig(3, 2048, 128, 0, 2, -1), binding.GptConfig(3, 2048, 128, 0, 0, 3),
           binding.GptConfig(3, 2048, 128, 0, 0, -2), binding.GptConfig(0, 2048, 128, 0, 1, -1),
           binding.GptConfig(3, 2048, 128, 0, 0, -1, 2)]
    for cfg in bad:
        assert lib.gpt_create_config(C.byref(cfg), C.byref(h)) == binding.GPT_EINVAL
    assert lib.gpt_create_config(None, C.byref(h)) == binding.GPT_EINVAL


def test_value_embedding_tensors_and_validation():
    depth, vocab = 4, 2048
    m = binding.GptModel(depth, vocab, 128, 1, False, None, False, (1, 3))
    specs = syn.tensor_specs(depth, vocab, 1, ve_layers=(1, 3))
    assert [(t["name"], t["rows"], t["cols"], t["kind"]) for t in m.tensors()] == [sp[:4] for sp in specs]
    assert m.adamw_state_elems() == 2 * vocab * m.d + 2 * (vocab * 128 + 32)
    lib = binding.lib()
    h = C.c_void_p()
    cfg = binding.GptConfig(4, 2048, 128, 0, 0, -1, 0, 1 << 4)  # layer 4 does not exist
    assert lib.gpt_create_config(C.byref(cfg), C.byref(h)) == binding.GPT_EINVAL
