"""Parity and invariants at the workload sizes: depth 12, 20, 26 and 32.

Shapes (width = 64 * depth, heads of 128, MLP 4 * width, vocab 32768):
  d12: seq 2048, microbatch 8      d20: seq 2048, microbatch 32 (bench workload)
  d26: seq 2048, microbatch 16     d32: seq 4096, microbatch 4
Weights are the seeded N(0, 0.02) draws, tokens seeded Zipf(1.1).

For each depth:
* One sequence through the whole model against the fp64 oracle, which is
  given the bf16 weights gpt_fwd_bwd computes with (at d12 and d20 also with
  the "SSSL" window pattern, short window seq / 2, and at d20 with 2 key/value
  heads for the 10 query heads plus value embeddings on the odd layers, and
  with residual scalars, a backout at layer 10 and smear): loss |delta| <= 1e-2,
  every gradient tensor rel-L2 <= 2e-2, embedding rows of absent tokens exactly
  zero. The sequence is the workload's full length, 4096 tokens at d32 (the
  oracle recomputes each head's probabilities in the backward, so it holds
  one T x T array per head at a time; about 40 GB of host memory and several
  minutes at d32).
* The full microbatch against the same sequences run one at a time and
  accumulated (accumulate=1) in the same workspace. Per token the forward and
  the activation gradients are the same arithmetic (no product is split over
  k along the token axis there); what differs is the fp32 summation order of
  the weight gradients over tokens (split-K plans and head chunks depend on
  the token count) and of the embedding scatter. The loss agrees to 1e-4
  relative and the gradient to ACC_TOL rel-L2 (fp32 reassociation; measured
  about 1e-6).
* A repeated full microbatch gives a bit-identical loss and bit-identical
  gradients for every tensor, the embedding's included (every sum has a fixed
  order; the embedding scatter sums each token's rows by sorted position).
* muon_step on the whole model against the oracle Muon step for the matrices
  of the first block (and the last, at d12 and d20), from identical fp32
  weights, gradients and momenta: momentum rel-L2 <= 1e-6, update rel-L2 <= 2e-2.
"""
import numpy as np
import pytest

from gpu_util import assert_scalar_grads, bf16_round, log, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpt_pretraining_step_bf16_amd import synthetic as syn  # noqa: E402
from gpt_pretraining_step_bf16_amd.step import TrainState, window_pattern  # noqa: E402

LOSS_TOL = 1e-2
REL_TOL = 2e-2
ACC_TOL = 1e-5
# Scalar and value-embedding-gate gradients: allowed |delta| as a fraction of
# their Cauchy-Schwarz scale S (gpu_util.assert_scalar_grads), a few times
# the largest error measured at these sizes.
SCALAR_EPS = {"resid_lambdas": 2e-4, "x0_lambdas": 2e-4, "backout_lambda": 2e-4, "smear_lambda": 2e-4,
              "smear_gate": 1e-3}
VE_GATE_EPS = 1e-3
ORACLE_SEQ = {"d12": 2048, "d20": 2048, "d26": 2048, "d32": 4096}
MUON_LAYERS = {"d12": "first_last", "d20": "first_last", "d26": "first_last", "d32": "first_last"}
NAMES = ("wq", "wk", "wv", "wo", "wfc", "wproj")


def _cfg(name):
    c = syn.CONFIGS[name]
    return c["depth"], c["vocab"], c["seq"], c["batch"]


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# The fp64 oracle needs from a few seconds (d12) to about a minute (d26) of
# host time for one sequence, and several minutes for d32's 4096 tokens.
@pytest.mark.timeout(1000)
@pytest.mark.parametrize("name,pattern,kv_heads,scalars,ve", [
    ("d12", None, None, False, False), ("d20", None, None, False, False), ("d26", None, None, False, False),
    ("d32", None, None, False, False), ("d12", "SSSL", None, False, False), ("d20", "SSSL", None, False, False),
    ("d20", None, 2, False, True), ("d20", None, None, True, False)])
def test_one_sequence_matches_oracle(name, pattern, kv_heads, scalars, ve):
    L, V, _, _ = _cfg(name)
    T = ORACLE_SEQ[name]
    windows = None if pattern is None else window_pattern(L, T, pattern)
    log(f"{name} one sequence of {T} vs oracle" + (f", windows {pattern} (short {T // 2})" if pattern else "")
        + (f", {kv_heads} kv heads" if kv_heads else ""))
    backout = L // 2 if scalars else None
    ve_layers = tuple(range(1, L, 2)) if ve else ()
    w = syn.init_weights(L, V, seed=0, kv_heads=kv_heads, resid_scalars=scalars, backout=scalars, smear=scalars,
                         ve_layers=ve_layers)
    if scalars:
        w["smear_gate"] = (np.random.default_rng(4).standard_normal((1, 24)) * 2.0).astype(np.float32)
        w["smear_lambda"] = np.array([[0.5]], dtype=np.float32)
        rng = np.random.default_rng(3)
        w["resid_lambdas"] = rng.uniform(0.7, 1.3, size=(1, L)).astype(np.float32)
        w["x0_lambdas"] = rng.uniform(-0.3, 0.3, size=(1, L)).astype(np.float32)
        w["backout_lambda"] = np.array([[0.9]], dtype=np.float32)
    tok, tgt = syn.split_tokens(syn.zipf_ids(1, T, V, seed=1))
    st = TrainState(L, V, T, 1, kv_heads=kv_heads, resid_scalars=scalars, backout_layer=backout, smear=scalars,
                    ve_layers=ve_layers)
    st.load_weights(w)
    st.set_windows(windows)
    st.fwd_bwd(_cuda(tok), _cuda(tgt))
    torch.cuda.synchronize()
    assert st.check() == 0
    loss = float(st.loss.cpu()[0])
    grads = st.to_host(st.grads)
    del st
    torch.cuda.empty_cache()
    w64 = {k: bf16_round(v).astype(np.float64) for k, v in w.items()}
    del w
    scales = {}
    ref_loss, ref_grads = oracle.forward_backward(
        w64, tok, tgt, windows=None if windows is None else [None if x < 0 else x for x in windows],
        backout_layer=backout, scalar_scales=scales)
    del w64
    if scales:
        # Scalar and gate gradients are checked against their Cauchy-Schwarz
        # scale (see gpu_util.assert_scalar_grads), the rest by rel-L2.
        sg = {k: grads.pop(k) for k in scales}
        sref = {k: ref_grads.pop(k) for k in scales}
    errs = sorted(((rel_l2(grads[k], ref_grads[k]), k) for k in ref_grads), reverse=True)
    log(f"  loss {loss:.6f} oracle {ref_loss:.6f}; worst grad rel-L2 "
        + " ".join(f"{k}:{e:.4f}" for e, k in errs[:4]))
    assert abs(loss - ref_loss) <= LOSS_TOL
    assert errs[0][0] < REL_TOL, errs[0]
    num = sum(float(np.sum((grads[k].astype(np.float64) - ref_grads[k]) ** 2)) for k in ref_grads)
    den = sum(float(np.sum(ref_grads[k] ** 2)) for k in ref_grads)
    assert np.sqrt(num / den) < REL_TOL
    absent = np.setdiff1d(np.arange(V), tok.ravel())
    assert not np.any(grads["wte"][absent])
    if scales:
        gates = {k: v for k, v in scales.items() if k.endswith(".ve_gate")}
        others = {k: v for k, v in scales.items() if k not in gates}
        assert_scalar_grads(sg, sref, others, log, eps=SCALAR_EPS)
        assert_scalar_grads(sg, sref, gates, log, eps=VE_GATE_EPS)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["d12", "d20", "d26", "d32"])
def test_full_batch_consistent_and_deterministic(name):
    L, V, T, B = _cfg(name)
    log(f"{name} microbatch {B} x {T}: repeat, then one sequence at a time")
    tok, tgt = syn.split_tokens(syn.zipf_ids(B, T, V, seed=1))
    st = TrainState(L, V, T, B)
    st.load_weights(syn.init_weights(L, V, seed=0))
    tok_d, tgt_d = _cuda(tok), _cuda(tgt)
    st.fwd_bwd(tok_d, tgt_d)
    torch.cuda.synchronize()
    assert st.check() == 0
    loss_b = st.loss.clone()
    grads_b = st.grads.clone()
    st.fwd_bwd(tok_d, tgt_d)
    torch.cuda.synchronize()
    assert st.loss.item() == loss_b.item()
    assert torch.equal(st.grads, grads_b)
    assert np.isfinite(loss_b.item())

    losses = []
    for b in range(B):
        st.fwd_bwd(tok_d[b:b + 1], tgt_d[b:b + 1], accumulate=b > 0)
        losses.append(st.loss.clone())
    torch.cuda.synchronize()
    assert st.check() == 0
    mean_loss = torch.stack(losses).double().mean().item()
    log(f"  loss {loss_b.item():.6f}, mean over sequences {mean_loss:.6f}")
    assert abs(loss_b.item() - mean_loss) <= 1e-4 * abs(mean_loss)
    # Every target is valid and every sequence has T of them, so the batch
    # gradient is the mean of the per-sequence gradients.
    acc = st.grads.double() / B
    ref = grads_b.double()
    err = (torch.linalg.vector_norm(acc - ref) / torch.linalg.vector_norm(ref)).item()
    log(f"  gradient rel-L2 {err:.2e}")
    assert err < ACC_TOL


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["d12", "d20", "d26", "d32"])
def test_muon_matches_oracle(name):
    L, V, T, _ = _cfg(name)
    log(f"{name} muon")
    w = syn.init_weights(L, V, seed=0)
    g = syn.random_like_grads(L, V, seed=7, scale=1e-2)
    m0 = syn.random_like_grads(L, V, seed=8, scale=1e-2)
    st = TrainState(L, V, T, 1)
    st.load_weights(w)
    st.load_grads(g)
    st.load_momentum(m0)
    st.muon(syn.MUON_LR, syn.MUON_MOMENTUM, syn.NS_COEFFS)
    torch.cuda.synchronize()
    new_w = st.to_host(st.params)
    new_m = st.to_host(st.momentum)
    del st
    torch.cuda.empty_cache()
    layers = (0, L - 1) if MUON_LAYERS[name] == "first_last" else (0,)
    names = [f"h{l}.{n}" for l in layers for n in NAMES]
    f64 = lambda d: {k: d[k].astype(np.float64) for k in names}
    _, ref_m, ref_upd = oracle.muon_step(f64(w), f64(g), f64(m0), syn.MUON_LR, syn.MUON_MOMENTUM,
                                         syn.NS_COEFFS, names=names)
    worst = []
    for k in names:
        assert rel_l2(new_m[k], ref_m[k]) < 1e-6, k
        e = rel_l2(w[k].astype(np.float64) - new_w[k], ref_upd[k])
        worst.append((e, k))
        assert e < REL_TOL, (k, e)
    log("  worst update rel-L2 " + " ".join(f"{k}:{e:.2e}" for e, k in sorted(worst)[-3:]))
    np.testing.assert_array_equal(new_w["wte"], w["wte"])
    np.testing.assert_array_equal(new_w["lm_head"], w["lm_head"])


@pytest.mark.timeout(300)
def test_muon_step_is_bit_reproducible_and_takes_the_built_in_table():
    """muon_step at d20 twice from identical weights, gradients and momenta:
    identical parameters, bf16 shadow and momenta, bit for bit (the staged
    Newton-Schulz epilogues included); the NULL table (the library's built-in
    one) gives the same bits as passing that table explicitly."""
    L, V, T, _ = _cfg("d20")
    log("d20 muon repeat")
    w = syn.init_weights(L, V, seed=0)
    g = syn.random_like_grads(L, V, seed=7, scale=1e-2)
    m0 = syn.random_like_grads(L, V, seed=8, scale=1e-2)
    st = TrainState(L, V, T, 1)
    st.load_grads(g)
    outs = []
    for coeffs in (syn.NS_COEFFS, syn.NS_COEFFS, None):
        st.load_weights(w)
        st.load_momentum(m0)
        st.muon(syn.MUON_LR, syn.MUON_MOMENTUM, coeffs)
        torch.cuda.synchronize()
        outs.append((st.params.clone(), st.params_bf16.clone(), st.momentum.clone()))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)
