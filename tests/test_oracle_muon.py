"""Pins of the oracle's Muon step against closed forms and the coefficient rule."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import muon as om
from oracle import polar_express as pe
from gpt_pretraining_step_bf16_amd import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_triples(path):
    rows = []
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def test_printed_triples_are_the_first_two_rows():
    printed = _read_triples(os.path.join(GOLDEN, "ns_coeffs_printed.txt"))
    assert printed.shape == (2, 3)
    np.testing.assert_array_equal(syn.NS_COEFFS[:2], printed)


def test_greedy_minimax_reproduces_table_rows_3_to_5():
    printed = _read_triples(os.path.join(GOLDEN, "ns_coeffs_printed.txt"))
    table, images = pe.greedy_minimax_triples(printed)
    np.testing.assert_allclose(table[2:], syn.NS_COEFFS[2:], atol=2e-4)
    # Equioscillation: each minimax step maps its interval onto [1 - E, 1 + E].
    for lo, hi in images[2:]:
        assert abs((1.0 - lo) - (hi - 1.0)) < 1e-3
    lo, hi = images[-1]
    assert 0.86 < lo < 0.88 and 1.12 < hi < 1.14


@pytest.mark.parametrize("shape", [(64, 32), (48, 48), (20, 70)])
def test_iteration_equals_svd_closed_form(shape):
    rng = np.random.default_rng(sum(shape))
    m = rng.standard_normal(shape)
    x_iter = om.newton_schulz(m, syn.NS_COEFFS)
    x_svd = om.newton_schulz_svd(m, syn.NS_COEFFS)
    np.testing.assert_allclose(x_iter, x_svd, rtol=0, atol=1e-11)


def test_singular_values_land_in_band_for_tall_gaussians():
    rng = np.random.default_rng(0)
    for shape in ((512, 128), (640, 160)):
        m = rng.standard_normal(shape)
        s = np.linalg.svd(om.newton_schulz(m, syn.NS_COEFFS), compute_uv=False)
        assert s.min() >= 0.870 and s.max() <= 1.130, (s.min(), s.max())


def test_orthogonal_input_gives_scalar_multiple():
    rng = np.random.default_rng(1)
    q, _ = np.linalg.qr(rng.standard_normal((40, 24)))
    x = om.newton_schulz(q, syn.NS_COEFFS)
    # All singular values equal 1/sqrt(24) after normalisation, so each step
    # multiplies the matrix by the same scalar.
    s = 1.0 / (math.sqrt(24) + 1e-7)
    for a, b, c in syn.NS_COEFFS:
        s = a * s + b * s ** 3 + c * s ** 5
    np.testing.assert_allclose(x, s * q, rtol=1e-10, atol=1e-12)


def test_zero_gradient_gives_zero_update():
    w = {"h0.wq": np.ones((8, 8)), "wte": np.ones((4, 8))}
    z = {k: np.zeros_like(v) for k, v in w.items()}
    nw, nm, upd = om.muon_step(w, z, z, 0.02, 0.95, syn.NS_COEFFS)
    assert not np.any(upd["h0.wq"]) and np.all(np.isfinite(nw["h0.wq"]))
    np.testing.assert_array_equal(nw["h0.wq"], w["h0.wq"])


def test_muon_step_momentum_scale_and_untouched_tensors():
    depth, vocab = 1, 64
    w = {k: v.astype(np.float64) for k, v in syn.init_weights(depth, vocab, seed=0).items()}
    g = {k: v.astype(np.float64) for k, v in syn.random_like_grads(depth, vocab, seed=1).items()}
    m0 = {k: v.astype(np.float64) for k, v in syn.random_like_grads(depth, vocab, seed=2).items()}
    lr, mu = 0.02, 0.95
    nw, nm, upd = om.muon_step(w, g, m0, lr, mu, syn.NS_COEFFS)
    np.testing.assert_array_equal(nw["wte"], w["wte"])
    np.testing.assert_array_equal(nw["lm_head"], w["lm_head"])
    for name in ("h0.wq", "h0.wfc", "h0.wproj"):
        np.testing.assert_allclose(nm[name], mu * m0[name] + g[name], rtol=1e-15)
        rows, cols = w[name].shape
        scale = max(1.0, rows / cols) ** 0.5
        s = np.linalg.svd(upd[name] / (lr * scale), compute_uv=False)
        # Square Gaussians have singular values near 0, below the table's
        # design floor of 1e-3 relative, so only the bulk is checked there.
        lo = s.min() if rows != cols else np.percentile(s, 5)
        assert lo > 0.85 and s.max() < 1.15, (name, lo, s.max())
        np.testing.assert_allclose(nw[name], w[name] - upd[name], rtol=1e-15)
    assert upd["h0.wfc"].shape == (512, 128)
    # fan-out > fan-in takes sqrt(rows / cols); the wide matrix takes 1.
    assert om.muon_scale(512, 128) == 2.0 and om.muon_scale(128, 512) == 1.0
