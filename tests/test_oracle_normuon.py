"""Pins of the NorMuon oracle against a hand-worked example, closed forms and
invariants that follow from the definition (see the oracle module header)."""
import numpy as np
import pytest

from oracle.muon import muon_step
from oracle.normuon import normuon_step, variance_reduction


def test_hand_worked_two_by_two():
    # o rows (3, 4) and (6, 8): per-row means of squares 12.5 and 50, so
    # v_norm = sqrt(62.5). beta2 = 0.5 from a zero state: v = (6.25, 25),
    # step sizes (0.4, 0.2); v_norm_new = sqrt(12.5 * 0.16 + 50 * 0.04) = 2.
    # Final scales 0.4 * sqrt(62.5) / 2 and 0.2 * sqrt(62.5) / 2 make both
    # rows (3, 4) * sqrt(62.5) / 5.
    o = np.array([[3.0, 4.0], [6.0, 8.0]])
    got, v = variance_reduction(o, np.zeros(2), 0.5)
    np.testing.assert_allclose(v, [6.25, 25.0], rtol=1e-15)
    row = np.array([3.0, 4.0]) * np.sqrt(62.5) / 5.0
    np.testing.assert_allclose(got, [row, row], rtol=1e-14)


@pytest.mark.parametrize("shape", [(48, 16), (16, 48), (32, 32)])
def test_frobenius_norm_preserved_for_any_state(shape):
    rng = np.random.default_rng(1)
    o = rng.standard_normal(shape) * rng.uniform(0.1, 3.0, size=(shape[0], 1))
    v = rng.uniform(1e-4, 1.0, size=max(shape))
    got, _ = variance_reduction(o, v, 0.9)
    np.testing.assert_allclose(np.linalg.norm(got), np.linalg.norm(o), rtol=1e-12)


@pytest.mark.parametrize("shape", [(40, 12), (12, 40)])
def test_beta2_zero_gives_equal_neuron_norms(shape):
    # The state becomes this update's own statistic, so step_size scales every
    # neuron (row of a tall matrix, column of a wide one) to unit mean square,
    # and the norm is then restored: each neuron has norm ||O|| / sqrt(count).
    rng = np.random.default_rng(2)
    o = rng.standard_normal(shape) * rng.uniform(0.1, 5.0, size=shape[0] if shape[0] >= shape[1] else shape[1])[
        (slice(None), None) if shape[0] >= shape[1] else (None, slice(None))]
    got, _ = variance_reduction(o, np.full(max(shape), 7.0), 0.0)
    axis = 1 if shape[0] >= shape[1] else 0
    count = max(shape)
    want = np.linalg.norm(o) / np.sqrt(count)
    np.testing.assert_allclose(np.linalg.norm(got, axis=axis), want, rtol=1e-12)
    # Direction of each neuron is kept.
    on = o / np.linalg.norm(o, axis=axis, keepdims=True)
    gn = got / np.linalg.norm(got, axis=axis, keepdims=True)
    np.testing.assert_allclose(gn, on, rtol=1e-12, atol=1e-15)


def test_uniform_neurons_and_state_leave_update_unchanged():
    # Orthonormal rows (all of mean square 1/cols) and a uniform state: every
    # step size is the same, and the norm ratio cancels it.
    rng = np.random.default_rng(3)
    q, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    got, _ = variance_reduction(q, np.full(24, 0.3), 0.95)
    np.testing.assert_allclose(got, q, rtol=1e-12, atol=1e-15)


def test_wide_is_the_transpose_of_tall():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((36, 10)) * rng.uniform(0.2, 2.0, size=(36, 1))
    v = rng.uniform(0.01, 1.0, size=36)
    tall, vt = variance_reduction(o, v, 0.8)
    wide, vw = variance_reduction(o.T.copy(), v, 0.8)
    np.testing.assert_allclose(wide, tall.T, rtol=1e-14)
    np.testing.assert_allclose(vw, vt, rtol=1e-15)


def test_zero_update_stays_zero():
    got, v = variance_reduction(np.zeros((8, 4)), np.zeros(8), 0.9)
    assert not np.any(got) and not np.any(v)


def _model(seed):
    rng = np.random.default_rng(seed)
    shapes = {"h0.wq": (16, 16), "h0.wfc": (64, 16), "h0.wproj": (16, 64), "wte": (32, 16), "lm_head": (32, 16)}
    w = {k: rng.standard_normal(s) * 0.02 for k, s in shapes.items()}
    g = {k: rng.standard_normal(s) * 0.01 for k, s in shapes.items()}
    return w, g


def test_step_changes_only_block_matrices_and_rescales_the_muon_update():
    w, g = _model(5)
    coeffs = [(3.4445, -4.775, 2.0315)] * 5
    m0 = {k: np.zeros_like(v) for k, v in w.items()}
    v0 = {k: np.zeros(max(v.shape)) for k, v in w.items()}
    nw, nm, nv, upd = normuon_step(w, g, m0, v0, 0.02, 0.95, 0.95, coeffs)
    _, _, mupd = muon_step(w, g, m0, 0.02, 0.95, coeffs)
    for k in ("wte", "lm_head"):
        np.testing.assert_array_equal(nw[k], w[k])
        np.testing.assert_array_equal(nv[k], v0[k])
    for k in ("h0.wq", "h0.wfc", "h0.wproj"):
        # Same norm as the plain Muon update; per-neuron rescaling of it.
        np.testing.assert_allclose(np.linalg.norm(upd[k]), np.linalg.norm(mupd[k]), rtol=1e-12)
        axis = 1 if w[k].shape[0] >= w[k].shape[1] else 0
        ratio = upd[k] / mupd[k]
        spread = np.ptp(ratio, axis=axis)
        assert np.all(spread < 1e-9 * np.abs(ratio).max())
        np.testing.assert_allclose(nw[k], w[k] - upd[k], rtol=0, atol=0)
