"""Pins of the AdamW oracle against closed forms that follow from the update's
definition (not from re-running it): see the oracle module header."""
import numpy as np

from oracle.adamw import adamw_step, adamw_update


def _rng_arrays(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape), rng.standard_normal(shape)


def test_first_step_is_normalised_gradient_plus_decay():
    w, g = _rng_arrays((7, 5), 0)
    lr, eps, wd = 0.01, 1e-8, 0.1
    z = np.zeros_like(w)
    w1, m1, v1 = adamw_update(w, g, z, z, 1, lr, 0.9, 0.95, eps, wd)
    # mhat = g and vhat = g^2 after one step from zero moments.
    np.testing.assert_allclose(w - w1, lr * wd * w + lr * g / (np.abs(g) + eps), rtol=1e-12, atol=0)
    # (1 - 0.95 is 0.05 only to within fp64 rounding.)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v1, 0.05 * g * g, rtol=1e-14)


def test_constant_gradient_gives_the_same_step_every_time():
    w, g = _rng_arrays((4, 6), 1)
    lr, eps = 0.003, 1e-8
    m = v = np.zeros_like(w)
    want = lr * g / (np.abs(g) + eps)
    for t in range(1, 8):
        w_new, m, v = adamw_update(w, g, m, v, t, lr, 0.8, 0.95, eps, 0.0)
        np.testing.assert_allclose(w - w_new, want, rtol=1e-9, atol=1e-15)
        w = w_new


def test_zero_betas_are_sign_descent():
    rng = np.random.default_rng(2)
    w = rng.standard_normal(50)
    m = v = np.zeros_like(w)
    for t in range(1, 4):
        g = rng.standard_normal(50)
        w_new, m, v = adamw_update(w, g, m, v, t, 0.5, 0.0, 0.0, 0.0, 0.0)
        np.testing.assert_allclose(w - w_new, 0.5 * np.sign(g), rtol=1e-14)
        w = w_new


def test_zero_gradient_with_decay_is_geometric_shrink():
    w0 = np.random.default_rng(3).standard_normal(20)
    w, m, v = w0, np.zeros(20), np.zeros(20)
    lr, wd = 0.02, 0.3
    for t in range(1, 6):
        w, m, v = adamw_update(w, np.zeros(20), m, v, t, lr, 0.9, 0.99, 1e-8, wd)
        np.testing.assert_allclose(w, w0 * (1.0 - lr * wd) ** t, rtol=1e-14)


def test_update_is_invariant_to_gradient_scale_without_eps():
    rng = np.random.default_rng(4)
    w = rng.standard_normal(30)
    gs = [rng.standard_normal(30) for _ in range(3)]
    outs = []
    for c in (1.0, 1e3):
        ww, m, v = w, np.zeros(30), np.zeros(30)
        for t, g in enumerate(gs, 1):
            ww, m, v = adamw_update(ww, c * g, m, v, t, 0.01, 0.9, 0.95, 0.0, 0.0)
        outs.append(ww)
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-12)


def test_only_embedding_and_head_change():
    rng = np.random.default_rng(5)
    weights = {k: rng.standard_normal((3, 4)) for k in ("wte", "h0.wq", "lm_head")}
    grads = {k: rng.standard_normal((3, 4)) for k in weights}
    zeros = {k: np.zeros((3, 4)) for k in ("wte", "lm_head")}
    new_w, new_m, new_v = adamw_step(weights, grads, zeros, zeros, 1, 0.1, 0.9, 0.95, 1e-8, 0.0)
    np.testing.assert_array_equal(new_w["h0.wq"], weights["h0.wq"])
    assert set(new_m) == set(new_v) == {"wte", "lm_head"}
    assert not np.array_equal(new_w["wte"], weights["wte"])


def test_scalar_tensors_join_the_adamw_group():
    from gpt_pretraining_step_bf16_amd import synthetic as syn

    w = {k: v.astype(np.float64) for k, v in syn.init_weights(2, 64, resid_scalars=True, backout=True).items()}
    rng = np.random.default_rng(5)
    g = {k: rng.standard_normal(v.shape) for k, v in w.items()}
    names = ("wte", "lm_head", "resid_lambdas", "x0_lambdas", "backout_lambda")
    z = {k: np.zeros_like(w[k]) for k in names}
    new_w, m1, _ = adamw_step(w, g, z, z, 1, 0.01, 0.9, 0.95, 1e-8, 0.0)
    for k in w:
        if k in names:
            # First step from zero moments: a normalised-gradient step.
            np.testing.assert_allclose(w[k] - new_w[k], 0.01 * g[k] / (np.abs(g[k]) + 1e-8), rtol=1e-9)
            assert k in m1
        else:
            np.testing.assert_array_equal(new_w[k], w[k])
