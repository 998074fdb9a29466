"""Oracle: NorMuon variance reduction of the orthogonalised Muon update.

TEST INFRASTRUCTURE ONLY (see the package header).

[CT50] "2. Otimizador Muon", the NorMuon paragraph after the Polar Express
iteration: the orthogonalised update O gets a per-neuron second moment, the
mean of O^2 along one dimension; v_norm is the square root of the sum of those
means; the update is multiplied by step_size * v_norm / max(v_norm_new, 1e-10).

The page prints only that fragment. Readings taken where it stops short:
  * O is the Newton-Schulz output in the stored orientation of the weight;
  * the mean runs over the shorter side (over columns when rows >= cols), so
    there is one statistic per element of the longer side: per output row of
    a square or tall matrix, per column of a wide one;
  * the statistic feeds an exponential moving average state
    v <- beta2 v + (1 - beta2) v_mean, zero before the first step, fp32 on
    the device; step_size = 1 / sqrt(max(v, 1e-10)) per neuron;
  * v_norm_new is v_norm of the rescaled update O * step_size, i.e.
    sqrt(sum v_mean * step_size^2); so the result has the Frobenius norm of O
    and only the split of that norm between neurons changes;
  * the Muon step then uses the rescaled update in place of O:
    W <- W - lr * sqrt(max(1, rows / cols)) * O'.

Parity pins (tests/test_oracle_normuon.py): a worked 2x2 example computed by
hand; Frobenius norm preserved for any state; with beta2 = 0 every neuron of
the result has the same norm, in closed form; equal neuron norms and a uniform
state leave O unchanged; wide and tall orientations agree under transposition;
a zero update stays zero; only block matrices change.
"""
from __future__ import annotations

import numpy as np

from .muon import muon_scale, newton_schulz

NORMUON_FLOOR = 1e-10


def normuon_axis(rows, cols):
    """Axis the second moment averages over: the shorter side."""
    return 1 if rows >= cols else 0


def normuon_state_len(rows, cols):
    return max(rows, cols)


def variance_reduction(o, v, beta2):
    """Rescale the orthogonalised update o; returns (o', new state v).

    v holds one value per element of o's longer side.
    """
    axis = normuon_axis(*o.shape)
    v_mean = np.mean(o * o, axis=axis)
    v_norm = np.sqrt(np.sum(v_mean))
    v_new = beta2 * v + (1.0 - beta2) * v_mean
    step_size = 1.0 / np.sqrt(np.maximum(v_new, NORMUON_FLOOR))
    v_norm_new = np.sqrt(np.sum(v_mean * step_size ** 2))
    final = step_size * (v_norm / max(v_norm_new, NORMUON_FLOOR))
    scaled = o * (final[:, None] if axis == 1 else final[None, :])
    return scaled, v_new


def normuon_step(weights, grads, momentum, second_moment, lr, mu, beta2, coeffs, steps=None,
                 names=None):
    """One Muon step with NorMuon variance reduction on the block matrices.

    Returns (new_weights, new_momentum, new_second_moment, updates). Tensors
    not in ``names`` (default: the block matrices, names with a layer prefix)
    are copied unchanged.
    """
    if names is None:
        names = [k for k in weights if k.startswith("h") and not k.endswith((".ve", ".ve_gate"))]
    new_w = {k: v.copy() for k, v in weights.items()}
    new_m = {k: v.copy() for k, v in momentum.items()}
    new_v = {k: v.copy() for k, v in second_moment.items()}
    updates = {}
    for k in names:
        m = mu * momentum[k] + grads[k]
        new_m[k] = m
        o = newton_schulz(m, coeffs, steps)
        o, new_v[k] = variance_reduction(o, second_moment[k], beta2)
        rows, cols = weights[k].shape
        upd = lr * muon_scale(rows, cols) * o
        updates[k] = upd
        new_w[k] = weights[k] - upd
    return new_w, new_m, new_v, updates
