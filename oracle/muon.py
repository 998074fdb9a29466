"""Oracle: Muon update of the block matrices (momentum, Newton-Schulz, step).

TEST INFRASTRUCTURE ONLY (see the package header).

[CT50] "2. Otimizador Muon": the 2-D matrices are updated with momentum that is
orthogonalised by a Newton-Schulz iteration whose k-th step, with coefficients
(a, b, c), is
      A = X^T X,   B = b A + c A A,   X = a X + X B.
Embeddings and lm_head belong to the AdamW group on that page, so this update
leaves them unchanged.

Readings where the page is silent:
  * momentum is heavy-ball: M <- mu M + G, starting from M = 0;
  * the iteration starts from X = M / (||M||_F + 1e-7) with X oriented tall
    (transposed when rows < cols), and the result is transposed back;
  * the step is W <- W - lr * sqrt(max(1, rows / cols)) * X, rows = fan-out;
  * the (a, b, c) table is an input (the page truncates it after two rows).

Parity pins (tests/test_oracle_muon.py): the iteration equals the closed form
U p5(...p1(S)) V^T from an fp64 SVD; singular values of the output lie in the
band the coefficient table guarantees; both orientations agree; a zero
gradient gives a zero update.
"""
from __future__ import annotations

import numpy as np

NS_EPS = 1e-7


def newton_schulz(m, coeffs, steps=None):
    """Apply the Newton-Schulz iteration to m (any orientation); returns X."""
    coeffs = np.asarray(coeffs, dtype=np.float64)
    steps = len(coeffs) if steps is None else steps
    transposed = m.shape[0] < m.shape[1]
    x = m.T if transposed else m
    x = x / (np.linalg.norm(x) + NS_EPS)
    for a, b, c in coeffs[:steps]:
        A = x.T @ x
        Bm = b * A + c * (A @ A)
        x = a * x + x @ Bm
    return x.T if transposed else x


def newton_schulz_svd(m, coeffs, steps=None):
    """Closed form of the same map: U diag(p_k(...p_1(s))) V^T of the normalised m.

    Each step maps a singular value s to a s + b s^3 + c s^5 and keeps the
    singular vectors, because X^T X shares right singular vectors with X.
    """
    coeffs = np.asarray(coeffs, dtype=np.float64)
    steps = len(coeffs) if steps is None else steps
    x = m / (np.linalg.norm(m) + NS_EPS)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    for a, b, c in coeffs[:steps]:
        s = a * s + b * s ** 3 + c * s ** 5
    return (u * s) @ vt


def muon_scale(rows, cols):
    return max(1.0, rows / cols) ** 0.5


def muon_step(weights, grads, momentum, lr, mu, coeffs, steps=None, names=None):
    """One Muon step on the block matrices; returns (new_weights, new_momentum, updates).

    ``names`` selects the tensors (default: every tensor whose name has a layer
    prefix, i.e. the block matrices). Other tensors are copied unchanged.
    """
    if names is None:
        names = [k for k in weights if k.startswith("h") and not k.endswith((".ve", ".ve_gate"))]
    new_w = {k: v.copy() for k, v in weights.items()}
    new_m = {k: v.copy() for k, v in momentum.items()}
    updates = {}
    for k in names:
        m = mu * momentum[k] + grads[k]
        new_m[k] = m
        x = newton_schulz(m, coeffs, steps)
        rows, cols = weights[k].shape
        upd = lr * muon_scale(rows, cols) * x
        updates[k] = upd
        new_w[k] = weights[k] - upd
    return new_w, new_m, updates
