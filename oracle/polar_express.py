"""Oracle: greedy minimax construction of Newton-Schulz coefficient triples.

TEST INFRASTRUCTURE ONLY (see the package header).

[CT50] "2. Otimizador Muon" labels the coefficient table "Polar Express" with
five iterations and prints only the first two (a, b, c) triples. Each triple
defines an odd quintic p(s) = a s + b s^3 + c s^5 acting on singular values.
The Polar Express construction (Amsel, Persson, Musco and Gower, 2025) picks,
step by step, the odd quintic that minimises max |1 - p(s)| over the interval
the previous steps leave. Here that rule is solved as a linear program on a
dense grid and continued after the two printed triples, starting from singular
values in [1e-3, 1].

Parity: the derived rows are a reading of a truncated table; whether they equal
the original project's rows 3-5 is unpinned. The test pins what the rule itself
fixes: equioscillation (the image is [1 - E, 1 + E]) and the final band.
"""
from __future__ import annotations

import numpy as np


def odd_quintic(coef, s):
    a, b, c = coef
    return a * s + b * s ** 3 + c * s ** 5


def image_interval(coef, lo, hi, n=200001):
    s = np.linspace(lo, hi, n)
    p = odd_quintic(coef, s)
    return float(p.min()), float(p.max())


def minimax_quintic(lo, hi, n=4001):
    """Odd quintic minimising max |1 - p(s)| on a grid of [lo, hi]; returns (coef, E)."""
    from scipy.optimize import linprog

    s = np.linspace(lo, hi, n)
    basis = np.stack([s, s ** 3, s ** 5], axis=1)
    ones = np.ones((n, 1))
    # Variables (a, b, c, E); minimise E subject to |1 - basis @ abc| <= E.
    a_ub = np.vstack([np.hstack([-basis, -ones]), np.hstack([basis, -ones])])
    b_ub = np.concatenate([-np.ones(n), np.ones(n)])
    res = linprog([0, 0, 0, 1], A_ub=a_ub, b_ub=b_ub,
                  bounds=[(None, None)] * 3 + [(0, None)], method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    return res.x[:3], float(res.x[3])


def greedy_minimax_triples(printed, total=5, lo=1e-3, hi=1.0):
    """Apply the printed triples to [lo, hi], then append greedy minimax triples.

    Returns (table [total, 3], list of (lo, hi) images after each step).
    """
    table = [tuple(map(float, t)) for t in printed]
    images = []
    for coef in table:
        lo, hi = image_interval(coef, lo, hi)
        images.append((lo, hi))
    while len(table) < total:
        coef, _err = minimax_quintic(lo, hi)
        table.append(tuple(map(float, coef)))
        lo, hi = image_interval(coef, lo, hi)
        images.append((lo, hi))
    return np.array(table), images
