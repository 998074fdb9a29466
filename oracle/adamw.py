"""Oracle: AdamW update of the embedding and unembedding tables.

TEST INFRASTRUCTURE ONLY (see the package header).

[CT50] "2. Otimizador Muon" splits the parameters: the 2-D block matrices take
Muon, while the embeddings and lm_head (and scalar factors, which this model
does not have) take AdamW. The page names the optimizer and nothing more.

Readings where the page is silent:
  * AdamW is the decoupled-weight-decay Adam of Loshchilov and Hutter, in the
    form PyTorch implements (nanochat is a PyTorch program): with g the
    gradient, t >= 1 the 1-based step count,
        m <- beta1 m + (1 - beta1) g
        v <- beta2 v + (1 - beta2) g^2
        mhat = m / (1 - beta1^t),  vhat = v / (1 - beta2^t)
        w <- w - lr * wd * w - lr * mhat / (sqrt(vhat) + eps)
    (the decay is scaled by lr and uses the weights before the step);
  * lr, beta1, beta2, eps and wd are arguments: the page fixes none of them;
  * the moments start at zero and are kept per element in the parameter's
    shape.

Parity pins (tests/test_oracle_adamw.py): the first step from zero moments is
lr * g / (|g| + eps) plus the decay term; a gradient held constant gives that
same step every time (the bias corrections cancel the moment ramp exactly);
beta1 = beta2 = 0 gives sign descent at every step; zero gradients with decay
shrink w by (1 - lr wd) per step; with eps = 0 the update does not change when
every gradient is scaled by a positive constant.
"""
from __future__ import annotations

import numpy as np

ADAMW_TENSORS = ("wte", "lm_head")


def adamw_update(w, g, m, v, step, lr, beta1, beta2, eps, wd):
    """One AdamW step of one tensor; returns (new w, new m, new v)."""
    if step < 1:
        raise ValueError("step is 1-based")
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * (g * g)
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    w = w - lr * wd * w - lr * mhat / (np.sqrt(vhat) + eps)
    return w, m, v


SCALAR_TENSORS = ("resid_lambdas", "x0_lambdas", "backout_lambda", "smear_gate", "smear_lambda")


def adamw_step(weights, grads, exp_avg, exp_avg_sq, step, lr, beta1, beta2, eps, wd):
    """AdamW on wte, lm_head, the value embeddings and their gates, and the
    scalar tensors the model has ([CT50] "2. Otimizador Muon": embeddings and
    scalars are in the AdamW group; the small value-embedding gates join them
    here); every other tensor is copied unchanged.

    exp_avg / exp_avg_sq are dicts holding the moments of those tensors.
    Returns (new weights, new exp_avg, new exp_avg_sq).
    """
    new_w = {k: v.copy() for k, v in weights.items()}
    new_m, new_v = {}, {}
    group = ADAMW_TENSORS + tuple(k for k in weights if k.endswith((".ve", ".ve_gate")))
    for k in group + tuple(t for t in SCALAR_TENSORS if t in weights):
        new_w[k], new_m[k], new_v[k] = adamw_update(weights[k], grads[k], exp_avg[k], exp_avg_sq[k],
                                                    step, lr, beta1, beta2, eps, wd)
    return new_w, new_m, new_v
