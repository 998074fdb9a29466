"""Oracle: forward pass, loss and hand-written reverse-mode gradients of the GPT.

TEST INFRASTRUCTURE ONLY (see the package header).

What is computed, following [CT50] "1. Modelo GPT" and "3. Gerenciamento de
Precisão" (architecture list and the bias-free Linear), with the readings where
the page is silent:

  x   = wte[tokens]                                   (untied input table)
  per layer:
    xn  = rms(x)                                      (pre-norm, no gain)
    q,k,v = xn Wq^T, xn Wk^T, xn Wv^T, split into 128-wide heads
    q,k = rope(rms(q)), rope(rms(k))                  (QK-norm per head, then RoPE)
    o   = causal softmax(q k^T / sqrt(128)) v        (optionally windowed per layer)
    x   = x + o Wo^T
    x   = x + relu(rms(x) Wfc^T)^2 Wproj^T            (ReLU^2 MLP)
  z    = rms(x) Wlm^T                                 (final norm, untied head)
  loss = mean over valid targets of (logsumexp(z) - z[target])

Readings (the pages do not print these): RMSNorm eps = 1e-6 with statistics
over the last axis; RoPE pairs element j with j+64, angle t * 10000^(-j/64),
positions restart at 0 for every row; no biases, no softcap, no dropout;
targets equal to -1 are ignored in the mean.

The backward pass is derived by hand per operation (no autodiff library), so
the finite-difference tests in tests/ check it against the forward pass.

Window attention (optional, per layer): the pages list alternating short and
long attention windows but give no sizes, so the windows are an input; a
window W lets query i see keys i - W .. i.

Residual scalars (optional): with tensors resid_lambdas and x0_lambdas [1, L],
block i reads resid_lambdas[i] * x + x0_lambdas[i] * x0 (x0 the embedding
output) as its input stream; with backout_lambda [1, 1] and a backout layer k,
backout_lambda times the stream entering block k is subtracted before the
final norm. The pages print these two lines and nothing around them.

Smear (optional): with tensors smear_gate [1, 24] and smear_lambda [1, 1] the
embedding output becomes x_t + smear_lambda * sigmoid(smear_gate . x_t[:24])
* x_(t-1) (zero before a sequence's first token); this is the x0 that the
residual scalars mix in.

Value embeddings (optional, per layer): with tensors h{i}.ve [V, Hkv*128]
and h{i}.ve_gate [Hkv, 32], block i adds to v, per key/value head, the
token's table row gated by 3 * sigmoid(ve_gate . xn[:32]), xn being the
block's normalised input (the input of its QKV projection).

Grouped-query attention (optional): the pages list "fewer KV heads". When wk
and wv have Hkv * 128 rows (Hkv dividing H), query head h attends with key and
value head h // (H / Hkv); QK-norm and RoPE act per head as before.

Parity pins (tests/test_oracle_model.py): central finite differences in fp64 on
depth-1 and depth-2 models (one with a windowed layer); loss = ln V and a
closed-form lm_head gradient for a zero unembedding; causal invariance;
attention closed forms (T = 1, q = 0, window 0 returns v); a window equals
causal attention over the trailing slice; a window covering the sequence is
the causal mask; RMSNorm / RoPE invariants; cross-entropy row sums;
embedding-gradient support.
"""
from __future__ import annotations

import numpy as np

EPS_NORM = 1e-6
ROPE_BASE = 10000.0
HEAD_DIM = 128


# ----------------------------------------------------------------------------
# Elementary operations and their adjoints
# ----------------------------------------------------------------------------
def rms_norm(x, eps=EPS_NORM):
    """y = x / sqrt(mean(x^2) + eps) over the last axis; returns (y, rstd)."""
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * rstd, rstd


def rms_norm_bwd(dy, y, rstd):
    """Adjoint of rms_norm: dx = rstd * (dy - y * mean(dy * y))."""
    return rstd * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(seq, head_dim=HEAD_DIM, base=ROPE_BASE, dtype=np.float64):
    """cos/sin of angle t * base^(-j/half) for t < seq, j < head_dim / 2."""
    half = head_dim // 2
    theta = base ** (-np.arange(half, dtype=np.float64) / half)
    phi = np.arange(seq, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(phi).astype(dtype), np.sin(phi).astype(dtype)


def rope(x, cos, sin):
    """Rotate pairs (j, j + half) of x [T, H, hd] by the per-position angle."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_bwd(dy, cos, sin):
    """Adjoint of rope: rotation by the opposite angle."""
    half = dy.shape[-1] // 2
    d1, d2 = dy[..., :half], dy[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def _repeat_kv(x, heads):
    """Grouped-query attention ([CT50] "1. Modelo GPT": fewer key/value heads):
    with Hkv key/value heads, query head h reads key/value head h // (H / Hkv)."""
    hkv = x.shape[1]
    return x if hkv == heads else np.repeat(x, heads // hkv, axis=1)


def _sum_kv_groups(dx, hkv):
    """Adjoint of _repeat_kv: sum the gradients of each group of query heads."""
    T, H, hd = dx.shape
    return dx if hkv == H else dx.reshape(T, hkv, H // hkv, hd).sum(axis=2)


def causal_attention(q, k, v, window=None):
    """Softmax attention with mask j <= i; q is [T, H, hd], k and v [T, Hkv, hd]
    with Hkv dividing H (grouped-query attention when Hkv < H).

    With a window W (an int >= 0) key j is visible to query i only when
    i - W <= j <= i as well ([CT50] "1. Modelo GPT" lists short/long window
    attention, and "5. Flash Attention Unificado" passes a window_size to the
    attention call; W keys to the left of the query plus the query itself).
    None is the plain causal mask.
    Returns o [T, H, hd] and the probabilities P [H, T, T].
    """
    T, H, hd = q.shape
    k, v = _repeat_kv(k, H), _repeat_kv(v, H)
    scale = 1.0 / np.sqrt(hd)
    qh, kh, vh = (a.transpose(1, 0, 2) for a in (q, k, v))  # [H, T, hd]
    s = np.matmul(qh, kh.transpose(0, 2, 1)) * scale
    mask = np.tril(np.ones((T, T), dtype=bool))
    if window is not None:
        mask &= np.triu(np.ones((T, T), dtype=bool), -int(window))
    s = np.where(mask[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    o = np.matmul(p, vh).transpose(1, 0, 2)
    return o, p


def causal_attention_bwd(do, q, k, v, p):
    """Adjoint of causal_attention given the saved probabilities p; dk and dv
    have k's and v's head count."""
    hd = q.shape[-1]
    hkv = k.shape[1]
    k, v = _repeat_kv(k, q.shape[1]), _repeat_kv(v, q.shape[1])
    scale = 1.0 / np.sqrt(hd)
    qh, kh, vh, doh = (a.transpose(1, 0, 2) for a in (q, k, v, do))
    dp = np.matmul(doh, vh.transpose(0, 2, 1))
    dv = np.matmul(p.transpose(0, 2, 1), doh)
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    dq = np.matmul(ds, kh) * scale
    dk = np.matmul(ds.transpose(0, 2, 1), qh) * scale
    return (dq.transpose(1, 0, 2), _sum_kv_groups(dk.transpose(1, 0, 2), hkv),
            _sum_kv_groups(dv.transpose(1, 0, 2), hkv))


def _head_pool():
    """Threads for the per-head loops: heads are independent, and NumPy
    releases the interpreter lock inside its array operations, so running
    heads side by side changes no arithmetic, only wall time."""
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os

        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


_POOL = None


def attention_by_head(q, k, v, window=None):
    """causal_attention one query head at a time (query head h with key/value
    head h // (H / Hkv)), so that only one head's T x T probabilities exist per
    worker; returns o [T, H, hd]."""
    T, H, hd = q.shape
    g = H // k.shape[1]
    o = np.empty_like(q)

    def head(h):
        o[:, h:h + 1], _ = causal_attention(q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1], window)

    list(_head_pool().map(head, range(H)))
    return o


def attention_by_head_bwd(do, q, k, v, window=None):
    """Adjoint of attention_by_head: per query head, the probabilities are
    recomputed (causal_attention) and causal_attention_bwd applied; the key and
    value gradients of the query heads that share a key/value head are then
    summed in head order."""
    T, H, hd = q.shape
    g = H // k.shape[1]

    def head(h):
        qh, kh, vh = q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1]
        _, p = causal_attention(qh, kh, vh, window)
        return causal_attention_bwd(do[:, h:h + 1], qh, kh, vh, p)

    per_head = list(_head_pool().map(head, range(H)))
    dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
    for h, (dqh, dkh, dvh) in enumerate(per_head):
        dq[:, h:h + 1] = dqh
        dk[:, h // g:h // g + 1] += dkh
        dv[:, h // g:h // g + 1] += dvh
    return dq, dk, dv


def log_softmax_rows(z):
    """Row-wise logsumexp of z [T, V]."""
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[:, 0]


# ----------------------------------------------------------------------------
# Model
# ----------------------------------------------------------------------------
def _depth(weights):
    n = 0
    while f"h{n}.wq" in weights:
        n += 1
    return n


def _layer_window(windows, layer):
    return None if windows is None else windows[layer]


def _scalars(weights):
    """Per-layer residual scalars and the backout scalar, when the model has them."""
    rl = weights["resid_lambdas"][0] if "resid_lambdas" in weights else None
    xl = weights["x0_lambdas"][0] if "x0_lambdas" in weights else None
    bl = float(weights["backout_lambda"][0, 0]) if "backout_lambda" in weights else None
    return rl, xl, bl


SMEAR_CHANNELS = 24
VE_GATE_CHANNELS = 32


def _smear(x, weights):
    """Smear ([CT50] "Truques de Eficiência", item 2: mix in the previous
    token's embedding): gate_t = smear_lambda * sigmoid(smear_gate . x_t[:24]),
    y_t = x_t + gate_t * x_(t-1), with x_(-1) = 0 (the first token of a
    sequence has no previous one). Returns y and the saved (gate logits)."""
    w = weights["smear_gate"][0]
    lam = float(weights["smear_lambda"][0, 0])
    a = x[:, :SMEAR_CHANNELS] @ w
    prev = np.concatenate([np.zeros_like(x[:1]), x[:-1]], axis=0)
    g = lam / (1.0 + np.exp(-a))
    return x + g[:, None] * prev, a


def _smear_bwd(dy, x, a, weights, grads, sc=None):
    """Adjoint of _smear: returns dx and adds the gate's gradients (and, with
    sc, the Cauchy-Schwarz bounds of the sums that form them)."""
    w = weights["smear_gate"][0]
    lam = float(weights["smear_lambda"][0, 0])
    sig = 1.0 / (1.0 + np.exp(-a))
    prev = np.concatenate([np.zeros_like(x[:1]), x[:-1]], axis=0)
    s = np.sum(dy * prev, axis=1)             # d loss / d gate_t
    grads["smear_lambda"][0, 0] += float(np.sum(sig * s))
    c = lam * sig * (1.0 - sig) * s           # d loss / d a_t
    grads["smear_gate"][0] += c @ x[:, :SMEAR_CHANNELS]
    if sc is not None:
        bound = np.linalg.norm(dy, axis=1) * np.linalg.norm(prev, axis=1)
        sc["smear_lambda"][0, 0] += float(np.sum(sig * bound))
        sc["smear_gate"][0] += (np.abs(lam) * sig * (1.0 - sig) * bound) @ np.abs(x[:, :SMEAR_CHANNELS])
    g = lam * sig
    dx = dy.copy()
    dx[:-1] += g[1:, None] * dy[1:]           # x_t is the previous token of t + 1
    dx[:, :SMEAR_CHANNELS] += c[:, None] * w[None, :]
    return dx


def _forward_sequence(weights, tok, cos, sin, windows=None, backout_layer=None):
    """Forward pass of one sequence; returns the logits and the saved values.

    windows: None, or one attention window per layer (an int, or None for the
    full causal context).
    Residual scalars ([CT50] "Truques de Eficiência", items 1 and 3), when the
    weights hold them: before block i the stream becomes
    resid_lambdas[i] * x + x0_lambdas[i] * x0, x0 being the embedding output;
    with backout_layer k, the stream entering block k (after its mix) is kept
    and backout_lambda times it is subtracted before the final norm.
    """
    L = _depth(weights)
    wte = weights["wte"]
    d = wte.shape[1]
    H = d // HEAD_DIM
    T = tok.shape[0]
    rl, xl, bl = _scalars(weights)
    x = wte[tok]
    x_emb, smear_a = x, None
    if "smear_gate" in weights:
        x, smear_a = _smear(x, weights)
    x0 = x
    x_backout = None
    layers = []
    for layer in range(L):
        w = {n: weights[f"h{layer}.{n}"] for n in ("wq", "wk", "wv", "wo", "wfc", "wproj")}
        x_prev = x
        if rl is not None:
            x = rl[layer] * x + xl[layer] * x0
        if backout_layer == layer:
            x_backout = x
        xn1, r1 = rms_norm(x)
        q = (xn1 @ w["wq"].T).reshape(T, H, HEAD_DIM)
        k = (xn1 @ w["wk"].T).reshape(T, -1, HEAD_DIM)
        v = (xn1 @ w["wv"].T).reshape(T, -1, HEAD_DIM)
        ve_name = f"h{layer}.ve"
        ve_logit = None
        if ve_name in weights:
            # Value embeddings ([CT50] "Embeddings de Valor (ResFormer)"): a
            # per-layer table row of the token, gated per key/value head by
            # 3 sigmoid(ve_gate . xn1[:32]), is added to v.
            ve = weights[ve_name][tok].reshape(T, -1, HEAD_DIM)
            ve_logit = xn1[:, :VE_GATE_CHANNELS] @ weights[f"h{layer}.ve_gate"].T
            v = v + (3.0 / (1.0 + np.exp(-ve_logit)))[:, :, None] * ve
        qn, rq = rms_norm(q)
        kn, rk = rms_norm(k)
        qr, kr = rope(qn, cos, sin), rope(kn, cos, sin)
        o = attention_by_head(qr, kr, v, _layer_window(windows, layer))
        o2 = o.reshape(T, d)
        x_mid = x + o2 @ w["wo"].T
        xn2, r2 = rms_norm(x_mid)
        u = xn2 @ w["wfc"].T
        a = np.maximum(u, 0.0) ** 2
        x = x_mid + a @ w["wproj"].T
        layers.append(dict(xn1=xn1, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, qr=qr, kr=kr,
                           v=v, o2=o2, xn2=xn2, r2=r2, u=u, a=a, x_prev=x_prev, ve_logit=ve_logit))
    if backout_layer is not None:
        x = x - bl * x_backout
    xnf, rf = rms_norm(x)
    z = xnf @ weights["lm_head"].T
    return z, dict(layers=layers, xnf=xnf, rf=rf, x0=x0, x_backout=x_backout, x_emb=x_emb, smear_a=smear_a)


def forward_logits(weights, tokens, windows=None, backout_layer=None):
    """Logits [B, T, V] for int tokens [B, T] (no loss, no gradients)."""
    tokens = np.asarray(tokens)
    T = tokens.shape[1]
    dt = weights["wte"].dtype
    cos, sin = rope_tables(T, dtype=dt)
    return np.stack([_forward_sequence(weights, tokens[b], cos, sin, windows, backout_layer)[0]
                     for b in range(tokens.shape[0])])


def _cs(a, b):
    """Cauchy-Schwarz bound of sum(a * b): sum over rows of |a_row| |b_row|."""
    return float(np.sum(np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1)))


def forward_backward(weights, tokens, targets, want_grads=True, windows=None, backout_layer=None,
                     scalar_scales=None):
    """Mean cross-entropy loss and the gradient of every tensor.

    windows: None, or one attention window per layer (see causal_attention).
    backout_layer: the layer whose input stream the backout subtracts (the
    weights then hold backout_lambda); residual scalars apply when the weights
    hold resid_lambdas and x0_lambdas (see _forward_sequence).
    scalar_scales: optional dict; for each scalar tensor and value-embedding
    gate it receives, shaped like the tensor, the Cauchy-Schwarz bound of the
    sum that forms its gradient (a tolerance scale for comparisons; not part
    of the step).

    Sequences are independent, so the batch is processed one row at a time and
    the per-row contributions are summed (this bounds memory; it is exact).
    Returns (loss, grads) with grads a dict shaped like ``weights``.
    """
    tokens = np.asarray(tokens)
    targets = np.asarray(targets)
    B, T = tokens.shape
    dt = weights["wte"].dtype
    cos, sin = rope_tables(T, dtype=dt)
    n_valid = int(np.count_nonzero(targets >= 0))
    grads = {k: np.zeros_like(v) for k, v in weights.items()} if want_grads else None
    loss_sum = 0.0
    L = _depth(weights)
    d = weights["wte"].shape[1]
    H = d // HEAD_DIM
    for b in range(B):
        tok, tgt = tokens[b], targets[b]
        z, c = _forward_sequence(weights, tok, cos, sin, windows, backout_layer)
        lse = log_softmax_rows(z)
        valid = tgt >= 0
        t = np.where(valid, tgt, 0)
        rows = np.arange(T)
        loss_sum += float(np.sum(np.where(valid, lse - z[rows, t], 0.0)))
        if not want_grads or n_valid == 0:
            continue
        # Cross-entropy: d loss / d z = (softmax(z) - onehot(target)) / n_valid.
        dz = np.exp(z - lse[:, None])
        dz[rows, t] -= 1.0
        dz *= (valid.astype(dt) / n_valid)[:, None]
        grads["lm_head"] += dz.T @ c["xnf"]
        dx = rms_norm_bwd(dz @ weights["lm_head"], c["xnf"], c["rf"])
        rl, xl, bl = _scalars(weights)
        sc = scalar_scales
        if sc is not None:
            for k in ("resid_lambdas", "x0_lambdas", "backout_lambda", "smear_gate", "smear_lambda"):
                if k in weights:
                    sc.setdefault(k, np.zeros_like(weights[k]))
        if backout_layer is not None:
            # x_final = x_L - bl * x_backout
            grads["backout_lambda"][0, 0] -= float(np.sum(dx * c["x_backout"]))
            if sc is not None:
                sc["backout_lambda"][0, 0] += _cs(dx, c["x_backout"])
            d_backout = -bl * dx
        dx0 = np.zeros_like(dx)
        for layer in reversed(range(L)):
            s = c["layers"][layer]
            w = {n: weights[f"h{layer}.{n}"] for n in ("wq", "wk", "wv", "wo", "wfc", "wproj")}
            g = {n: f"h{layer}.{n}" for n in w}
            # x_out = x_mid + relu(u)^2 Wproj^T
            grads[g["wproj"]] += dx.T @ s["a"]
            da = dx @ w["wproj"]
            du = da * 2.0 * np.maximum(s["u"], 0.0)
            grads[g["wfc"]] += du.T @ s["xn2"]
            dx_mid = dx + rms_norm_bwd(du @ w["wfc"], s["xn2"], s["r2"])
            # x_mid = x_in + o Wo^T
            grads[g["wo"]] += dx_mid.T @ s["o2"]
            do = (dx_mid @ w["wo"]).reshape(T, H, HEAD_DIM)
            # The probabilities are recomputed from the saved q, k, one head at
            # a time (the forward's definition; keeping them would need H T^2
            # values per layer).
            dqr, dkr, dv = attention_by_head_bwd(do, s["qr"], s["kr"], s["v"], _layer_window(windows, layer))
            dq = rms_norm_bwd(rope_bwd(dqr, cos, sin), s["qn"], s["rq"]).reshape(T, d)
            dk = rms_norm_bwd(rope_bwd(dkr, cos, sin), s["kn"], s["rk"]).reshape(T, -1)
            dxn1_ve = 0.0
            if s["ve_logit"] is not None:
                # v = v_proj + gate * ve, gate = 3 sigmoid(logit), logit = xn1[:32] . ve_gate
                ve_name = f"h{layer}.ve"
                ve = weights[ve_name][tok].reshape(T, -1, HEAD_DIM)
                sig = 1.0 / (1.0 + np.exp(-s["ve_logit"]))
                np.add.at(grads[ve_name], tok, (3.0 * sig[:, :, None] * dv).reshape(T, -1))
                dlogit = 3.0 * sig * (1.0 - sig) * np.sum(dv * ve, axis=-1)   # [T, Hkv]
                grads[f"h{layer}.ve_gate"] += dlogit.T @ s["xn1"][:, :VE_GATE_CHANNELS]
                if scalar_scales is not None:
                    bound = 3.0 * sig * (1.0 - sig) * np.linalg.norm(dv, axis=-1) * np.linalg.norm(ve, axis=-1)
                    sk = scalar_scales.setdefault(f"h{layer}.ve_gate", np.zeros_like(weights[f"h{layer}.ve_gate"]))
                    sk += bound.T @ np.abs(s["xn1"][:, :VE_GATE_CHANNELS])
                dxn1_ve = np.zeros_like(s["xn1"])
                dxn1_ve[:, :VE_GATE_CHANNELS] = dlogit @ weights[f"h{layer}.ve_gate"]
            dv = dv.reshape(T, -1)
            grads[g["wq"]] += dq.T @ s["xn1"]
            grads[g["wk"]] += dk.T @ s["xn1"]
            grads[g["wv"]] += dv.T @ s["xn1"]
            dxn1 = dq @ w["wq"] + dk @ w["wk"] + dv @ w["wv"] + dxn1_ve
            dx = dx_mid + rms_norm_bwd(dxn1, s["xn1"], s["r1"])
            # dx is now the gradient of the stream entering block `layer`.
            if backout_layer == layer:
                dx = dx + d_backout
            if rl is not None:
                # x_in = rl * x_prev + xl * x0
                grads["resid_lambdas"][0, layer] += float(np.sum(dx * s["x_prev"]))
                grads["x0_lambdas"][0, layer] += float(np.sum(dx * c["x0"]))
                if sc is not None:
                    sc["resid_lambdas"][0, layer] += _cs(dx, s["x_prev"])
                    sc["x0_lambdas"][0, layer] += _cs(dx, c["x0"])
                dx0 += xl[layer] * dx
                dx = rl[layer] * dx
        dx = dx + dx0
        if "smear_gate" in weights:
            dx = _smear_bwd(dx, c["x_emb"], c["smear_a"], weights, grads, sc)
        np.add.at(grads["wte"], tok, dx)
    loss = loss_sum / n_valid if n_valid else 0.0
    return loss, grads
