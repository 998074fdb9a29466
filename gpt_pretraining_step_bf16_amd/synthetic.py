"""Seeded synthetic inputs for one pretraining step of the depth-parameterised GPT.

This module is the only code shared by the HIP path and the oracle: it draws
inputs and holds the workload table. It contains none of the step's arithmetic.

Sources (cited by page title and section):
  [CT50]  dev.to, "Como treinar seu próprio ChatGPT por 50 dólares".
  [HADA]  GeekNews (hada.io) summary of the nanochat launch README.

* Shapes come from one depth knob ([CT50] "Filosofia: Um Único Seletor Para
  Controlar Tudo"). The pages do not print the rule; the reading used here is
  width = 64 * depth rounded up to a multiple of the 128-wide head, heads =
  width / 128, MLP hidden = 4 * width.
* Vocabulary 32768 comes from the BPE tokenizer row of [CT50] "O Que o nanochat
  Abrange". The training text and tokenizer are not available, so token ids are
  drawn from a truncated Zipf(s=1.1) law over the vocabulary, as a head-heavy
  stand-in for tokenised web text; targets are the ids shifted by one.
* Weights are N(0, 0.02^2), drawn in float32 in canonical tensor order.
* The Newton-Schulz coefficient table is an input of Muon ([CT50] "2. Otimizador
  Muon"): the page prints the first two triples and truncates the rest. The last
  three triples are this build's reading: the greedy minimax (Polar Express)
  construction continued over the interval the first two leave. They are plain
  data here; the oracle re-derives them independently in its tests.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128

# Workloads: (depth, vocab, seq, microbatch). "tiny" is the small case the
# oracle finishes in seconds; d20 is the headline single-GPU configuration.
CONFIGS = {
    "tiny": dict(depth=2, vocab=2048, seq=64, batch=2),
    "d12": dict(depth=12, vocab=32768, seq=2048, batch=8),
    "d20": dict(depth=20, vocab=32768, seq=2048, batch=32),
    "d26": dict(depth=26, vocab=32768, seq=2048, batch=16),
    "d32": dict(depth=32, vocab=32768, seq=4096, batch=4),
}

# Newton-Schulz (a, b, c) triples, five iterations. Rows 1-2: printed on the
# page. Rows 3-5: greedy minimax continuation (reading stated in the header).
NS_COEFFS = np.array(
    [
        [8.156, -22.483, 15.879],
        [4.043, -2.809, 0.500],
        [3.982257, -2.970416, 0.565427],
        [3.335133, -2.500934, 0.511459],
        [2.315341, -1.682053, 0.420229],
    ],
    dtype=np.float64,
)

MUON_MOMENTUM = 0.95
MUON_LR = 0.02
INIT_STD = 0.02
ZIPF_S = 1.1


def model_dims(depth: int) -> dict:
    """Width, heads and MLP size from the depth knob (reading stated above)."""
    if depth < 1:
        raise ValueError("depth must be >= 1")
    d = HEAD_DIM * ((64 * depth + HEAD_DIM - 1) // HEAD_DIM)
    return dict(depth=depth, d=d, heads=d // HEAD_DIM, mlp=4 * d)


def tensor_specs(depth: int, vocab: int, kv_heads=None, resid_scalars=False, backout=False, smear=False,
                 ve_layers=()):
    """Canonical tensor order: wte; per layer wq, wk, wv, wo, wfc, wproj; lm_head;
    then, for each layer i in ve_layers (ascending), the value embedding
    h{i}.ve [vocab, kv_heads*128] and its gate h{i}.ve_gate [kv_heads, 32]; then
    the optional scalar tensors resid_lambdas [1, depth], x0_lambdas [1, depth],
    backout_lambda [1, 1], smear_gate [1, 24] and smear_lambda [1, 1].

    Each entry is (name, rows, cols, kind, layer) with kind in
    {"emb", "matrix", "lm_head", "scalar"}; matrices are [out, in] as in a
    Linear layer. kv_heads (default: every head) sets the rows of wk and wv to
    kv_heads * 128 (grouped-query attention).
    """
    dm = model_dims(depth)
    d, f = dm["d"], dm["mlp"]
    dkv = d if kv_heads is None else HEAD_DIM * int(kv_heads)
    specs = [("wte", vocab, d, "emb", -1)]
    for layer in range(depth):
        specs += [
            (f"h{layer}.wq", d, d, "matrix", layer),
            (f"h{layer}.wk", dkv, d, "matrix", layer),
            (f"h{layer}.wv", dkv, d, "matrix", layer),
            (f"h{layer}.wo", d, d, "matrix", layer),
            (f"h{layer}.wfc", f, d, "matrix", layer),
            (f"h{layer}.wproj", d, f, "matrix", layer),
        ]
    specs.append(("lm_head", vocab, d, "lm_head", -1))
    for layer in sorted(ve_layers):
        specs += [(f"h{layer}.ve", vocab, dkv, "emb", layer),
                  (f"h{layer}.ve_gate", dkv // HEAD_DIM, 32, "gate", layer)]
    if resid_scalars:
        specs += [("resid_lambdas", 1, depth, "scalar", -1), ("x0_lambdas", 1, depth, "scalar", -1)]
    if backout:
        specs.append(("backout_lambda", 1, 1, "scalar", -1))
    if smear:
        specs += [("smear_gate", 1, 24, "scalar", -1), ("smear_lambda", 1, 1, "scalar", -1)]
    return specs


# Start values of the scalar tensors: the plain residual stream (no x0 mix, no
# backout). The pages give none; tests set other values explicitly.
SCALAR_INIT = {"resid_lambdas": 1.0, "x0_lambdas": 0.0, "backout_lambda": 0.0, "smear_gate": 0.0,
               "smear_lambda": 0.0}


def init_weights(depth: int, vocab: int, seed: int = 0, std: float = INIT_STD, kv_heads=None,
                 resid_scalars=False, backout=False, smear=False, ve_layers=()) -> dict:
    """Every matrix N(0, std^2), float32, drawn in canonical order from one seed;
    scalar tensors take SCALAR_INIT (no draw)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, rows, cols, kind, _layer in tensor_specs(depth, vocab, kv_heads, resid_scalars, backout, smear,
                                                       ve_layers):
        if kind == "scalar":
            out[name] = np.full((rows, cols), SCALAR_INIT[name], dtype=np.float32)
            continue
        w = rng.standard_normal((rows, cols), dtype=np.float32)
        w *= np.float32(std)
        out[name] = w
    return out


def zipf_ids(batch: int, seq: int, vocab: int, seed: int = 1, s: float = ZIPF_S) -> np.ndarray:
    """Draw int32 ids [batch, seq + 1] from Zipf(s) truncated to ranks 1..vocab.

    p(rank k) is proportional to k^-s; id = k - 1. Sampling is by inverse CDF:
    a uniform draw u is mapped to the first id whose cumulative probability
    exceeds u.
    """
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    cdf[-1] = 1.0
    u = np.random.default_rng(seed).random(batch * (seq + 1))
    ids = np.searchsorted(cdf, u, side="right").astype(np.int32)
    return ids.reshape(batch, seq + 1)


# Documents of the packing workload: lengths round(exp(N(DOC_LEN_MU,
# DOC_LEN_SIGMA))) tokens (mean ~1100), at least 2; with a best-fit buffer of
# PACK_BUFFER_DOCS documents about 35% of the tokens are cut at sequence length
# 2048 once the buffer has settled, the figure the pages give.
DOC_LEN_MU = 6.5
DOC_LEN_SIGMA = 1.0
PACK_BUFFER_DOCS = 64


def synthetic_documents(n_docs: int, vocab: int, seed: int = 3, mu: float = DOC_LEN_MU,
                        sigma: float = DOC_LEN_SIGMA, s: float = ZIPF_S):
    """Seeded documents: (tokens int32 [total], offsets int64 [n_docs + 1]).

    Token 0 of each document is BOS = vocab - 1; the others are Zipf(s) ids over
    0 .. vocab - 2 (the zipf_ids sampling).
    """
    rng = np.random.default_rng(seed)
    lens = np.maximum(2, np.rint(np.exp(rng.normal(mu, sigma, n_docs)))).astype(np.int64)
    offsets = np.zeros(n_docs + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    ranks = np.arange(1, vocab, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    cdf[-1] = 1.0
    tokens = np.searchsorted(cdf, rng.random(int(offsets[-1])), side="right").astype(np.int32)
    tokens[offsets[:-1]] = vocab - 1
    return tokens, offsets


def split_tokens(ids: np.ndarray):
    """Inputs are positions 0..T-1 and targets positions 1..T of each row."""
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def random_like_grads(depth: int, vocab: int, seed: int, scale: float = 1e-3, kv_heads=None,
                      resid_scalars=False, backout=False, smear=False, ve_layers=()) -> dict:
    """Seeded Gaussian arrays shaped like the parameters (for optimizer-only cases)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, rows, cols, _kind, _layer in tensor_specs(depth, vocab, kv_heads, resid_scalars, backout, smear,
                                                        ve_layers):
        g = rng.standard_normal((rows, cols), dtype=np.float32)
        g *= np.float32(scale)
        out[name] = g
    return out
