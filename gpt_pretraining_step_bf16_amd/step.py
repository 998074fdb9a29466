"""Device buffers for repeated training steps (torch allocates, the HIP library computes).

``TrainState`` owns the flat fp32 parameters, their bf16 shadow, gradients,
Muon momentum, the NorMuon second moments, the AdamW moments of wte and
lm_head and the two workspaces, laid out as the library's tensor table says. A
step is ``fwd_bwd`` (loss + gradients) followed by ``muon`` or ``normuon``
(block matrices) and ``adamw`` (wte, lm_head).
"""
from __future__ import annotations

import numpy as np

from . import binding


def window_pattern(depth: int, seq: int, pattern: str = "SSSL", short_window=None):
    """Per-layer attention windows from a short/long pattern string.

    Layer l takes pattern[l % len(pattern)]: "L" is the full causal context
    (-1), "S" a window of short_window keys to the left of each query
    (default seq // 2).
    """
    pattern = pattern.upper()
    if not pattern or set(pattern) - {"S", "L"}:
        raise ValueError(f"window pattern must be made of S and L: {pattern!r}")
    short = seq // 2 if short_window is None else int(short_window)
    return [short if pattern[l % len(pattern)] == "S" else -1 for l in range(depth)]


class TrainState:
    def __init__(self, depth: int, vocab: int, seq: int, batch: int, device="cuda", kv_heads=None,
                 resid_scalars=False, backout_layer=None, smear=False, ve_layers=()):
        import torch

        self.torch = torch
        self.model = binding.GptModel(depth, vocab, seq, kv_heads, resid_scalars, backout_layer, smear, ve_layers)
        self.batch, self.seq = batch, seq
        self.device = device
        n = self.model.num_params
        self.tensors = self.model.tensors()
        self.params = torch.zeros(n, dtype=torch.float32, device=device)
        self.params_bf16 = torch.zeros(n, dtype=torch.int16, device=device)
        self.grads = torch.zeros(n, dtype=torch.float32, device=device)
        self.momentum = torch.zeros(n, dtype=torch.float32, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.ws = torch.empty(self.model.workspace_bytes(batch, seq), dtype=torch.uint8, device=device)
        self.muon_ws = torch.empty(self.model.muon_workspace_bytes(), dtype=torch.uint8, device=device)
        # AdamW moments of wte and lm_head (packed: wte, then lm_head).
        na = self.model.adamw_state_elems()
        self.exp_avg = torch.zeros(na, dtype=torch.float32, device=device)
        self.exp_avg_sq = torch.zeros(na, dtype=torch.float32, device=device)
        self.second_moment = torch.zeros(self.model.normuon_state_elems(), dtype=torch.float32,
                                         device=device)

    # -- host <-> device ------------------------------------------------------
    def flatten(self, arrays: dict) -> np.ndarray:
        flat = np.empty(self.model.num_params, dtype=np.float32)
        for t in self.tensors:
            a = arrays[t["name"]]
            assert a.shape == (t["rows"], t["cols"]), (t["name"], a.shape)
            flat[t["offset"]: t["offset"] + a.size] = a.ravel()
        return flat

    def unflatten(self, flat: np.ndarray) -> dict:
        return {t["name"]: flat[t["offset"]: t["offset"] + t["rows"] * t["cols"]].reshape(t["rows"], t["cols"])
                for t in self.tensors}

    def load_weights(self, weights: dict):
        self.params.copy_(self.torch.from_numpy(self.flatten(weights)))
        self.model.refresh_bf16(self.params, self.params_bf16)

    def load_momentum(self, momentum: dict):
        self.momentum.copy_(self.torch.from_numpy(self.flatten(momentum)))

    def load_grads(self, grads: dict):
        self.grads.copy_(self.torch.from_numpy(self.flatten(grads)))

    def to_host(self, t) -> dict:
        return self.unflatten(t.detach().cpu().numpy())

    # -- compute --------------------------------------------------------------
    def set_windows(self, windows):
        """Per-layer attention windows for later fwd_bwd calls (None: all causal)."""
        self.model.set_windows(windows)

    def fwd_bwd(self, tokens, targets, accumulate=False):
        self.model.fwd_bwd(self.params_bf16, tokens, targets, self.loss, self.grads, self.ws,
                           accumulate=accumulate)

    def muon(self, lr, momentum_coef, ns_coeffs):
        self.model.muon_step(self.params, self.params_bf16, self.grads, self.momentum, lr,
                             momentum_coef, ns_coeffs, self.muon_ws)

    def normuon(self, lr, momentum_coef, beta2, ns_coeffs):
        self.model.normuon_step(self.params, self.params_bf16, self.grads, self.momentum,
                                self.second_moment, lr, momentum_coef, beta2, ns_coeffs, self.muon_ws)

    def adamw(self, lr, beta1, beta2, eps, weight_decay, step):
        self.model.adamw_step(self.params, self.params_bf16, self.grads, self.exp_avg, self.exp_avg_sq,
                              lr, beta1, beta2, eps, weight_decay, step)

    def check(self) -> int:
        return self.model.check(self.ws)
