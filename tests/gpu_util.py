"""Helpers for the GPU tests (test infrastructure; no method arithmetic here)."""
import numpy as np


def bf16_bits(x):
    """Round float array to bf16 (nearest even); return the raw uint16 bits as int16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r.view(np.int16)


def bits_to_f32(b):
    b = np.ascontiguousarray(b).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x):
    return bits_to_f32(bf16_bits(x)).reshape(np.shape(x))


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def dev(torch, arr, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def log(msg):
    print(msg, flush=True)
