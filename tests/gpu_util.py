"""Helpers for the GPU tests (test infrastructure: tolerance helpers may call the oracle)."""
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


def assert_scalar_grads(grads, ref_grads, scales, log=None, eps=1e-3):
    """Gradients of the scalar tensors are dot products, over every token and
    channel, of a stream gradient g with a kept stream v. The final norm makes
    the loss insensitive to the stream's scale, so these sums cancel down to a
    small fraction (6e-5 to 4e-3 here) of their Cauchy-Schwarz bound
    S = sum over rows of |g_row| |v_row| (the oracle reports S per scalar).
    Their error is at most |delta g| |v| <= eps S, eps being the relative error
    of the device's stream gradient (bounded by the 2e-2 gradient bar); the
    errors measured on these models stay below 5e-5 S, except the smear gate
    at the end of the backward chain (up to 2.6e-4 S), so per scalar:
    |delta| <= 2e-2 |ref| + eps S with eps = 1e-3. A sign error or a wrong
    kept stream also breaks the matrix and embedding gradients that the same
    stream gradient feeds, which the rel-L2 checks catch. The value-embedding
    gates sum products of dv, which comes out of the bf16 attention backward
    with about 1e-2 relative error (within the 2e-2 bar): they take eps = 1e-2
    (measured up to 2.9e-3 S)."""
    for k, s in scales.items():
        got = np.asarray(grads[k], dtype=np.float64).ravel()
        ref = np.asarray(ref_grads[k]).ravel()
        sv = np.asarray(s).ravel()
        if log is not None:
            log(f"  {k}: |delta|/S = {np.max(np.abs(got - ref) / sv):.2e}")
        tol = 2e-2 * np.abs(ref) + eps * sv
        assert np.all(np.abs(got - ref) <= tol), (k, got, ref, sv)
