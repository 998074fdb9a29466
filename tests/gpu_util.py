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


def assert_scalar_grads(grads, ref_grads, scales, log=None, eps=2e-4, rel=2e-2):
    """Gradients of the scalar tensors (and of the value-embedding gates) are
    dot products, over every token and channel, of a stream gradient g with a
    kept stream v. For a sum of N*d weakly correlated terms |sum| is of order
    S / sqrt(N d), S = sum over rows of |g_row| |v_row| being its
    Cauchy-Schwarz bound (the oracle reports S per element), so at the test
    sizes the references sit at 1e-4 to 3e-2 of S. The device's error in such
    a sum is at most |delta g| |v|, a small multiple of S times the relative
    error of the stream gradient it reads.

    Per element: |delta| <= max(rel |ref|, eps S). A reference above
    (eps / rel) S is thus held to the plain relative bar, and every reference
    above eps S to the right sign; eps is a few times the error measured on the
    device (see the callers)."""
    for k, s in scales.items():
        got = np.asarray(grads[k], dtype=np.float64).ravel()
        ref = np.asarray(ref_grads[k]).ravel()
        sv = np.asarray(s).ravel()
        e = eps[k] if isinstance(eps, dict) else eps
        if log is not None:
            log(f"  {k}: |delta|/S = {np.max(np.abs(got - ref) / sv):.2e} (eps {e:.0e}); "
                f"|ref|/S in [{np.min(np.abs(ref) / sv):.1e}, {np.max(np.abs(ref) / sv):.1e}]")
        tol = np.maximum(rel * np.abs(ref), e * sv)
        assert np.all(np.abs(got - ref) <= tol), (k, got, ref, sv)
        big = np.abs(ref) > e * sv
        assert np.all(np.sign(got[big]) == np.sign(ref[big])), (k, got, ref)
