"""ctypes binding of the C ABI in include/gpt.h (argument marshalling only).

Every compute call runs in the HIP library libgptstep.so; torch tensors only
supply device pointers and the current stream. If the library has not been
built, ``lib()`` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgptstep.so")

GPT_OK, GPT_EINVAL, GPT_ESHAPE, GPT_EHIP, GPT_ETOKEN, GPT_EWORKSPACE, GPT_EDATA = 0, -1, -2, -3, -4, -5, -6
KIND_NAMES = {0: "emb", 1: "matrix", 2: "lm_head", 3: "scalar", 4: "gate"}

# gpt_op_gemm out_mode values
OUT_F32, OUT_F32_ACC, OUT_BF16, OUT_RELU_BF16, OUT_RESID_BF16 = 0, 1, 2, 3, 4


class GptTensor(C.Structure):
    _fields_ = [
        ("name", C.c_char * 32),
        ("offset", C.c_int64),
        ("rows", C.c_int32),
        ("cols", C.c_int32),
        ("kind", C.c_int32),
        ("layer", C.c_int32),
    ]


class GptConfig(C.Structure):
    _fields_ = [
        ("depth", C.c_int32),
        ("vocab", C.c_int32),
        ("max_seq", C.c_int32),
        ("kv_heads", C.c_int32),
        ("resid_scalars", C.c_int32),
        ("backout_layer", C.c_int32),
        ("smear", C.c_int32),
        ("ve_layers", C.c_int64),
    ]


class GptError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


_lib = None
_P = C.c_void_p
_I = C.c_int32
_L = C.c_int64
_S = C.c_size_t
_F = C.c_float


def _sig(lib, name, res, args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = args


EXPORTS = {
    "gpt_create": (C.c_int, [_I, _I, _I, C.POINTER(_P)]),
    "gpt_create_gqa": (C.c_int, [_I, _I, _I, _I, C.POINTER(_P)]),
    "gpt_kv_heads": (C.c_int32, [_P]),
    "gpt_create_config": (C.c_int, [C.POINTER(GptConfig), C.POINTER(_P)]),
    "gpt_backout_layer": (C.c_int32, [_P]),
    "gpt_destroy": (None, [_P]),
    "gpt_dims": (C.c_int, [_P, C.POINTER(C.c_int32)]),
    "gpt_num_params": (C.c_int64, [_P]),
    "gpt_num_tensors": (C.c_int32, [_P]),
    "gpt_tensor_info": (C.c_int, [_P, _I, C.POINTER(GptTensor)]),
    "gpt_workspace_bytes": (C.c_size_t, [_P, _I, _I]),
    "gpt_fwd_bwd": (C.c_int, [_P, _P, _P, _P, _I, _I, _P, _P, _I, _P, _S, _P]),
    "muon_workspace_bytes": (C.c_size_t, [_P]),
    "gpt_ns_default_coeffs": (C.c_int32, [C.POINTER(C.c_float), _I]),
    "muon_step": (C.c_int, [_P, _P, _P, _P, _P, _F, _F, C.POINTER(C.c_float), _I, _P, _S, _P]),
    "normuon_state_elems": (C.c_int64, [_P]),
    "normuon_step": (C.c_int, [_P, _P, _P, _P, _P, _P, _F, _F, _F, C.POINTER(C.c_float), _I, _P, _S, _P]),
    "adamw_state_elems": (C.c_int64, [_P]),
    "adamw_step": (C.c_int, [_P, _P, _P, _P, _P, _P, _F, _F, _F, _F, _F, _I, _P]),
    "gpt_refresh_bf16": (C.c_int, [_P, _P, _P, _P]),
    "gpt_check": (C.c_int, [_P, _P, _P]),
    "gpt_status_str": (C.c_char_p, [C.c_int]),
    "gpt_op_gemm": (C.c_int, [_I, _I, _I, _I, _P, _L, _L, _I, _P, _L, _L, _I, _P, _L, _L, _I, _P]),
    "gpt_op_qkv_projection": (C.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gpt_op_attention_bwd_qknorm": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gpt_op_attention_fwd": (C.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gpt_op_attention_bwd": (C.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gpt_set_attention_windows": (C.c_int, [_P, C.POINTER(C.c_int32), _I]),
    "gpt_get_attention_windows": (C.c_int, [_P, C.POINTER(C.c_int32), _I]),
    "gpt_op_ns_scratch_bytes": (C.c_size_t, [_I, _I, _I]),
    "gpt_op_newton_schulz": (C.c_int, [_P, _I, _I, _I, C.POINTER(C.c_float), _I, _P, _S, _P]),
    "gpt_op_newton_schulz_noalloc": (C.c_int, [_P, _I, _I, _I, C.POINTER(C.c_float), _I, _P]),
    "gpt_probe_mfma_bf16": (C.c_int, [_I, _I, _P, C.POINTER(C.c_double), _P]),
    "gpt_pack_best_fit": (C.c_int, [_P, _P, C.c_int64, _P, C.POINTER(C.c_int32), _I, C.POINTER(C.c_int64), _I,
                                    _I, _P, C.POINTER(C.c_int64)]),
    "gpt_profile_enable": (C.c_int, [_P, _I]),
    "gpt_profile_reset": (C.c_int, [_P]),
    "gpt_profile_read": (C.c_int, [_P, _I, C.POINTER(C.c_double), C.POINTER(C.c_double),
                                   C.POINTER(C.c_int64)]),
}

PROF_GEMM, PROF_ATTN_FWD, PROF_ATTN_BWD, PROF_NS = 0, 1, 2, 3


def lib():
    """Load libgptstep.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gpt_pretraining_step_bf16_amd.build`"
            )
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            _sig(handle, name, res, args)
        _lib = handle
    return _lib


def status_str(status) -> str:
    return lib().gpt_status_str(int(status)).decode()


def _check(status, what):
    if status != GPT_OK:
        raise GptError(status, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return C.c_void_p(stream)
    import torch

    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _coeffs(table, steps=None):
    """(host float buffer, rows) for a Newton-Schulz table; None passes NULL
    (the library's built-in table) with `steps` rows of it (default 5)."""
    if table is None:
        return None, 5 if steps is None else int(steps)
    arr = np.ascontiguousarray(np.asarray(table, dtype=np.float32).reshape(-1, 3))
    buf = (C.c_float * arr.size)(*arr.ravel().tolist())
    return buf, arr.shape[0]


def ns_default_coeffs():
    """The library's built-in Newton-Schulz table as a float32 [rows, 3] array."""
    rows = lib().gpt_ns_default_coeffs(None, 0)
    buf = (C.c_float * (3 * rows))()
    lib().gpt_ns_default_coeffs(buf, rows)
    return np.array(buf[:], dtype=np.float32).reshape(rows, 3)


class GptModel:
    """Host-side plan of a model (no device memory)."""

    def __init__(self, depth: int, vocab: int, max_seq: int, kv_heads=None, resid_scalars=False,
                 backout_layer=None, smear=False, ve_layers=()):
        h = C.c_void_p()
        if not resid_scalars and backout_layer is None and not smear and not ve_layers:
            if kv_heads is None:
                _check(lib().gpt_create(depth, vocab, max_seq, C.byref(h)), "gpt_create")
            else:
                _check(lib().gpt_create_gqa(depth, vocab, max_seq, int(kv_heads), C.byref(h)), "gpt_create_gqa")
        else:
            cfg = GptConfig(depth, vocab, max_seq, 0 if kv_heads is None else int(kv_heads),
                            1 if resid_scalars else 0, -1 if backout_layer is None else int(backout_layer),
                            1 if smear else 0, sum(1 << int(l) for l in set(ve_layers)))
            _check(lib().gpt_create_config(C.byref(cfg), C.byref(h)), "gpt_create_config")
        self._h = h
        dims = (C.c_int32 * 6)()
        _check(lib().gpt_dims(h, dims), "gpt_dims")
        self.depth, self.d, self.heads, self.mlp, self.vocab, self.max_seq = list(dims)
        self.kv_heads = int(lib().gpt_kv_heads(h))
        bl = int(lib().gpt_backout_layer(h))
        self.backout_layer = None if bl < 0 else bl

    def close(self):
        if getattr(self, "_h", None):
            lib().gpt_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    @property
    def num_params(self) -> int:
        return int(lib().gpt_num_params(self._h))

    def tensors(self):
        out = []
        for i in range(lib().gpt_num_tensors(self._h)):
            t = GptTensor()
            _check(lib().gpt_tensor_info(self._h, i, C.byref(t)), "gpt_tensor_info")
            out.append(dict(name=t.name.decode(), offset=int(t.offset), rows=int(t.rows),
                            cols=int(t.cols), kind=KIND_NAMES[int(t.kind)], layer=int(t.layer)))
        return out

    def set_windows(self, windows):
        """Per-layer attention windows (None entries or -1: full causal context)."""
        if windows is None:
            _check(lib().gpt_set_attention_windows(self._h, None, 0), "gpt_set_attention_windows")
            return
        vals = [-1 if w is None else int(w) for w in windows]
        arr = (C.c_int32 * len(vals))(*vals)
        _check(lib().gpt_set_attention_windows(self._h, arr, len(vals)), "gpt_set_attention_windows")

    def windows(self):
        arr = (C.c_int32 * self.depth)()
        _check(lib().gpt_get_attention_windows(self._h, arr, self.depth), "gpt_get_attention_windows")
        return list(arr)

    def workspace_bytes(self, batch: int, seq: int) -> int:
        return int(lib().gpt_workspace_bytes(self._h, batch, seq))

    def muon_workspace_bytes(self) -> int:
        return int(lib().muon_workspace_bytes(self._h))

    # -- compute (torch device tensors) -------------------------------------
    def fwd_bwd(self, params_bf16, tokens, targets, loss, grads, workspace, accumulate=False,
                stream=None):
        batch, seq = tokens.shape
        st = lib().gpt_fwd_bwd(self._h, _ptr(params_bf16), _ptr(tokens), _ptr(targets), batch, seq,
                               _ptr(loss), _ptr(grads), 1 if accumulate else 0, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "gpt_fwd_bwd")

    def muon_step(self, params, params_bf16, grads, momentum, lr, momentum_coef, ns_coeffs,
                  workspace, stream=None):
        buf, steps = _coeffs(ns_coeffs)
        st = lib().muon_step(self._h, _ptr(params), _ptr(params_bf16), _ptr(grads), _ptr(momentum),
                             float(lr), float(momentum_coef), buf, steps, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "muon_step")

    def normuon_state_elems(self) -> int:
        return int(lib().normuon_state_elems(self._h))

    def normuon_step(self, params, params_bf16, grads, momentum, second_moment, lr, momentum_coef, beta2,
                     ns_coeffs, workspace, stream=None):
        buf, steps = _coeffs(ns_coeffs)
        st = lib().normuon_step(self._h, _ptr(params), _ptr(params_bf16), _ptr(grads), _ptr(momentum),
                                _ptr(second_moment), float(lr), float(momentum_coef), float(beta2), buf,
                                steps, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
        _check(st, "normuon_step")

    def adamw_state_elems(self) -> int:
        return int(lib().adamw_state_elems(self._h))

    def adamw_step(self, params, params_bf16, grads, exp_avg, exp_avg_sq, lr, beta1, beta2, eps,
                   weight_decay, step, stream=None):
        st = lib().adamw_step(self._h, _ptr(params), _ptr(params_bf16), _ptr(grads), _ptr(exp_avg),
                              _ptr(exp_avg_sq), float(lr), float(beta1), float(beta2), float(eps),
                              float(weight_decay), int(step), _stream(stream))
        _check(st, "adamw_step")

    def refresh_bf16(self, params, params_bf16, stream=None):
        _check(lib().gpt_refresh_bf16(self._h, _ptr(params), _ptr(params_bf16), _stream(stream)),
               "gpt_refresh_bf16")

    def check(self, workspace, stream=None) -> int:
        return int(lib().gpt_check(self._h, _ptr(workspace), _stream(stream)))

    # -- launch timing ----------------------------------------------------------
    def profile_enable(self, on: bool = True):
        _check(lib().gpt_profile_enable(self._h, 1 if on else 0), "gpt_profile_enable")

    def profile_reset(self):
        _check(lib().gpt_profile_reset(self._h), "gpt_profile_reset")

    def profile_read(self, category: int):
        ms, fl, n = C.c_double(), C.c_double(), C.c_int64()
        _check(lib().gpt_profile_read(self._h, category, C.byref(ms), C.byref(fl), C.byref(n)),
               "gpt_profile_read")
        return ms.value, fl.value, n.value


# -- step-level entry points ---------------------------------------------------
def op_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, Cout, ldc, out_mode, batch=1, stride_a=0,
            stride_b=0, stride_c=0, stream=None):
    st = lib().gpt_op_gemm(M, N, K, batch, _ptr(A), lda, stride_a, int(a_kmajor), _ptr(B), ldb,
                           stride_b, int(b_kmajor), _ptr(Cout), ldc, stride_c, out_mode,
                           _stream(stream))
    _check(st, "gpt_op_gemm")


def op_qkv_projection(xn, w, qkv, rstd, rope_scratch, batch, seq, d, heads, kv_heads=None, stream=None):
    kvh = heads if kv_heads is None else int(kv_heads)
    _check(lib().gpt_op_qkv_projection(_ptr(xn), _ptr(w), _ptr(qkv), _ptr(rstd), _ptr(rope_scratch), batch, seq,
                                       d, heads, kvh, _stream(stream)), "gpt_op_qkv_projection")


def op_attention_fwd(qkv, o, lse, batch, seq, heads, window=-1, kv_heads=None, stream=None):
    kvh = heads if kv_heads is None else int(kv_heads)
    _check(lib().gpt_op_attention_fwd(_ptr(qkv), _ptr(o), _ptr(lse), batch, seq, heads, kvh, int(window),
                                      _stream(stream)), "gpt_op_attention_fwd")


def op_attention_bwd(qkv, o, lse, dO, dqkv, scratch, batch, seq, heads, window=-1, kv_heads=None,
                     stream=None):
    kvh = heads if kv_heads is None else int(kv_heads)
    _check(lib().gpt_op_attention_bwd(_ptr(qkv), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dqkv),
                                      _ptr(scratch), batch, seq, heads, kvh, int(window), _stream(stream)),
           "gpt_op_attention_bwd")


def op_attention_bwd_qknorm(qkv, o, lse, dO, rstd, rope_table, dqkv, scratch, batch, seq, heads, window=-1,
                            kv_heads=None, stream=None):
    kvh = heads if kv_heads is None else int(kv_heads)
    _check(lib().gpt_op_attention_bwd_qknorm(_ptr(qkv), _ptr(o), _ptr(lse), _ptr(dO), _ptr(rstd), _ptr(rope_table),
                                             _ptr(dqkv), _ptr(scratch), batch, seq, heads, kvh, int(window),
                                             _stream(stream)),
           "gpt_op_attention_bwd_qknorm")


def ns_scratch_bytes(count, rows, cols) -> int:
    return int(lib().gpt_op_ns_scratch_bytes(count, rows, cols))


# Size of the library's fixed device array behind gpt_op_newton_schulz_noalloc
# (GPT_NS_STATIC_SCRATCH_BYTES in include/gpt.h).
NS_STATIC_SCRATCH_BYTES = 128 << 20


def op_newton_schulz_noalloc(X, count, rows, cols, ns_coeffs, stream=None):
    buf, steps = _coeffs(ns_coeffs)
    st = lib().gpt_op_newton_schulz_noalloc(_ptr(X), count, rows, cols, buf, steps, _stream(stream))
    _check(st, "gpt_op_newton_schulz_noalloc")


def op_newton_schulz(X, count, rows, cols, ns_coeffs, scratch, stream=None):
    buf, steps = _coeffs(ns_coeffs)
    st = lib().gpt_op_newton_schulz(_ptr(X), count, rows, cols, buf, steps, _ptr(scratch),
                                    scratch.numel() * scratch.element_size(), _stream(stream))
    _check(st, "gpt_op_newton_schulz")


def probe_mfma_bf16(blocks, iters, sink, stream=None) -> float:
    """Launch the MFMA issue-rate probe; returns the flops of the launch."""
    fl = C.c_double(0.0)
    st = lib().gpt_probe_mfma_bf16(int(blocks), int(iters), _ptr(sink), C.byref(fl), _stream(stream))
    _check(st, "gpt_probe_mfma_bf16")
    return float(fl.value)


class BestFitPacker:
    """State of gpt_pack_best_fit over one document stream (host arrays).

    tokens: int32 [total], offsets: int64 [n_docs + 1]; every call of pack()
    fills `rows` rows of `row_len` tokens and carries the buffer to the next.
    """

    def __init__(self, tokens, offsets, buffer_cap):
        import numpy as np

        self.tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        self.offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.n_docs = len(self.offsets) - 1
        self.buffer = np.zeros(int(buffer_cap), dtype=np.int64)
        self.count = C.c_int32(0)
        self.next_doc = C.c_int64(0)
        self.tokens_cut = 0

    def pack(self, rows, row_len):
        import numpy as np

        out = np.zeros((int(rows), int(row_len)), dtype=np.int32)
        cut = C.c_int64(0)
        vp = lambda a: C.c_void_p(a.ctypes.data)
        st = lib().gpt_pack_best_fit(vp(self.tokens), vp(self.offsets), self.n_docs, vp(self.buffer),
                                     C.byref(self.count), len(self.buffer), C.byref(self.next_doc), int(rows),
                                     int(row_len), vp(out), C.byref(cut))
        self.tokens_cut += int(cut.value)
        _check(st, "gpt_pack_best_fit")
        return out

    @property
    def state(self):
        """(buffered document ids in order, next stream document)."""
        return [int(x) for x in self.buffer[:self.count.value]], int(self.next_doc.value)
