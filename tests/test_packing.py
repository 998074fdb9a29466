"""gpt_pack_best_fit (the library's host-side packer) against the oracle,
bit for bit, and its error handling. CPU only: the packer uses no GPU."""
import ctypes as C

import numpy as np
import pytest

import oracle
from gpt_pretraining_step_bf16_amd import binding
from gpt_pretraining_step_bf16_amd import synthetic as syn


@pytest.mark.parametrize("seed,cap,row_len,rows,calls", [
    (0, 64, 2049, 8, 3),     # the packing workload's buffer at sequence length 2048
    (1, 1, 129, 12, 2),      # one buffered document
    (2, 7, 65, 40, 3),       # short rows: most documents are cut
    (3, 500, 4097, 3, 2),    # a buffer larger than the rows need
    (4, 16, 1, 10, 1),       # rows of one token: every row is a cut BOS
])
def test_matches_oracle(seed, cap, row_len, rows, calls):
    tok, off = syn.synthetic_documents(3000, 4096, seed=seed)
    pk = binding.BestFitPacker(tok, off, cap)
    state = None
    cut_total = 0
    for _ in range(calls):
        got = pk.pack(rows, row_len)
        want, state, cut, _ = oracle.pack_best_fit(tok, off, rows, row_len, cap, state)
        np.testing.assert_array_equal(got, want)
        cut_total += cut
        assert pk.state == (state[0], state[1])
    assert pk.tokens_cut == cut_total
    assert (got[:, 0] == 4095).all()  # every row starts with BOS


def test_cut_fraction_of_the_packing_workload():
    """Once the buffer has settled (its long documents wait until they are
    the shortest left), about 35% of the tokens are cut at sequence length
    2048 with the workload's document lengths and buffer, as the pages report."""
    tok, off = syn.synthetic_documents(20000, 32768, seed=11)
    pk = binding.BestFitPacker(tok, off, syn.PACK_BUFFER_DOCS)
    for _ in range(20):
        pk.pack(32, 2049)
    before = pk.tokens_cut
    for _ in range(20):
        pk.pack(32, 2049)
    cut = pk.tokens_cut - before
    frac = cut / (20 * 32 * 2049 + cut)
    assert 0.25 < frac < 0.45, frac


def test_stream_exhaustion_keeps_a_consistent_state():
    tok, off = syn.synthetic_documents(6, 4096, seed=1, mu=3.0, sigma=0.5)
    total = int(off[-1])
    pk = binding.BestFitPacker(tok, off, 4)
    with pytest.raises(binding.GptError) as e:
        pk.pack(total, 3)  # more rows than the stream can fill
    assert e.value.status == binding.GPT_EDATA
    buf, nxt = pk.state
    assert nxt == 6 and buf == []


def _raw(tok, off, n_docs, buf, count, cap, nxt, rows, row_len, out):
    vp = lambda a: None if a is None else C.c_void_p(a.ctypes.data)
    c, n = C.c_int32(count), C.c_int64(nxt)
    st = binding.lib().gpt_pack_best_fit(vp(tok), vp(off), n_docs, vp(buf), C.byref(c), cap, C.byref(n), rows,
                                         row_len, vp(out), None)
    return st, c.value, n.value


def test_bad_arguments():
    tok, off = syn.synthetic_documents(10, 512, seed=2)
    buf = np.zeros(4, dtype=np.int64)
    out = np.zeros((2, 16), dtype=np.int32)
    assert _raw(tok, off, 10, buf, 0, 4, 0, 2, 16, out)[0] == binding.GPT_OK
    assert _raw(None, off, 10, buf, 0, 4, 0, 2, 16, out)[0] == binding.GPT_EINVAL
    assert _raw(tok, off, 10, buf, 5, 4, 0, 2, 16, out)[0] == binding.GPT_EINVAL   # count > cap
    assert _raw(tok, off, 10, buf, 0, 0, 0, 2, 16, out)[0] == binding.GPT_EINVAL   # no buffer
    assert _raw(tok, off, 10, buf, 0, 4, 11, 2, 16, out)[0] == binding.GPT_EINVAL  # next past the stream
    buf[0] = 10
    assert _raw(tok, off, 10, buf, 1, 4, 0, 2, 16, out)[0] == binding.GPT_EINVAL   # buffered id out of range
    empty = off.copy()
    empty[3] = empty[2]  # document 2 empty
    assert _raw(tok, empty, 10, np.zeros(4, np.int64), 0, 4, 0, 2, 16, out)[0] == binding.GPT_EDATA
