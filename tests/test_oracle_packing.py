"""Pins of the oracle's best-fit packer (oracle/packing.py), CPU only."""
import numpy as np
import pytest

from gpt_pretraining_step_bf16_amd import synthetic as syn
from oracle.packing import pack_best_fit

BOS = 99


def _docs(lengths):
    """Document d = [BOS, 100 d + 1, 100 d + 2, ...] of the given length."""
    toks, offs = [], [0]
    for d, n in enumerate(lengths):
        toks += [BOS] + [100 * d + j for j in range(1, n)]
        offs.append(len(toks))
    return np.array(toks, dtype=np.int32), np.array(offs, dtype=np.int64)


def test_hand_worked_stream():
    # lengths 5, 3, 8, 2, 4; rows of 6; a buffer of 3 documents.
    # row 0: buffer {0,1,2}: doc 0 (5) fits best; 1 left, refill {1,2,3}: none
    #        fits, the shortest (doc 3, 2 tokens) gives 1 token, 1 cut.
    # row 1: refill {1,2,4}: doc 4 (4); 2 left, {1,2}: none fits, doc 1 (3)
    #        gives 2 tokens, 1 cut.
    # row 2: {2}: doc 2 (8) gives 6 tokens, 2 cut.
    tok, off = _docs([5, 3, 8, 2, 4])
    out, state, cut, log = pack_best_fit(tok, off, 3, 6, 3)
    assert out.tolist() == [[99, 1, 2, 3, 4, 99],
                            [99, 401, 402, 403, 99, 101],
                            [99, 201, 202, 203, 204, 205]]
    assert cut == 4
    assert state == ([], 5)
    assert [[(d, w) for d, _, w in row] for row in log] == [[(0, True), (3, False)], [(4, True), (1, False)],
                                                            [(2, False)]]
    with pytest.raises(ValueError):
        pack_best_fit(tok, off, 1, 6, 3, state)


def _replay_check(tok, off, rows, row_len, cap, calls=1):
    """Row and document invariants, and the choice rule in a set form: the
    buffer at any choice is the `cap` lowest-numbered documents not yet placed
    (documents arrive in stream order and leave only when placed), and the
    choice is the longest of them that fits, else the shortest (lowest number
    among equal lengths either way)."""
    lens = np.diff(off)
    placed = set()
    state = None
    total_cut = 0
    for _ in range(calls):
        out, state, cut, log = pack_best_fit(tok, off, rows, row_len, cap, state)
        total_cut += cut
        for r, row in enumerate(log):
            assert out[r, 0] == tok[off[row[0][0]]]  # starts with a document's first token (BOS)
            assert sum(t for _, t, _ in row) == row_len
            assert all(w for _, _, w in row[:-1])  # only the last placement may be cut
            pos = 0
            remaining = row_len
            for d, take, whole in row:
                cand = sorted(set(range(len(lens))) - placed)[:cap]
                fit = [c for c in cand if lens[c] <= remaining]
                if fit:
                    want = min(fit, key=lambda c: (-lens[c], c))
                    assert whole and take == lens[d]
                else:
                    want = min(cand, key=lambda c: (lens[c], c))
                    assert not whole and take == remaining < lens[d]
                assert d == want
                np.testing.assert_array_equal(out[r, pos:pos + take], tok[off[d]:off[d] + take])
                placed.add(d)
                pos += take
                remaining -= take
    # Conservation: every token of a document that left the buffer was placed or cut.
    assert sum(lens[d] for d in placed) == calls * rows * row_len + total_cut
    assert state[0] == sorted(set(range(state[1])) - placed)


@pytest.mark.parametrize("seed,cap,row_len,rows,calls", [(0, 8, 257, 16, 3), (1, 64, 2049, 6, 2), (2, 1, 100, 20, 1),
                                                         (3, 300, 513, 10, 2)])
def test_invariants_and_choice_rule(seed, cap, row_len, rows, calls):
    tok, off = syn.synthetic_documents(2000, 512, seed=seed, mu=5.0, sigma=1.2)
    _replay_check(tok, off, rows, row_len, cap, calls)


def test_buffer_of_one_cuts_the_stream_in_order():
    tok, off = syn.synthetic_documents(300, 512, seed=5, mu=4.0, sigma=1.0)
    out, state, cut, log = pack_best_fit(tok, off, 10, 64, 1)
    order = [d for row in log for d, _, _ in row]
    assert order == list(range(len(order)))  # documents in stream order
    for row in log:
        for d, take, whole in row:
            assert whole == (take == off[d + 1] - off[d])


def test_documents_of_row_length_fill_one_row_each():
    tok, off = _docs([6] * 5)
    out, state, cut, log = pack_best_fit(tok, off, 5, 6, 3)
    assert cut == 0 and [row[0][0] for row in log] == [0, 1, 2, 3, 4]


def test_documents_longer_than_a_row_are_cut_shortest_first():
    tok, off = _docs([9, 7, 8, 7, 10])
    out, state, cut, log = pack_best_fit(tok, off, 3, 6, 5)
    assert [row[0][0] for row in log] == [1, 3, 2]  # 7 (first of the equal ones), 7, 8
    assert cut == 1 + 1 + 2


def test_empty_document_is_an_error():
    tok, off = _docs([3, 2])
    off = np.array([0, 3, 3, 5], dtype=np.int64)
    with pytest.raises(ValueError):
        pack_best_fit(tok, off, 1, 4, 4)


def test_synthetic_documents_start_with_bos():
    tok, off = syn.synthetic_documents(50, 1000, seed=9)
    assert (tok[off[:-1]] == 999).all() and (np.diff(off) >= 2).all()
    assert tok.max() <= 999 and tok.min() >= 0
