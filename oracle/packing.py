"""Oracle: BOS-aligned best-fit packing of documents into fixed-length rows.

TEST INFRASTRUCTURE ONLY (see the package header).

[CT50] "4. Carregamento de Dados" describes the loader: every row starts with
the BOS token; rows are filled with whole documents chosen best-fit (the
longest buffered document that still fits the space left); when no buffered
document fits, one is cut to fill the row exactly; about 100% of the row
tokens are used and about 35% of the tokens are cut away at sequence length
2048. Its example scans the buffer in order and keeps the first document whose
length beats the best so far (so among equal lengths the earliest wins), and
removes the chosen document from the buffer.

Readings where the page is silent or cut short:
  * A document is a token sequence that begins with BOS (the tokenizer puts it
    there); the packer inserts nothing, so a row starts with BOS because it
    starts with the beginning of a document.
  * The document that is cut is the shortest buffered one (the page's comment
    says so), earliest among equal lengths; its first `remaining` tokens fill
    the row, the rest is dropped (counted as cut), and it leaves the buffer.
  * The buffer holds up to `buffer_cap` documents in arrival order. Before each
    choice it is topped up from the document stream; a chosen document leaves
    it and the others keep their order (a list pop).
  * A row holds `row_len` tokens (sequence length + 1: inputs are positions
    0..T-1, targets 1..T). Running out of documents in mid-row is an error.

Parity pins (tests/test_oracle_packing.py): a hand-worked stream; the row and
document invariants on seeded streams (every row full and starting with BOS,
whole documents contiguous and in the order chosen, at most one cut document
per row and always last, token conservation); the best-fit choice checked
against a brute-force replay of the buffer; a buffer of one document reduces
the packer to cutting the stream into rows document by document.
"""
from __future__ import annotations

import numpy as np


def pack_best_fit(tokens, offsets, rows, row_len, buffer_cap, state=None):
    """Pack `rows` rows of `row_len` tokens from the document stream.

    tokens, offsets: document d is tokens[offsets[d]:offsets[d + 1]].
    state: (buffer list of document ids, next stream document), carried between
    calls; None starts with an empty buffer at document 0.
    Returns (out [rows, row_len] int32, new state, tokens cut, log) where log
    lists, per row, the (document id, tokens taken, whole) placements in order.
    """
    offsets = [int(o) for o in offsets]
    n_docs = len(offsets) - 1
    buffer, next_doc = ([], 0) if state is None else (list(state[0]), int(state[1]))
    out = np.zeros((rows, row_len), dtype=np.int32)
    cut = 0
    log = []

    def length(d):
        return offsets[d + 1] - offsets[d]

    for r in range(rows):
        remaining = row_len
        pos = 0
        placed = []
        while remaining > 0:
            while len(buffer) < buffer_cap and next_doc < n_docs:
                if length(next_doc) <= 0:
                    raise ValueError("empty document")
                buffer.append(next_doc)
                next_doc += 1
            if not buffer:
                raise ValueError("document stream exhausted")
            # Longest buffered document that fits; earliest among equals.
            best_idx, best_len = -1, 0
            for i, d in enumerate(buffer):
                n = length(d)
                if n <= remaining and n > best_len:
                    best_idx, best_len = i, n
            if best_idx >= 0:
                d = buffer.pop(best_idx)
                take = best_len
                whole = True
            else:
                # Nothing fits: cut the shortest (earliest among equals).
                short_idx = 0
                for i, d in enumerate(buffer):
                    if length(d) < length(buffer[short_idx]):
                        short_idx = i
                d = buffer.pop(short_idx)
                take = remaining
                cut += length(d) - take
                whole = False
            out[r, pos:pos + take] = tokens[offsets[d]:offsets[d] + take]
            placed.append((d, take, whole))
            pos += take
            remaining -= take
        log.append(placed)
    return out, (buffer, next_doc), cut, log
