"""Ragged paged KV bookkeeping (oracle; test infrastructure).

After a verify step sequences accept different numbers of drafts, so their
cached lengths, position ids and KV state diverge; handling that exactly is
what makes a batched speculative step reproduce each sequence decoded alone
(proofoftech.org, "'Lossless' speculative decoding is a property of the
math, not your deployment.", section "Batching breaks the implementation":
the ragged tensor problem).

State per sequence: committed length C (positions 0..C-1 are valid) and the
position id of the next query token (equal to C).  APPEND writes the n_s
rows of a verify block at positions C..C+n_s-1 (page ``table[s][p // 16]``,
offset ``p % 16``; keys stored ``[page][Hkv][16][D]``, values
``[page][Hkv][D][16]``).  COMMIT keeps the last committed token plus the
a_s accepted drafts: C <- C + a_s + 1, position id <- C.  Rollback is
truncation: rejected rows stay in the cache beyond C and are overwritten by
the next APPEND.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


def slot_location(page_table, s: int, p: int):
    return int(page_table[s][p // PAGE]), p % PAGE


MAX_ROWS = 8  # rows of one verify block (k <= 7 drafts)


def append(k_pages, v_pages, page_table, seq_len, row_start, k_new, v_new):
    """Return copies of the caches with every block row written in place.

    A block has at most MAX_ROWS rows (later rows are not written).  A row
    whose position lies outside the table (negative, or at or past 16 *
    max_pages) or on a page whose id lies outside [0, num_pages) is
    skipped: the pages' tables are always whole, this is the library's
    reading of such entries."""
    k_pages = np.array(k_pages, copy=True)
    v_pages = np.array(v_pages, copy=True)
    num_pages = k_pages.shape[0]
    rs = [int(v) for v in row_start]
    for s in range(len(rs) - 1):
        cap = PAGE * len(page_table[s])
        for j in range(min(rs[s + 1] - rs[s], MAX_ROWS)):
            p = int(seq_len[s]) + j
            if not 0 <= p < cap:
                continue
            pg, off = slot_location(page_table, s, p)
            if not 0 <= pg < num_pages:
                continue
            k_pages[pg, :, off, :] = k_new[rs[s] + j]
            v_pages[pg, :, :, off] = v_new[rs[s] + j]
    return k_pages, v_pages


def commit(seq_len, accept_len):
    """(new committed lengths, new position ids)."""
    c = np.asarray(seq_len, dtype=np.int64) + np.asarray(accept_len, dtype=np.int64) + 1
    return c.astype(np.int32), c.astype(np.int32)

