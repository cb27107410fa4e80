"""Causal decode attention over a paged cache (oracle; test infrastructure).

For sequence ``s`` whose verify block has ``n_s`` query rows, row ``i`` sits
at position ``q_pos[s] + i`` and attends to the cached positions
``0 .. q_pos[s] + i`` (the block's own keys and values are appended to the
cache before attention runs).  For query head ``h`` the key/value head is
``g = h // (Hq // Hkv)`` (grouped heads are contiguous), and

    score_j = scale * sum_d Q[h][d] * K_j[g][d]
    out[h]  = sum_j softmax(score)_j * V_j[g]

over the visible positions only.  Position ``p`` of sequence ``s`` lives in
page ``page_table[s][p // 16]`` at offset ``p % 16``; the key cache is
``[page][Hkv][16][D]`` and the value cache ``[page][Hkv][D][16]``.  A
position past the table or on a page whose id lies outside [0, num_pages)
holds nothing and takes no part in the softmax; a row that sees no position
gives zeros (the library's reading of such entries, which the pages never
have).

This is the plain definition the batched and width-one evaluations must
agree on (ramgpt.org, "When Lossless Speculation Stops Being Lossless on
Blackwell", section "Flash Attention Changes Geometry With Batch Width":
tile geometry chosen by query width changes the KV traversal and the
reduction/combine order; tokenstrom.com, "'Lossless,' but not quite",
section "Why the math checks out and the text still flips": one token and a
batch take different attention kernels).  The per-sequence positions and
masks after ragged accepts follow proofoftech.org, "'Lossless' speculative
decoding is a property of the math, not your deployment.", section
"Batching breaks the implementation".

``decode_attn`` is the plain full-softmax definition.  ``decode_attn_chunked``
evaluates the same quantity as per-256-position-chunk partial results folded
in ascending chunk order with the log-sum-exp rule; it exists only so the
tests can pin the chunked formulation against the plain one.
"""
from __future__ import annotations

import numpy as np

from .formats import f16_to_f64

PAGE = 16
CHUNK = 256


def slot_location(page_table, s: int, p: int):
    """(page, offset) of position p of sequence s."""
    return int(page_table[s][p // PAGE]), p % PAGE


def gather_kv(k_pages, v_pages, page_table, s: int, g: int, length: int):
    """fp64 K[length][D] and V[length][D] of kv-head g of sequence s."""
    D = k_pages.shape[-1]
    K = np.empty((length, D))
    V = np.empty((length, D))
    for p in range(length):
        pg, off = slot_location(page_table, s, p)
        K[p] = f16_to_f64(k_pages[pg, g, off, :])
        V[p] = f16_to_f64(v_pages[pg, g, :, off])
    return K, V


def _rows(row_start):
    rs = [int(v) for v in row_start]
    for s in range(len(rs) - 1):
        for i in range(rs[s + 1] - rs[s]):
            yield s, i, rs[s] + i


def present_positions(page_table, num_pages: int, s: int, end: int):
    """Positions p < end of sequence s that hold a key and value: inside the
    table (p < 16 * max_pages) and on a page whose id lies in [0,
    num_pages).  A position outside the table or on an absent page is read
    as missing; the pages never have one, this is the library's reading of
    such entries."""
    cap = PAGE * len(page_table[s])
    return [p for p in range(max(0, min(end, cap)))
            if 0 <= int(page_table[s][p // PAGE]) < num_pages]


def decode_attn(q, k_pages, v_pages, page_table, q_pos, row_start, scale: float):
    """fp64 out[R][Hq][D] for q f16[R][Hq][D] (rows of all sequences).

    Row i of sequence s attends to the present positions (see
    ``present_positions``) before q_pos[s] + i + 1; a row with none gives
    zeros."""
    q = f16_to_f64(np.asarray(q))
    R, Hq, D = q.shape
    num_pages, Hkv = k_pages.shape[0], k_pages.shape[1]
    grp = Hq // Hkv
    out = np.zeros((R, Hq, D))
    cache = {}
    for s, i, r in _rows(row_start):
        n = int(row_start[s + 1]) - int(row_start[s])
        if s not in cache:  # the positions the block's last row sees
            cache[s] = present_positions(page_table, num_pages, s, int(q_pos[s]) + n)
        pos = cache[s]
        # the rows' visible positions are prefixes of the last row's
        m = int(np.searchsorted(pos, int(q_pos[s]) + i + 1))
        if m == 0:
            continue
        for g in range(Hkv):
            key = (s, g)
            if key not in cache:
                K = np.empty((len(pos), D))
                V = np.empty((len(pos), D))
                for e, p in enumerate(pos):
                    pg, off = slot_location(page_table, s, p)
                    K[e] = f16_to_f64(k_pages[pg, g, off, :])
                    V[e] = f16_to_f64(v_pages[pg, g, :, off])
                cache[key] = (K, V)
            K, V = cache[key]
            Kv, Vv = K[:m], V[:m]
            for hh in range(grp):
                h = g * grp + hh
                sc = scale * (Kv @ q[r, h])
                w = np.exp(sc - sc.max())
                out[r, h] = (w / w.sum()) @ Vv
    return out


def decode_attn_chunked(q, k_pages, v_pages, page_table, q_pos, row_start,
                        scale: float):
    """Same quantity as ``decode_attn`` via chunk partials and an in-order
    log-sum-exp fold.  Chunk c covers absolute positions [256c, 256c+256);
    a chunk's partial is (m_c, l_c, a_c) = (max score, sum of exp(score-m_c),
    sum of exp(score-m_c)*V) over its visible positions; the fold walks the
    chunks in ascending order: M' = max(M, m_c), L' = L e^{M-M'} + l_c
    e^{m_c-M'}, A' likewise, and the result is A/L."""
    q = f16_to_f64(np.asarray(q))
    R, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    grp = Hq // Hkv
    out = np.zeros((R, Hq, D))
    for s, i, r in _rows(row_start):
        vis = int(q_pos[s]) + i + 1
        for g in range(Hkv):
            K, V = gather_kv(k_pages, v_pages, page_table, s, g, vis)
            for hh in range(grp):
                h = g * grp + hh
                M, L, A = -np.inf, 0.0, np.zeros(D)
                for c0 in range(0, vis, CHUNK):
                    sc = scale * (K[c0:c0 + CHUNK] @ q[r, h])
                    mc = sc.max()
                    e = np.exp(sc - mc)
                    lc, ac = e.sum(), e @ V[c0:c0 + CHUNK]
                    Mn = max(M, mc)
                    a_old = np.exp(M - Mn) if M != -np.inf else 0.0
                    L = L * a_old + lc * np.exp(mc - Mn)
                    A = A * a_old + ac * np.exp(mc - Mn)
                    M = Mn
                out[r, h] = A / L
    return out


def softmax_weights(q_row_head, K):
    """Attention weights of one query against visible keys (scale 1)."""
    sc = np.asarray(K, dtype=np.float64) @ np.asarray(q_row_head, dtype=np.float64)
    w = np.exp(sc - sc.max())
    return w / w.sum()
