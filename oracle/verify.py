"""Verification of a block of drafted tokens (oracle; test infrastructure).

Layout shared with the library's verify call: sequence ``s`` owns target
rows ``row_start[s] .. row_start[s+1]-1`` (``k_s + 1`` rows; row ``j`` holds
the target's logits for the token after input ``j``), and draft entries
``row_start[s]-s .. row_start[s+1]-s-2`` (``k_s`` drafts ``d_1..d_k`` and, for
sampling, the drafter's logits for each of them).  Output: the accepted
prefix length ``a_s`` and the ``a_s + 1`` emitted tokens, padded with -1.

Greedy (temperature 0).  The target picks the highest logit, ties going to
the lowest token id (ramgpt.org, "When Lossless Speculation Stops Being
Lossless on Blackwell", section "The Hidden Contract Behind Lossless
Speculation": ordinary decoding selects the maximum-probability token and
the verifier must reproduce it).  Draft ``d_j`` is accepted while it equals
the target's choice after input ``j-1``; the first mismatch is replaced by
the target's choice, and if every draft matches the target's choice after
the last draft is emitted as a bonus (proofoftech.org, "'Lossless'
speculative decoding is a property of the math, not your deployment.",
opening section: accept the prefix it can and correct the first token it
cannot).

Sampling (temperature T > 0).  With p_j = softmax(z_target[j-1] / T) and
q_j = softmax(z_draft[j] / T), draft x = d_j is accepted when
u < min(1, p_j(x) / q_j(x)); on the first rejection a token is drawn from
the normalised residual max(0, p_j - q_j) by inverse CDF over ascending ids;
if all drafts are accepted a bonus token is drawn from p_{k+1}.  This is
the accept-or-reject rule of Leviathan et al. and Chen et al. that the
pages cite as distribution-preserving "within hardware numerics"
(proofoftech.org, same page, section "Lossless is a theorem, and theorems
have hypotheses").  Uniforms come from ``philox.uniform`` keyed by
(seed, sequence id, position, stream); position of draft j is
``pos0[s] + j - 1``.
"""
from __future__ import annotations

import numpy as np

from . import philox

MAX_OUT = 9  # at most 8 drafts + 1 correction/bonus token


# ------------------------------------------------------------------ greedy

def argmax_lowest(z) -> int:
    """Smallest index of the maximum (NaN never wins; -0 ties +0)."""
    z = np.asarray(z, dtype=np.float64)
    zz = np.where(np.isnan(z), -np.inf, z)
    best = zz.max()
    return int(np.flatnonzero(zz == best)[0])


def top2_margin(z) -> float:
    """max - second-largest value of a logit row (0 for an exact tie)."""
    z = np.sort(np.asarray(z, dtype=np.float64))
    return float(z[-1] - z[-2])


def greedy_accept(targets, drafts):
    """targets t_0..t_k, drafts d_1..d_k -> (a, emitted tokens)."""
    k = len(drafts)
    a = 0
    while a < k and int(drafts[a]) == int(targets[a]):
        a += 1
    return a, [int(v) for v in drafts[:a]] + [int(targets[a])]


def _seq_ranges(row_start):
    rs = [int(v) for v in row_start]
    for s in range(len(rs) - 1):
        yield s, rs[s], rs[s + 1] - rs[s] - 1  # (seq, first target row, k)


def verify_greedy(target_logits, drafts, row_start):
    """Greedy verify of a ragged batch.  Returns (accept_len[B],
    out_tokens[B][9], argmax tokens per target row, top-2 margins)."""
    z = np.asarray(target_logits)
    B = len(row_start) - 1
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, MAX_OUT), -1, dtype=np.int32)
    t_all = np.array([argmax_lowest(row) for row in z], dtype=np.int32)
    margins = np.array([top2_margin(row) for row in z])
    for s, r0, k in _seq_ranges(row_start):
        d = np.asarray(drafts)[r0 - s: r0 - s + k]
        a, em = greedy_accept(t_all[r0:r0 + k + 1], d)
        acc[s] = a
        out[s, :len(em)] = em
    return acc, out, t_all, margins


def recheck_rows(margins, row_start, accept_len, threshold: float):
    """Margin-gated re-check of a greedy verify.  A step whose two best logits
    lie within a tiny distance of each other is the one where the last
    rounding digit decides the token (tokenstrom.com, "'Lossless,' but not
    quite", section "Why the math checks out and the text still flips");
    re-checking only such uncertain steps is the remedy the page names
    (same page, section "What the big servers offer and what it costs").
    For sequence s the rows that decided its emitted tokens are its target
    rows 0..a_s; the result is the first of them whose top-2 margin is below
    `threshold`, as a row offset within the sequence, or -1."""
    out = np.full(len(row_start) - 1, -1, dtype=np.int32)
    for s, r0, k in _seq_ranges(row_start):
        for j in range(int(accept_len[s]) + 1):
            if margins[r0 + j] < threshold:
                out[s] = j
                break
    return out


# ------------------------------------------------------------------ sampling

def softmax(z, temperature: float) -> np.ndarray:
    x = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def inverse_cdf(weights, u: float):
    """Smallest v with sum_{w<=v} weights_w > u * sum(weights), and the
    distance from that threshold to the nearest cumulative step (relative
    to the total), for exclusion of ties with the GPU's fp32 scan."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    S = c[-1]
    t = u * S
    v = int(np.searchsorted(c, t, side="right"))
    v = min(v, len(c) - 1)
    lo = c[v - 1] if v > 0 else 0.0
    gap = min(abs(t - lo), abs(c[v] - t)) / S
    return v, gap


def draw_candidates(weights, u: float, tol: float):
    """Every entry the inverse-CDF draw of ``inverse_cdf`` selects for some
    threshold within ``tol * S`` of u * S: the entries of positive weight
    whose cumulative interval [c[v-1], c[v]) meets [u S - tol S, u S + tol
    S].  For u < 1 this holds the last entry of positive weight whenever
    the window reaches S (its interval ends at S > u S - tol S), the entry
    a threshold clamped at the top selects.  A draw computed with rounding
    errors below tol * S lands on one of them."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    S = c[-1]
    lo_t, hi_t = (u - tol) * S, (u + tol) * S
    prev = np.concatenate([[0.0], c[:-1]])
    return tuple(int(v) for v in np.nonzero((w > 0) & (c > lo_t) & (prev <= hi_t))[0])


def accept_or_resample(p, q, x, u, u2):
    """One speculative decision, vectorised over independent trials.

    p, q: fp64 distributions over the vocabulary; x, u, u2: arrays of drafted
    tokens, accept uniforms and resample uniforms.  Returns (token, accepted).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    x = np.asarray(x)
    u = np.asarray(u, dtype=np.float64)
    u2 = np.asarray(u2, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(q[x] > 0, p[x] / np.where(q[x] > 0, q[x], 1.0), np.inf)
    accepted = u < np.minimum(1.0, ratio)
    r = np.maximum(0.0, p - q)
    if r.sum() == 0.0:
        r = p
    c = np.cumsum(r)
    v = np.minimum(np.searchsorted(c, u2 * c[-1], side="right"), len(c) - 1)
    return np.where(accepted, x, v), accepted


def verify_sampled(target_logits, draft_logits, drafts, row_start, seq_id, pos0,
                   temperature: float, seed: int, tol: float = 1e-5):
    """Rejection-sampling verify of a ragged batch.

    Returns (accept_len[B], out_tokens[B][9], records) where records lists,
    per sequence, every decision taken as (kind, j, outcome, near,
    candidates): `near` tells whether it lies within ``tol`` of its
    threshold (an fp32 evaluation may decide it the other way); for a draw,
    `candidates` holds every token a threshold within ``tol`` of the drawn
    one selects (``draw_candidates``), for an accept test it is empty."""
    zt = np.asarray(target_logits)
    zd = np.asarray(draft_logits)
    dr = np.asarray(drafts)
    B = len(row_start) - 1
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, MAX_OUT), -1, dtype=np.int32)
    records = []
    for s, r0, k in _seq_ranges(row_start):
        sid, p0 = int(seq_id[s]), int(pos0[s])
        rec = []
        emitted = []
        a = 0
        while a < k:
            j = a + 1
            x = int(dr[r0 - s + a])
            p = softmax(zt[r0 + a], temperature)
            q = softmax(zd[r0 - s + a], temperature)
            u = philox.uniform(seed, sid, p0 + j - 1, philox.STREAM_ACCEPT)
            if 0 <= x < len(p):
                ratio = p[x] / q[x] if q[x] > 0 else np.inf
                near = abs(u - ratio) < tol * max(1.0, ratio) if np.isfinite(ratio) else False
                ok = u < min(1.0, ratio)
            else:
                # an id outside the vocabulary is not a token the target can
                # emit: never accepted, as a token of target probability 0
                near, ok = False, False
            rec.append(("accept", j, ok, near, ()))
            if not ok:
                r = np.maximum(0.0, p - q)
                if r.sum() == 0.0:
                    r = p
                u2 = philox.uniform(seed, sid, p0 + j - 1, philox.STREAM_SAMPLE)
                v, gap = inverse_cdf(r, u2)
                rec.append(("resample", j, v, gap < tol, draw_candidates(r, u2, tol)))
                emitted.append(v)
                break
            emitted.append(x)
            a += 1
        if a == k:
            p = softmax(zt[r0 + k], temperature)
            u2 = philox.uniform(seed, sid, p0 + k, philox.STREAM_SAMPLE)
            v, gap = inverse_cdf(p, u2)
            rec.append(("bonus", k + 1, v, gap < tol, draw_candidates(p, u2, tol)))
            emitted.append(v)
        acc[s] = a
        out[s, :len(emitted)] = emitted
        records.append(rec)
    return acc, out, records
