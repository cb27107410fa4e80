"""Row-wise operations of a synthetic decoder layer (oracle; test
infrastructure).

The verify pass evaluates a whole target model, not one matrix: the
batched-versus-single contract has to hold through every layer, and the
end-to-end check is that speculative output equals serial greedy decoding
(ramgpt.org, "When Lossless Speculation Stops Being Lossless on Blackwell",
sections "Why Tiny Numerical Differences Can Change Entire Answers" and "A
Better Backend Test Matrix": end-to-end greedy generation equivalence).
The pages run Qwen-family models (tokenstrom.com, "'Lossless,' but not
quite", section "What the measurements show"), whose layers chain RMS
normalisation, rotary position embedding and a SiLU-gated MLP around the
quantised projections; the pages give no formulas for these, so the plain
textbook definitions are used (the readings are listed in the design
notes): RMSNorm y = x / sqrt(mean(x^2) + eps) * w; rotary embedding in the
rotate-half form with frequencies theta^(-2i/D); SiLU(g) * u with SiLU(g) =
g / (1 + e^-g).

All arithmetic is fp64 from the exact values of the inputs.
"""
from __future__ import annotations

import numpy as np


def embed(tokens, table_f64):
    """Rows of an embedding table; ids outside [0, V) give zero rows."""
    table = np.asarray(table_f64, dtype=np.float64)
    V, H = table.shape
    out = np.zeros((len(tokens), H))
    for r, t in enumerate(tokens):
        if 0 <= int(t) < V:
            out[r] = table[int(t)]
    return out


def rmsnorm(h, w, eps: float):
    """x / sqrt(mean(x^2) + eps) * w for every row x of h."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * w


def rope_angles(pos: int, D: int, theta: float):
    """Rotation angles of position `pos` for the D/2 frequency pairs."""
    i = np.arange(D // 2, dtype=np.float64)
    return float(pos) * theta ** (-2.0 * i / D)


def rope(x, pos: int, theta: float):
    """Rotary embedding of one head vector x (length D) at position pos in
    the rotate-half form: the pair (x[i], x[i + D/2]) is rotated by angle
    pos * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    a = rope_angles(pos, D, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_qkv(qkv, positions, Hq: int, Hkv: int, D: int, theta: float):
    """Split rows of [q heads | k heads | v heads] and rotate q and k.
    Returns (q [R][Hq][D], k [R][Hkv][D], v [R][Hkv][D])."""
    qkv = np.asarray(qkv, dtype=np.float64)
    R = qkv.shape[0]
    q = qkv[:, : Hq * D].reshape(R, Hq, D)
    k = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(R, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(R, Hkv, D)
    qr = np.stack([rope(q[r], int(positions[r]), theta) for r in range(R)]) if R else q
    kr = np.stack([rope(k[r], int(positions[r]), theta) for r in range(R)]) if R else k
    return qr, kr, v.copy()


def silu_mul(gu, F: int):
    """SiLU(g) * u for rows [g (F values) | u (F values)]."""
    gu = np.asarray(gu, dtype=np.float64)
    g, u = gu[:, :F], gu[:, F:]
    return g / (1.0 + np.exp(-g)) * u
