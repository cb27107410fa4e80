"""Planting near-ties in bf16 hidden states (test infrastructure).

A near-tie is a logit row whose two largest entries differ by less than
1e-3: there the last bits of the arithmetic decide the argmax
(tokenstrom.com, "'Lossless,' but not quite", section "Why the math checks
out and the text still flips": batched and single evaluations flipped at
0.3-1.3 percent of steps).  Starting from the oracle's fp64 logits of a
hidden state, single bf16 coordinates are moved so that the top-two margin
lands in (0, 1e-3); all logits are updated through the changed
coordinate's weight column.  Everything here uses the oracle only.
"""
from __future__ import annotations

import numpy as np

from oracle import formats

TIE = 1e-3


def _bf16_round(v: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _bf16_val(bits) -> np.ndarray:
    return formats.bf16_to_f64(bits)


def weight_rows(codes, sm, rows) -> np.ndarray:
    return formats.dequant(codes[rows], sm[rows])


def weight_column(codes, sm, k: int) -> np.ndarray:
    byte = codes[:, k // 2].astype(np.int64)
    q = (byte & 15) if k % 2 == 0 else (byte >> 4)
    d = formats.f16_to_f64(sm[:, k // 32, 0])
    m = formats.f16_to_f64(sm[:, k // 32, 1])
    return d * q + m


def plant(codes, sm, x_bits: np.ndarray, z: np.ndarray, g: np.random.Generator,
          max_iter: int = 40):
    """Return (new bf16 bits of one hidden state, its updated fp64 logits).

    x_bits: uint16[K] bf16 hidden state; z: its fp64 logits (all V)."""
    x = x_bits.copy()
    z = z.copy()
    xv = _bf16_val(x)
    target = g.uniform(1e-4, 8e-4)
    for _ in range(max_iter):
        top = np.argpartition(-z, 2)[:2]
        a, b = (top[0], top[1]) if z[top[0]] >= z[top[1]] else (top[1], top[0])
        m = z[a] - z[b]
        if 0.0 < m < TIE:
            return x, z
        W = weight_rows(codes, sm, np.array([a, b]))
        delta = W[0] - W[1]
        ok = np.abs(delta) > 1e-12
        dx = np.where(ok, (target - m) / np.where(ok, delta, 1.0), 0.0)
        cand = np.clip(xv + dx, -4.0, 4.0)  # large gaps close over several steps
        nb = _bf16_round(cand)
        nv = _bf16_val(nb)
        got = m + (nv - xv) * delta
        bad = ~ok | ~np.isfinite(nv)
        err = np.where(bad, np.inf, np.abs(got - target))
        k = int(np.argmin(err))
        if not np.isfinite(err[k]):
            break
        col = weight_column(codes, sm, k)
        z = z + (nv[k] - xv[k]) * col
        x[k] = nb[k]
        xv[k] = nv[k]
    raise RuntimeError("could not plant a near-tie")
