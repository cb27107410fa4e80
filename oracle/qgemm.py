"""Block-quantised matrix times activation rows (oracle; test
infrastructure), for the 4-bit block format and the 6-bit super-block
format (see ``formats``).

Computes ``y[c][r] = sum_k W[r][k] * x[c][k]`` for every activation row
``c < n`` and output row ``r < N``, with ``W`` decoded exactly from its codes
(see ``formats.dequant``) and the sum taken in fp64.  This is the quantity a
batched verify pass and repeated width-one passes must both produce
(ramgpt.org, "When Lossless Speculation Stops Being Lossless on Blackwell",
section "Quantized Matrix Multiplication Shows the Same Class of Failure":
a batched matrix multiplication is compared with single-column ones over the
same weights; tokenstrom.com, "'Lossless,' but not quite", section "Why the
math checks out and the text still flips": the quantised mat-vec must not
change its partial-sum order with the number of tokens).

The definition has no order of summation; fp64 makes the oracle's own
rounding negligible against the fp32 results it is compared with.  Rows are
decoded in slabs only to bound memory; the slabs do not change the result.
"""
from __future__ import annotations

import numpy as np

from .formats import activations_to_f64, dequant, dequant_q6


def qgemm_w4(codes, scale_min, x, x_dtype: str, rows: slice | np.ndarray | None = None,
             slab: int = 4096) -> np.ndarray:
    """Return fp64 ``y[n][N]`` (or ``y[n][len(rows)]`` for a subset of rows)."""
    codes = np.asarray(codes)
    scale_min = np.asarray(scale_min)
    xs = activations_to_f64(x, x_dtype)
    if xs.ndim == 1:
        xs = xs[None, :]
    N = codes.shape[0]
    idx = np.arange(N) if rows is None else np.arange(N)[rows]
    out = np.empty((xs.shape[0], idx.size), dtype=np.float64)
    for s in range(0, idx.size, slab):
        sel = idx[s:s + slab]
        W = dequant(codes[sel], scale_min[sel])
        out[:, s:s + sel.size] = xs @ W.T
    return out


def qgemm_q6(ql, qh, sc, d, x, x_dtype: str, rows: slice | np.ndarray | None = None,
             slab: int = 4096) -> np.ndarray:
    """The same product for 6-bit super-block weights (``formats.dequant_q6``):
    fp64 ``y[n][N]`` or ``y[n][len(rows)]``."""
    ql, qh, sc, d = (np.asarray(a) for a in (ql, qh, sc, d))
    xs = activations_to_f64(x, x_dtype)
    if xs.ndim == 1:
        xs = xs[None, :]
    N = ql.shape[0]
    idx = np.arange(N) if rows is None else np.arange(N)[rows]
    out = np.empty((xs.shape[0], idx.size), dtype=np.float64)
    for s in range(0, idx.size, slab):
        sel = idx[s:s + slab]
        W = dequant_q6(ql[sel], qh[sel], sc[sel], d[sel])
        out[:, s:s + sel.size] = xs @ W.T
    return out
