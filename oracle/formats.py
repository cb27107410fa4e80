"""Exact decoding of the input formats into fp64 (oracle; test infrastructure).

The 4-bit block format: each output row of the weight matrix is split into
blocks of 32 consecutive input positions; every block carries an fp16 scale
``d`` and an fp16 minimum ``m`` and each weight is ``w = d*q + m`` for a code
``q`` in 0..15.  Codes are packed two per byte, element ``2t`` in the low
nibble of byte ``t`` and element ``2t+1`` in the high nibble.  The pages name
block-quantised formats of this family (tokenstrom.com, "'Lossless,' but not
quite", section "Why the math checks out and the text still flips": Q4_K and
Q6_K; ramgpt.org, "When Lossless Speculation Stops Being Lossless on
Blackwell", section "Quantized Matrix Multiplication Shows the Same Class of
Failure": IQ3_S and IQ4_XS); the sign convention ``d*q + m`` with a negative
minimum is the plain reading (with m = -8d it centres the codes on zero).
"""
from __future__ import annotations

import numpy as np


def f16_to_f64(bits_or_half) -> np.ndarray:
    a = np.asarray(bits_or_half)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    assert a.dtype == np.float16
    return a.astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def activations_to_f64(x, x_dtype: str) -> np.ndarray:
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == "bf16":
        return bf16_to_f64(x)
    raise ValueError(x_dtype)


def unpack_codes(codes) -> np.ndarray:
    """uint8[N][K/2] -> int64[N][K] codes in 0..15."""
    c = np.asarray(codes, dtype=np.uint8)
    N, half = c.shape
    q = np.empty((N, 2 * half), dtype=np.int64)
    q[:, 0::2] = c & 0x0F
    q[:, 1::2] = c >> 4
    return q


def dequant(codes, scale_min) -> np.ndarray:
    """W[r][32b+j] = d[r][b] * q[r][32b+j] + m[r][b], in fp64."""
    q = unpack_codes(codes).astype(np.float64)
    sm = np.asarray(scale_min, dtype=np.uint16)
    N, K = q.shape
    assert sm.shape == (N, K // 32, 2)
    d = f16_to_f64(sm[..., 0])
    m = f16_to_f64(sm[..., 1])
    qb = q.reshape(N, K // 32, 32)
    return (d[:, :, None] * qb + m[:, :, None]).reshape(N, K)
