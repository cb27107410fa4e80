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


def unpack_packed(codes_p, scales_p, N: int, K: int):
    """Decode the library's packed weight layout back to the row-major one.

    Packed layout (nb = K/32 blocks, steps of four blocks, tiles of 16 rows):
    codes: for tile T, step S and lane l = i + 16*g, 16 bytes whose bytes
    4j..4j+3 hold the codes of elements 8g..8g+7 of block 4S+j of row 16T+i,
    byte b carrying element 8g+b in its low nibble and element 8g+b+4 in its
    high nibble; scales: for tile T, step S and row i, the (d, m) fp16 pairs
    of blocks 4S..4S+3.  Returns (codes uint8[N][K/2], scale_min
    uint16[N][K/32][2]); padding (rows >= N, blocks >= nb) is checked to be
    zero."""
    nb = K // 32
    nsteps = -(-nb // 4)
    ntiles = -(-N // 16)
    cp = np.asarray(codes_p, dtype=np.uint8).reshape(ntiles, nsteps, 4, 16, 4, 4)
    # axes: tile, step, g, i, j, byte-in-k-group
    sp = np.asarray(scales_p).view(np.uint16).reshape(ntiles, nsteps, 16, 4, 2)
    # axes: tile, step, i, j, (d, m)
    codes = np.zeros((ntiles * 16, nsteps * 4, 4, 4), dtype=np.uint8)  # row, block, g, byte
    sm = np.zeros((ntiles * 16, nsteps * 4, 2), dtype=np.uint16)
    for T in range(ntiles):
        for S in range(nsteps):
            for g in range(4):
                for i in range(16):
                    for j in range(4):
                        pb = [int(v) for v in cp[T, S, g, i, j, :]]
                        e = [pb[b] & 15 for b in range(4)] + [pb[b] >> 4 for b in range(4)]
                        for t in range(4):  # row-major: byte t = e[2t] | e[2t+1] << 4
                            codes[16 * T + i, 4 * S + j, g, t] = e[2 * t] | (e[2 * t + 1] << 4)
            for i in range(16):
                for j in range(4):
                    sm[16 * T + i, 4 * S + j, :] = sp[T, S, i, j, :]
    assert not codes[N:].any() and not codes[:, nb:].any(), "nonzero padding"
    assert not sm[N:].any() and not sm[:, nb:].any(), "nonzero padding"
    return codes[:N, :nb].reshape(N, K // 2), sm[:N, :nb]
