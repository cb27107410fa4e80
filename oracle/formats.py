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

The 6-bit super-block format (the pages name Q6_K beside Q4_K as the
formats whose mat-vec changes its summation order with the token count:
tokenstrom.com, "'Lossless,' but not quite", section "Why the math checks
out and the text still flips").  The pages give no layout; the reading is
the K-quant structure that name stands for: a row is split into
super-blocks of 256 inputs with one fp16 scale ``d`` each, every
super-block into 16 sub-blocks of 16 inputs with one signed 8-bit scale
``s`` each, and ``w = d * s * (q - 32)`` for a code ``q`` in 0..63.  Codes
are stored as a low-nibble array (element ``2t`` in the low nibble of byte
``t``) and a high-bits array (element ``4t+i`` in bits ``2i, 2i+1`` of
byte ``t``).
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


# ------------------------------------------------------- 6-bit super-blocks

def unpack_q6_codes(ql, qh) -> np.ndarray:
    """(uint8[N][K/2], uint8[N][K/4]) -> int64[N][K] codes in 0..63."""
    lo = unpack_codes(ql)
    h = np.asarray(qh, dtype=np.uint8).astype(np.int64)
    N, quarter = h.shape
    assert lo.shape == (N, 4 * quarter)
    hi = np.empty((N, 4 * quarter), dtype=np.int64)
    for i in range(4):
        hi[:, i::4] = (h >> (2 * i)) & 3
    return lo + 16 * hi


def dequant_q6(ql, qh, sc, d) -> np.ndarray:
    """W[r][k] = d[r][k // 256] * s[r][k // 16] * (q[r][k] - 32), in fp64."""
    q = unpack_q6_codes(ql, qh).astype(np.float64)
    N, K = q.shape
    s = np.asarray(sc, dtype=np.int8).astype(np.float64)
    dd = f16_to_f64(np.asarray(d, dtype=np.uint16))
    assert s.shape == (N, K // 16) and dd.shape == (N, K // 256)
    per_sub = (dd[:, :, None] * s.reshape(N, K // 256, 16)).reshape(N, K // 16)
    return (per_sub[:, :, None] * (q.reshape(N, K // 16, 16) - 32.0)).reshape(N, K)


def q6_packed_sections(N: int, K: int):
    """Byte offsets and total size of the library's packed 6-bit layout:
    (codes offset, sub-scale offset, super-scale offset, total)."""
    ntiles = -(-N // 16)
    nsteps, nsup = K // 128, K // 256
    codes = ntiles * nsteps * 1536
    subs = ntiles * nsteps * 128
    sups = ntiles * nsup * 32
    return 0, codes, codes + subs, codes + subs + sups


def unpack_packed_q6(packed, N: int, K: int):
    """Decode the library's packed 6-bit layout back to (ql, qh, sc, d).

    Tiles of 16 rows, steps of 128 inputs (eight sub-blocks, four pairs),
    K % 256 == 0.  Section 1, one 1536-byte record per (tile T, step S):
    lane l = i + 16g (row 16T+i) has eight code words w[0..7]; byte e of
    w[2p + h] is the code of input 128S + 16(2p + g//2) + 8(g%2) + 4h + e.
    They are stored as six words: in group j (j = 0, 1), word k (k = 0..2)
    has byte e = w[4j+k] byte e | (bits 2k, 2k+1 of w[4j+3] byte e) << 6;
    the record holds the lanes' (P00, P01, P02, P10) as 16 bytes per lane,
    then (P11, P12) as 8 bytes per lane.  Section 2, one 128-byte record per
    (T, S): byte 8i + 4h + p = s of sub-block 8S + 2p + h of row 16T+i, plus
    128.  Section 3, one 32-byte record per (T, super-block): the fp16 d of
    each row.  Rows past N carry codes 0, scale bytes 128 and d = 0
    (checked)."""
    buf = np.asarray(packed, dtype=np.uint8).reshape(-1)
    o_codes, o_sub, o_sup, total = q6_packed_sections(N, K)
    assert buf.size == total
    ntiles, nsteps, nsup = -(-N // 16), K // 128, K // 256
    rows = ntiles * 16
    q = np.zeros((rows, K), dtype=np.int64)
    sc = np.zeros((rows, K // 16), dtype=np.int64)
    d = np.zeros((rows, nsup), dtype=np.uint16)
    for T in range(ntiles):
        for S in range(nsteps):
            rec = buf[o_codes + (T * nsteps + S) * 1536:][:1536]
            first = rec[:1024].reshape(64, 4, 4).astype(np.int64)   # lane, word, byte
            second = rec[1024:].reshape(64, 2, 4).astype(np.int64)
            for l in range(64):
                i, g = l % 16, l // 16
                P = [first[l, 0], first[l, 1], first[l, 2], first[l, 3], second[l, 0], second[l, 1]]
                w = [None] * 8
                for j in range(2):
                    last = np.zeros(4, dtype=np.int64)
                    for k in range(3):
                        w[4 * j + k] = P[3 * j + k] & 63
                        last |= (P[3 * j + k] >> 6) << (2 * k)
                    w[4 * j + 3] = last
                for p in range(4):
                    for h in range(2):
                        base = 128 * S + 16 * (2 * p + g // 2) + 8 * (g % 2) + 4 * h
                        q[16 * T + i, base:base + 4] = w[2 * p + h]
            srec = buf[o_sub + (T * nsteps + S) * 128:][:128].reshape(16, 2, 4).astype(np.int64)
            for h in range(2):
                for p in range(4):
                    sc[16 * T:16 * T + 16, 8 * S + 2 * p + h] = srec[:, h, p] - 128
        for U in range(nsup):
            d[16 * T:16 * T + 16, U] = buf[o_sup + (T * nsup + U) * 32:][:32].view(np.uint16)
    assert not q[N:].any() and not sc[N:].any() and not d[N:].any(), "nonzero padding"
    q = q[:N]
    lo, hi = q & 15, q >> 4
    ql = (lo[:, 0::2] | (lo[:, 1::2] << 4)).astype(np.uint8)
    qh = (hi[:, 0::4] | (hi[:, 1::4] << 2) | (hi[:, 2::4] << 4) | (hi[:, 3::4] << 6)).astype(np.uint8)
    return ql, qh, sc[:N].astype(np.int8), d[:N]
