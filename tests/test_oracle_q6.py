"""Pins for the oracle's 6-bit super-block format and its matrix product
(CPU only).

Each check reaches the answer another way than the oracle does: a reduction
to the 4-bit block format (itself pinned in test_oracle_qgemm.py), a
hand-worked row, exact integer arithmetic on the codes as generated (before
they were laid out in bytes), a pure-Python decode by division and modulo,
and a hand-written packer for the library's packed layout.
"""
import struct

import numpy as np
import pytest

import synth
from oracle import formats, qgemm


def _half(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def _brute_w(ql, qh, sc, d, r, k):
    """One weight by arithmetic on the byte values: the low four bits of
    element k are byte k//2 modulo 16 (k even) or divided by 16 (k odd); the
    high two bits are byte k//4 divided by 4**(k%4), modulo 4."""
    b = int(ql[r][k // 2])
    lo = b % 16 if k % 2 == 0 else b // 16
    hi = (int(qh[r][k // 4]) // (4 ** (k % 4))) % 4
    q = lo + 16 * hi
    return _half(d[r][k // 256]) * int(sc[r][k // 16]) * (q - 32)


def test_brute_force_decode_and_product():
    g = synth.rng(300)
    N, K = 3, 512
    ql, qh, sc, d = synth.quant_weights_q6(N, K, g)
    W = formats.dequant_q6(ql, qh, sc, d)
    for r in range(N):
        for k in range(K):
            assert W[r, k] == _brute_w(ql, qh, sc, d, r, k), (r, k)
    x = g.standard_normal((2, K)).astype(np.float32)
    y = qgemm.qgemm_q6(ql, qh, sc, d, x, "f32")
    for c in range(2):
        for r in range(N):
            ref = sum(float(x[c, k]) * _brute_w(ql, qh, sc, d, r, k) for k in range(K))
            assert abs(y[c, r] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_reduces_to_the_4bit_format():
    """Codes below 16 (no high bits) with the two 16-value halves of every
    32-value block sharing one scale: w = (d s) q - 32 (d s), which is the
    4-bit format with block scale d s and minimum -32 d s (both exact in
    fp16 for d a power of two and small s)."""
    g = synth.rng(301)
    N, K = 5, 768
    q = g.integers(0, 16, size=(N, K))
    s32 = g.integers(-6, 7, size=(N, K // 32))
    sc = np.repeat(s32, 2, axis=1)
    d = np.full((N, K // 256), 2.0 ** -9, dtype=np.float16)
    ql, qh, sc8, db = synth.q6_from_codes(q, sc, d)
    assert not qh.any()
    w6 = formats.dequant_q6(ql, qh, sc8, db)
    ds = (2.0 ** -9) * s32
    codes4, sm4 = synth.quant_weights_from(q, ds.astype(np.float16), (-32.0 * ds).astype(np.float16))
    assert np.array_equal(ds.astype(np.float16).astype(np.float64), ds)  # the scales are exact
    assert np.array_equal(w6, formats.dequant(codes4, sm4))


def test_hand_worked_row():
    """One row of 256 inputs: d = 0.5, s = 3 on sub-block 0, -2 on sub-block
    1 and 1 elsewhere; every code is 32 (weight 0) except
      element 0:   low 5,  high 2 -> q 37 -> 0.5 *  3 *   5 =   7.5
      element 1:   low 15, high 3 -> q 63 -> 0.5 *  3 *  31 =  46.5
      element 2:   low 0,  high 0 -> q 0  -> 0.5 *  3 * -32 = -48
      element 3:   low 0,  high 1 -> q 16 -> 0.5 *  3 * -16 = -24
      element 16:  low 1,  high 1 -> q 17 -> 0.5 * -2 * -15 =  15
      element 255: low 2,  high 2 -> q 34 -> 0.5 *  1 *   2 =   1
    Code 32 is low 0, high 2: low bytes 0x00 and high bytes 0b10101010."""
    ql = np.zeros((1, 128), dtype=np.uint8)
    qh = np.full((1, 64), 0xAA, dtype=np.uint8)
    ql[0, 0] = 5 | (15 << 4)            # elements 0, 1
    ql[0, 1] = 0                        # elements 2, 3
    qh[0, 0] = 2 | (3 << 2) | (0 << 4) | (1 << 6)   # elements 0..3
    ql[0, 8] = 1                        # element 16 (low), element 17 low 0
    qh[0, 4] = 1 | (2 << 2) | (2 << 4) | (2 << 6)   # elements 16..19
    ql[0, 127] = 2 << 4                 # element 255 (high nibble), element 254 low 0
    qh[0, 63] = 2 | (2 << 2) | (2 << 4) | (2 << 6)  # elements 252..255, all high 2
    sc = np.ones((1, 16), dtype=np.int8)
    sc[0, 0], sc[0, 1] = 3, -2
    d = np.array([[0x3800]], dtype=np.uint16)       # fp16 0.5
    w = formats.dequant_q6(ql, qh, sc, d)[0]
    expect = np.zeros(256)
    expect[[0, 1, 2, 3, 16, 255]] = [7.5, 46.5, -48.0, -24.0, 15.0, 1.0]
    assert np.array_equal(w, expect)


def test_subblock_and_superblock_indexing():
    """All codes 33 (q - 32 = 1): w[k] = d[k // 256] * s[k // 16]; a sub-block
    of 32 or a super-block of 128 would move the scale boundaries."""
    g = synth.rng(302)
    N, K = 4, 1024
    sc = g.integers(-128, 128, size=(N, K // 16))
    d = g.uniform(0.5, 2.0, size=(N, K // 256)).astype(np.float16)
    ql, qh, sc8, db = synth.q6_from_codes(np.full((N, K), 33), sc, d)
    w = formats.dequant_q6(ql, qh, sc8, db)
    k = np.arange(K)
    assert np.array_equal(w, d.astype(np.float64)[:, k // 256] * sc[:, k // 16])


def test_integer_exact_product():
    """d = 1, small integer scales and activations: y is an exact integer,
    computed here with int64 arithmetic from the codes as generated."""
    g = synth.rng(303)
    N, K, n = 37, 1280, 3
    q = g.integers(0, 64, size=(N, K))
    sc = g.integers(-3, 4, size=(N, K // 16))
    d = np.ones((N, K // 256), dtype=np.float16)
    xi = g.integers(-4, 5, size=(n, K))
    Wi = np.repeat(sc, 16, axis=1) * (q - 32)
    yi = xi @ Wi.T
    y = qgemm.qgemm_q6(*synth.q6_from_codes(q, sc, d), xi.astype(np.float32), "f32")
    assert np.array_equal(y, yi.astype(np.float64))


def test_one_hot_selects_column_and_extremes():
    g = synth.rng(304)
    N, K = 9, 256
    q = g.integers(0, 64, size=(N, K))
    q[0, :] = 0      # the most negative offset, -32
    q[1, :] = 63     # the most positive, +31
    sc = g.integers(-128, 128, size=(N, K // 16))
    sc[:2, :] = -128
    d = np.full((N, 1), 2.0 ** -12, dtype=np.float16)
    ql, qh, sc8, db = synth.q6_from_codes(q, sc, d)
    W = formats.dequant_q6(ql, qh, sc8, db)
    assert np.all(W[0] == 2.0 ** -12 * -128 * -32) and np.all(W[1] == 2.0 ** -12 * -128 * 31)
    for k in (0, 15, 16, 200, 255):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        assert np.array_equal(qgemm.qgemm_q6(ql, qh, sc8, db, x, "f32")[0], W[:, k])


def test_row_subset_matches_full():
    g = synth.rng(305)
    N, K = 70, 512
    w = synth.quant_weights_q6(N, K, g)
    x = synth.activations(2, K, "bf16", g)
    full = qgemm.qgemm_q6(*w, x, "bf16")
    sel = np.array([0, 13, 69, 40])
    assert np.array_equal(qgemm.qgemm_q6(*w, x, "bf16", rows=sel), full[:, sel])
    assert np.array_equal(qgemm.qgemm_q6(*w, x, "bf16", slab=16), full)


# ------------------------------------------------------ packed layout

def _pack_by_hand(q, sc, d, N, K):
    """The packed 6-bit layout written element by element from its
    description: per (16-row tile, 128-input step) a 1536-byte code record
    (lane l = i + 16g: code word 2p + h holds inputs 16(2p + g//2) + 8(g%2)
    + 4h + e of the step, packed three words per four with the fourth
    word's bits on top), a 128-byte sub-scale record (byte 8i + 4h + p = s
    of sub-block 2p + h, plus 128), per (tile, super-block) a 32-byte d
    record; rows past N are codes 0, scale bytes 128, d 0."""
    ntiles, nsteps, nsup = -(-N // 16), K // 128, K // 256
    rows = ntiles * 16
    qp = np.zeros((rows, K), dtype=np.int64)
    qp[:N] = q
    sp = np.zeros((rows, K // 16), dtype=np.int64)
    sp[:N] = sc
    dp = np.zeros((rows, nsup), dtype=np.uint16)
    dp[:N] = d
    codes = bytearray(ntiles * nsteps * 1536)
    subs = bytearray(ntiles * nsteps * 128)
    sups = bytearray(ntiles * nsup * 32)
    for T in range(ntiles):
        for S in range(nsteps):
            base = (T * nsteps + S) * 1536
            for lane in range(64):
                i, g = lane % 16, lane // 16
                r = 16 * T + i

                def word(wi, e):  # byte e of code word wi = 2p + h
                    p, h = wi // 2, wi % 2
                    return int(qp[r, 128 * S + 16 * (2 * p + g // 2) + 8 * (g % 2) + 4 * h + e])

                for j in range(2):
                    for k in range(3):
                        packed = [word(4 * j + k, e) | (((word(4 * j + 3, e) >> (2 * k)) & 3) << 6)
                                  for e in range(4)]
                        slot = 3 * j + k     # P00 P01 P02 P10 | P11 P12
                        off = base + 16 * lane + 4 * slot if slot < 4 else base + 1024 + 8 * lane + 4 * (slot - 4)
                        codes[off:off + 4] = bytes(packed)
            for i in range(16):
                for h in range(2):
                    for p in range(4):
                        subs[(T * nsteps + S) * 128 + 8 * i + 4 * h + p] = int(sp[16 * T + i, 8 * S + 2 * p + h]) + 128
        for U in range(nsup):
            for i in range(16):
                o = (T * nsup + U) * 32 + 2 * i
                sups[o:o + 2] = struct.pack("<H", int(dp[16 * T + i, U]))
    return np.frombuffer(bytes(codes + subs + sups), dtype=np.uint8)


@pytest.mark.parametrize("N,K", [(16, 256), (21, 512)])
def test_packed_layout_reader_roundtrip(N, K):
    g = synth.rng(306 + N)
    q = g.integers(0, 64, size=(N, K))
    sc = g.integers(-128, 128, size=(N, K // 16))
    d = g.uniform(0.1, 1.0, size=(N, K // 256)).astype(np.float16)
    ql, qh, sc8, db = synth.q6_from_codes(q, sc, d)
    buf = _pack_by_hand(q, sc, db, N, K)
    assert buf.size == formats.q6_packed_sections(N, K)[3]
    r = formats.unpack_packed_q6(buf, N, K)
    for a, b in zip(r, (ql, qh, sc8, db)):
        assert np.array_equal(a, b)
    if N % 16:
        # a planted non-zero code in a padding row must be caught
        bad = buf.copy()
        T = N // 16
        bad[(T * (K // 128)) * 1536 + 16 * 15] = 1   # lane 15 = row 16T + 15 >= N
        with pytest.raises(AssertionError):
            formats.unpack_packed_q6(bad, N, K)
