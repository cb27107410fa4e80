"""Pins for the oracle's 4-bit block matrix product (CPU only).

Each check is independent of the oracle's own code path: a pure-Python
brute force that decodes nibbles and fp16 bits another way, exact integer
arithmetic, and special cases with a known answer.
"""
import struct

import numpy as np
import pytest

import synth
from oracle import formats, qgemm


def _half(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def _brute(codes, sm, x_rows):
    """y[c][r] by explicit loops: nibble k of row r is byte k//2 taken
    modulo 16 (even k) or divided by 16 (odd k)."""
    N = len(codes)
    K = 2 * len(codes[0])
    out = []
    for xr in x_rows:
        row = []
        for r in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(codes[r][k // 2])
                q = byte % 16 if k % 2 == 0 else byte // 16
                d = _half(sm[r][k // 32][0])
                m = _half(sm[r][k // 32][1])
                acc += (d * q + m) * float(xr[k])
            row.append(acc)
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("N,K,n", [(7, 32, 1), (16, 64, 3), (33, 96, 8), (5, 64, 5)])
def test_brute_force_f32(N, K, n):
    g = synth.rng(100 + N)
    codes, sm = synth.quant_weights(N, K, g)
    x = synth.activations(n, K, "f32", g)
    ref = _brute(codes.tolist(), sm.tolist(), [list(map(float, r)) for r in x])
    got = qgemm.qgemm_w4(codes, sm, x, "f32")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_bf16():
    g = synth.rng(7)
    N, K, n = 12, 64, 4
    codes, sm = synth.quant_weights(N, K, g)
    xb = synth.activations(n, K, "bf16", g)
    # bf16 bits -> value through struct (upper half of an fp32)
    xv = [[struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in row] for row in xb]
    ref = _brute(codes.tolist(), sm.tolist(), xv)
    got = qgemm.qgemm_w4(codes, sm, xb, "bf16")
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_integer_exact():
    """d = 1, m = -8, x in {-4..4}: every weight is q-8 and every sum an
    integer, so the fp64 oracle must equal Python integer arithmetic."""
    g = synth.rng(3)
    N, K, n = 40, 256, 8
    q = g.integers(0, 16, size=(N, K))
    d = np.ones((N, K // 32), dtype=np.float16)
    m = np.full((N, K // 32), -8.0, dtype=np.float16)
    codes, sm = synth.quant_weights_from(q, d, m)
    xi = g.integers(-4, 5, size=(n, K))
    exact = [[sum(int(q[r, k] - 8) * int(xi[c, k]) for k in range(K)) for r in range(N)]
             for c in range(n)]
    got = qgemm.qgemm_w4(codes, sm, xi.astype(np.float32), "f32")
    assert np.array_equal(got, np.array(exact, dtype=np.float64))


def test_one_hot_selects_column():
    g = synth.rng(11)
    N, K = 20, 128
    codes, sm = synth.quant_weights(N, K, g)
    for k in (0, 1, 31, 32, 77, 127):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        got = qgemm.qgemm_w4(codes, sm, x, "f32")[0]
        byte = codes[:, k // 2].astype(np.int64)
        qk = byte % 16 if k % 2 == 0 else byte // 16
        d = sm[:, k // 32, 0].view(np.float16).astype(np.float64)
        m = sm[:, k // 32, 1].view(np.float16).astype(np.float64)
        assert np.array_equal(got, d * qk + m)


def test_all_codes_eight_give_zero():
    g = synth.rng(5)
    codes, sm = synth.quant_weights(9, 96, g, codes_fill=8)
    x = synth.activations(3, 96, "f32", g)
    assert np.array_equal(qgemm.qgemm_w4(codes, sm, x, "f32"), np.zeros((3, 9)))


def test_unpack_roundtrip_and_nibble_order():
    g = synth.rng(2)
    q = g.integers(0, 16, size=(6, 64))
    d = np.full((6, 2), 0.5, dtype=np.float16)
    m = np.zeros((6, 2), dtype=np.float16)
    codes, sm = synth.quant_weights_from(q, d, m)
    assert np.array_equal(formats.unpack_codes(codes), q)
    # element 0 in the low nibble, element 1 in the high nibble
    assert codes[0, 0] == q[0, 0] + 16 * q[0, 1]
    assert np.array_equal(formats.dequant(codes, sm), 0.5 * q)


def test_row_subset_and_slabs_do_not_change_result():
    g = synth.rng(9)
    codes, sm = synth.quant_weights(300, 64, g)
    x = synth.activations(2, 64, "bf16", g)
    full = qgemm.qgemm_w4(codes, sm, x, "bf16", slab=4096)
    small = qgemm.qgemm_w4(codes, sm, x, "bf16", slab=17)
    sub = qgemm.qgemm_w4(codes, sm, x, "bf16", rows=np.array([5, 299, 0]))
    assert np.array_equal(full, small)
    assert np.array_equal(sub, full[:, [5, 299, 0]])


def _pack_by_hand(codes, sm, N, K):
    """Packed layout written element by element from its definition."""
    nb = K // 32
    nsteps = -(-nb // 4)
    ntiles = -(-N // 16)
    cp = bytearray(ntiles * nsteps * 1024)
    sp = np.zeros(ntiles * nsteps * 16 * 8, dtype=np.uint16)
    for T in range(ntiles):
        for S in range(nsteps):
            for lane in range(64):
                i, g = lane % 16, lane // 16
                for j in range(4):
                    row, blk = 16 * T + i, 4 * S + j
                    if row >= N or blk >= nb:
                        continue
                    # the 8 codes of elements 8g..8g+7 of the block (element 2t in
                    # the low nibble of row-major byte t)
                    rb = [int(codes[row, 16 * blk + 4 * g + t]) for t in range(4)]
                    e = [(rb[k // 2] >> (4 * (k % 2))) & 15 for k in range(8)]
                    for b in range(4):
                        cp[((T * nsteps + S) * 64 + lane) * 16 + 4 * j + b] = e[b] | (e[b + 4] << 4)
            for i in range(16):
                for j in range(4):
                    row, blk = 16 * T + i, 4 * S + j
                    for e in range(2):
                        sp[((T * nsteps + S) * 16 + i) * 8 + 2 * j + e] = \
                            sm[row, blk, e] if row < N and blk < nb else 0
    return np.frombuffer(bytes(cp), dtype=np.uint8), sp


@pytest.mark.parametrize("N,K", [(16, 128), (5, 32), (33, 160), (17, 416)])
def test_packed_layout_reader_roundtrip(N, K):
    g = synth.rng(N * K)
    codes, sm = synth.quant_weights(N, K, g)
    cp, sp = _pack_by_hand(codes, sm, N, K)
    c2, s2 = formats.unpack_packed(cp, sp, N, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sm)
    # a planted non-zero padding byte is reported
    if N % 16:
        bad = cp.copy()
        bad[((N // 16) * (-(-(K // 32) // 4)) * 64 + 15) * 16] = 1
        with pytest.raises(AssertionError):
            formats.unpack_packed(bad, sp, N, K)
