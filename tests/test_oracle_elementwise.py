"""Pins of the row-wise oracle operations: closed forms, invariants and
special cases that a dropped term, a wrong sign or a swapped half breaks."""
import math

import numpy as np

from oracle import elementwise as ew


def test_embed_gathers_rows_and_zeroes_bad_ids():
    table = np.arange(12, dtype=np.float64).reshape(4, 3)
    out = ew.embed([2, 0, -1, 4, 3], table)
    assert np.array_equal(out, [[6, 7, 8], [0, 1, 2], [0, 0, 0], [0, 0, 0], [9, 10, 11]])


def test_rmsnorm_closed_forms():
    # a constant row c normalises to sign(c) * w (eps = 0)
    w = np.array([1.0, 2.0, -3.0, 0.5])
    assert np.allclose(ew.rmsnorm(np.full((1, 4), -7.5), w, 0.0), -w, rtol=0, atol=1e-15)
    # scale invariance for eps = 0, mean of squares 1 after normalisation
    g = np.random.default_rng(1)
    h = g.standard_normal((3, 64))
    y = ew.rmsnorm(h, np.ones(64), 0.0)
    assert np.allclose(ew.rmsnorm(37.0 * h, np.ones(64), 0.0), y, rtol=1e-14)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    # [3, 4] with eps 0: rms = sqrt(12.5)
    assert np.allclose(ew.rmsnorm([[3.0, 4.0]], [1.0, 1.0], 0.0),
                       [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    # eps enters under the root: a zero row stays zero, tiny rows are damped
    assert np.array_equal(ew.rmsnorm(np.zeros((1, 4)), w, 1e-6), np.zeros((1, 4)))
    assert abs(ew.rmsnorm([[1e-3, 1e-3]], [1.0, 1.0], 1e-6)[0, 0] - 1e-3 / math.sqrt(2e-6)) < 1e-15


def test_rope_pins():
    g = np.random.default_rng(2)
    D, theta = 64, 1e6
    x = g.standard_normal(D)
    # position 0 is the identity
    assert np.allclose(ew.rope(x, 0, theta), x, rtol=0, atol=0)
    # a rotation: each (i, i + D/2) pair keeps its length
    y = ew.rope(x, 1234, theta)
    assert np.allclose(x[:32] ** 2 + x[32:] ** 2, y[:32] ** 2 + y[32:] ** 2, rtol=1e-13)
    # rotations compose: rope(rope(x, a), b) = rope(x, a + b)
    assert np.allclose(ew.rope(ew.rope(x, 300, theta), 77, theta), ew.rope(x, 377, theta),
                       rtol=1e-12, atol=1e-12)
    # relative position: <rope(q, m), rope(k, n)> depends on m - n only
    q, k = g.standard_normal(D), g.standard_normal(D)
    d1 = ew.rope(q, 1000, theta) @ ew.rope(k, 990, theta)
    d2 = ew.rope(q, 20, theta) @ ew.rope(k, 10, theta)
    assert abs(d1 - d2) < 1e-10
    # pair 0 turns by exactly pos radians: x = e_0 -> (cos p, ..., sin p at D/2)
    e0 = np.zeros(D)
    e0[0] = 1.0
    y = ew.rope(e0, 5, theta)
    assert abs(y[0] - math.cos(5)) < 1e-15 and abs(y[D // 2] - math.sin(5)) < 1e-15
    assert np.count_nonzero(y) == 2


def test_rope_qkv_splits_heads_in_order():
    g = np.random.default_rng(3)
    Hq, Hkv, D = 4, 2, 8
    qkv = g.standard_normal((2, (Hq + 2 * Hkv) * D))
    q, k, v = ew.rope_qkv(qkv, [0, 0], Hq, Hkv, D, 1e4)
    # position 0: pure split, head h of q is columns h*D .. h*D + D - 1
    assert np.array_equal(q[1, 3], qkv[1, 3 * D: 4 * D])
    assert np.array_equal(k[0, 1], qkv[0, (Hq + 1) * D: (Hq + 2) * D])
    assert np.array_equal(v[1, 0], qkv[1, (Hq + Hkv) * D: (Hq + Hkv + 1) * D])
    q2, k2, v2 = ew.rope_qkv(qkv, [3, 9], Hq, Hkv, D, 1e4)
    assert np.array_equal(v2, v)  # values are never rotated
    assert np.allclose(q2[1, 2], ew.rope(qkv[1, 2 * D: 3 * D], 9, 1e4))


def test_silu_mul_closed_forms():
    gu = np.array([[0.0, 1.0, -1.0, 40.0, 2.0, 3.0, 5.0, 0.5]])
    y = ew.silu_mul(gu, 4)
    s1 = 1.0 / (1.0 + math.exp(-1.0))  # 0.7310585786...
    assert y[0, 0] == 0.0
    assert abs(y[0, 1] - s1 * 3.0) < 1e-15
    assert abs(y[0, 2] - (-1.0 + s1) * 5.0) < 1e-15  # silu(-1) = -1 * sigmoid(-1) = -(1 - s1)
    assert abs(y[0, 3] - 40.0 * 0.5) < 1e-15  # silu(40) = 40 to double precision


def test_round_bf16_and_f16_of_the_model():
    from oracle import model
    import torch
    # ties go to even, 8 significant bits
    assert model.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert model.round_bf16(1.0 + 3 * 2.0 ** -9) == 1.0 + 2.0 ** -7
    assert model.round_bf16(-(1.0 + 2.0 ** -7 + 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert model.round_bf16(0.0) == 0.0
    # against torch's fp32 -> bf16 conversion (round to nearest even) on
    # fp32-representable inputs
    g = np.random.default_rng(5)
    x = (g.standard_normal(10000) * np.exp(g.uniform(-20, 20, 10000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(model.round_bf16(x.astype(np.float64)), ref)
    assert model.round_f16(1.0 + 2.0 ** -11) == 1.0
    assert model.round_f16(1.0 + 3 * 2.0 ** -12) == 1.0 + 2.0 ** -10


def test_rope_frequencies_closed_form():
    """Pair i turns by pos * theta^(-2i/D): D = 4, theta = 100, pos = 3
    gives angles 3 and 3 / 10 for pairs (0, 2) and (1, 3)."""
    y = ew.rope([1.0, 1.0, 0.0, 0.0], 3, 100.0)
    ref = [math.cos(3.0), math.cos(0.3), math.sin(3.0), math.sin(0.3)]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ew.rope_angles(3, 4, 100.0), [3.0, 0.3], rtol=1e-15)
