"""Pins for the oracle's decode attention (CPU only): a pure-Python brute
force, the chunked log-sum-exp formulation, the softmax-sums-to-one
invariant and closed-form special cases."""
import math

import numpy as np
import pytest

import synth
from oracle import attention


def _setup(B, n, L, Hq, Hkv, D, seed, shuffle=True):
    g = synth.rng(seed)
    max_pages = (L + n - 1 + 15) // 16 + 1
    table, num_pages = synth.page_table(B, max_pages, g, shuffle=shuffle)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    q = synth.f16_normal((B * n, Hq, D), g)
    row_start = np.arange(B + 1, dtype=np.int32) * n
    q_pos = np.full(B, L - 1, dtype=np.int32)
    return q, kp, vp, table, q_pos, row_start


def test_brute_force_python_loops():
    q, kp, vp, table, q_pos, rs = _setup(1, 3, 37, 4, 2, 8, seed=1)
    scale = 0.35
    got = attention.decode_attn(q, kp, vp, table, q_pos, rs, scale)
    for i in range(3):
        vis = int(q_pos[0]) + i + 1
        for h in range(4):
            gk = h // 2
            sc = []
            for p in range(vis):
                page = int(table[0][p // 16])
                s = 0.0
                for d in range(8):
                    s += float(q[i, h, d]) * float(kp[page, gk, p % 16, d])
                sc.append(scale * s)
            mx = max(sc)
            w = [math.exp(v - mx) for v in sc]
            tot = sum(w)
            for d in range(8):
                acc = 0.0
                for p in range(vis):
                    page = int(table[0][p // 16])
                    acc += w[p] / tot * float(vp[page, gk, d, p % 16])
                assert abs(acc - got[i, h, d]) < 1e-12


@pytest.mark.parametrize("L", [1, 255, 256, 257, 400, 511, 512, 513, 1600])
def test_chunked_matches_plain(L):
    n = 3 if L < 1000 else 2
    q, kp, vp, table, q_pos, rs = _setup(1, n, L, 4, 2, 16, seed=L)
    a = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.25)
    b = attention.decode_attn_chunked(q, kp, vp, table, q_pos, rs, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_softmax_sums_to_one():
    g = synth.rng(4)
    for L in (1, 17, 256, 1000):
        K = g.standard_normal((L, 32)) * 3
        qv = g.standard_normal(32)
        w = attention.softmax_weights(qv, K)
        assert abs(w.sum() - 1.0) < 1e-12
        assert (w >= 0).all()


def test_constant_values_give_constant_output():
    q, kp, vp, table, q_pos, rs = _setup(2, 4, 300, 8, 2, 16, seed=5)
    vp = np.ones_like(vp)
    out = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.1)
    assert np.allclose(out, 1.0, atol=1e-14, rtol=0)


def test_single_position_returns_its_value():
    q, kp, vp, table, q_pos, rs = _setup(1, 1, 1, 4, 4, 16, seed=6)
    out = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.5)
    page = int(table[0][0])
    for h in range(4):
        assert np.array_equal(out[0, h], vp[page, h, :, 0].astype(np.float64))


def test_constant_keys_average_values():
    q, kp, vp, table, q_pos, rs = _setup(1, 2, 70, 2, 1, 8, seed=7)
    kp[:] = np.float16(0.5)
    out = attention.decode_attn(q, kp, vp, table, q_pos, rs, 1.0)
    for i in range(2):
        vis = int(q_pos[0]) + i + 1
        vals = np.array([vp[int(table[0][p // 16]), 0, :, p % 16] for p in range(vis)],
                        dtype=np.float64)
        np.testing.assert_allclose(out[i, 0], vals.mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(out[i, 1], vals.mean(axis=0), rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    q, kp, vp, table, q_pos, rs = _setup(1, 1, 50, 1, 1, 8, seed=8)
    q[:] = np.float16(0)
    q[0, 0, 0] = np.float16(1)
    kp[:] = np.float16(0)
    target = 23
    kp[int(table[0][target // 16]), 0, target % 16, 0] = np.float16(60000)
    out = attention.decode_attn(q, kp, vp, table, q_pos, rs, 1.0)
    ref = vp[int(table[0][target // 16]), 0, :, target % 16].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-12)


def test_page_table_indirection():
    """The same logical cache behind a shuffled and an identity table gives
    the same result."""
    q, kp, vp, table, q_pos, rs = _setup(1, 2, 90, 2, 1, 8, seed=9, shuffle=True)
    ident = np.arange(table.shape[1], dtype=np.int32)[None, :]
    kp2 = kp[table[0]]
    vp2 = vp[table[0]]
    a = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.3)
    b = attention.decode_attn(q, kp2, vp2, ident, q_pos, rs, 0.3)
    assert np.array_equal(a, b)


def test_grouped_heads_are_contiguous():
    q, kp, vp, table, q_pos, rs = _setup(1, 1, 20, 8, 2, 4, seed=10)
    vp[:, 0] = np.float16(1.0)
    vp[:, 1] = np.float16(-2.0)
    out = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.3)
    assert np.allclose(out[0, :4], 1.0) and np.allclose(out[0, 4:], -2.0)


def test_rows_see_growing_prefixes():
    """Row i of a width-n block equals a width-one evaluation at q_pos + i."""
    q, kp, vp, table, q_pos, rs = _setup(1, 5, 40, 2, 1, 8, seed=12)
    wide = attention.decode_attn(q, kp, vp, table, q_pos, rs, 0.3)
    for i in range(5):
        one = attention.decode_attn(q[i:i + 1], kp, vp, table, q_pos + i,
                                    np.array([0, 1]), 0.3)
        assert np.array_equal(one[0], wide[i])


def test_brute_force_ragged_batch_distinct_tables():
    """Two sequences of different lengths and widths, each behind its own
    shuffled page table, against pure-Python loops: every row reads its own
    sequence's pages and sees q_pos + i + 1 positions."""
    g = synth.rng(21)
    B, Hq, Hkv, D = 2, 4, 2, 8
    q_pos = np.array([20, 35], dtype=np.int32)
    rs = np.array([0, 2, 5], dtype=np.int32)
    max_pages = 4
    table, num_pages = synth.page_table(B, max_pages, g, shuffle=True)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    q = synth.f16_normal((5, Hq, D), g)
    scale = 0.3
    got = attention.decode_attn(q, kp, vp, table, q_pos, rs, scale)
    for s in range(B):
        for i in range(int(rs[s + 1] - rs[s])):
            r = int(rs[s]) + i
            vis = int(q_pos[s]) + i + 1
            for h in range(Hq):
                gk = h // (Hq // Hkv)
                sc = []
                for p in range(vis):
                    page = int(table[s][p // 16])
                    sc.append(scale * sum(float(q[r, h, d]) * float(kp[page, gk, p % 16, d])
                                          for d in range(D)))
                mx = max(sc)
                w = [math.exp(v - mx) for v in sc]
                tot = sum(w)
                for d in range(D):
                    acc = sum(w[p] / tot * float(vp[int(table[s][p // 16]), gk, d, p % 16])
                              for p in range(vis))
                    assert abs(acc - got[r, h, d]) < 1e-12


# -------------------------------------------- absent pages, table bounds

PAGE = 16


def _cache(num_pages, Hkv, D, g):
    kp = synth.f16_normal((num_pages, Hkv, PAGE, D), g)
    vp = synth.f16_normal((num_pages, Hkv, D, PAGE), g)
    return kp, vp


def test_absent_pages_equal_a_compacted_cache():
    """Pages with ids outside [0, num_pages) hold nothing: one row over a
    table with absent pages equals the plain definition over a cache holding
    only the present positions, in order, with no gaps."""
    g = synth.rng(61)
    Hq, Hkv, D, P = 4, 2, 16, 12
    kp, vp = _cache(P, Hkv, D, g)
    table = np.array([[3, -1, 7, P, 0, 5, P + 40, 2, 9, -7]], dtype=np.int32)
    q = synth.f16_normal((1, Hq, D), g)
    q_pos = 16 * 9 + 4  # the row sees 153 positions, 5 of them on page index 9
    got = attention.decode_attn(q, kp, vp, table, [q_pos], [0, 1], 0.3)
    present = [pi for pi in range(10) if 0 <= table[0, pi] < P]
    # compacted: the present pages' positions, in order, as a gap-free table
    n_full = sum(1 for pi in present if pi < 9)
    ids = [int(table[0, pi]) for pi in present]
    comp = np.array([ids], dtype=np.int32)
    ref = attention.decode_attn(q, kp, vp, comp, [16 * n_full + 4], [0, 1], 0.3)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_positions_past_the_table_are_absent():
    """A row whose prefix runs past the table sees the whole table."""
    g = synth.rng(62)
    kp, vp = _cache(6, 1, 16, g)
    table = np.array([[4, 1, 5]], dtype=np.int32)
    q = synth.f16_normal((3, 2, 16), g)
    past = attention.decode_attn(q, kp, vp, table, [60], [0, 3], 0.5)
    for i in range(3):
        last = attention.decode_attn(q[i:i + 1], kp, vp, table, [47], [0, 1], 0.5)
        assert np.array_equal(past[i], last[0])


def test_rows_before_position_zero_see_nothing():
    """q_pos = -3, five rows: rows 0..2 see no position (zeros), rows 3 and
    4 are rows 0 and 1 of a block at q_pos = 0."""
    g = synth.rng(63)
    kp, vp = _cache(4, 2, 16, g)
    table = np.array([[2, 0, 3]], dtype=np.int32)
    q = synth.f16_normal((5, 4, 16), g)
    neg = attention.decode_attn(q, kp, vp, table, [-3], [0, 5], 0.25)
    zero = attention.decode_attn(q[3:], kp, vp, table, [0], [0, 2], 0.25)
    assert not neg[:3].any()
    assert np.array_equal(neg[3:], zero)


def test_all_visible_pages_absent_gives_zeros():
    g = synth.rng(64)
    kp, vp = _cache(3, 1, 16, g)
    table = np.array([[-1, 3, 1]], dtype=np.int32)
    q = synth.f16_normal((2, 1, 16), g)
    out = attention.decode_attn(q, kp, vp, table, [20], [0, 2], 1.0)
    assert not out.any()
    wide = attention.decode_attn(q, kp, vp, table, [31], [0, 2], 1.0)
    assert wide[1].any()  # row 1 of that block reaches page index 2 (present)
