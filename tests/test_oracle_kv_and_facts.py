"""Pins for the oracle's paged-KV bookkeeping, plus the pages' two
arithmetic facts (CPU only)."""
import json
import os

import numpy as np

import synth
from oracle import kvcache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _state(B, max_pages, Hkv, D, seed):
    g = synth.rng(seed)
    table, num_pages = synth.page_table(B, max_pages, g)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    return g, table, kp, vp


def test_slot_mapping_is_injective_and_covers_pages():
    g, table, _, _ = _state(5, 7, 1, 4, 0)
    seen = {}
    for s in range(5):
        for p in range(7 * 16):
            loc = kvcache.slot_location(table, s, p)
            assert loc not in seen
            seen[loc] = (s, p)
    assert len({pg for pg, _ in seen}) == 35


def test_batched_step_equals_one_token_replay():
    """Append a verify block, commit a_s accepted drafts; the committed
    prefix equals appending the accepted rows one at a time."""
    B, Hkv, D = 4, 2, 8
    g, table, kp, vp = _state(B, 6, Hkv, D, 1)
    seq_len = np.array([3, 17, 30, 0], dtype=np.int32)
    n = 5
    rs = np.arange(B + 1, dtype=np.int32) * n
    kn = synth.f16_normal((B * n, Hkv, D), g)
    vn = synth.f16_normal((B * n, Hkv, D), g)
    acc = np.array([0, 4, 2, 1], dtype=np.int32)
    k1, v1 = kvcache.append(kp, vp, table, seq_len, rs, kn, vn)
    c1, pid1 = kvcache.commit(seq_len, acc)
    assert np.array_equal(c1, seq_len + acc + 1) and np.array_equal(pid1, c1)
    k2, v2, c2 = kp.copy(), vp.copy(), seq_len.copy()
    for j in range(n):
        for s in range(B):
            if j <= acc[s]:
                one = np.array([0, 1], dtype=np.int32)
                ks, vs = kvcache.append(k2, v2, table[s:s + 1], c2[s:s + 1], one,
                                        kn[s * n + j:s * n + j + 1], vn[s * n + j:s * n + j + 1])
                k2, v2 = ks, vs
                c2[s] += 1
    assert np.array_equal(c2, c1)
    for s in range(B):
        for p in range(int(c1[s])):
            pg, off = kvcache.slot_location(table, s, p)
            assert np.array_equal(k1[pg, :, off], k2[pg, :, off])
            assert np.array_equal(v1[pg, :, :, off], v2[pg, :, :, off])


def test_rollback_is_truncation_and_next_append_overwrites():
    B, Hkv, D = 1, 1, 4
    g, table, kp, vp = _state(B, 3, Hkv, D, 2)
    seq_len = np.array([10], dtype=np.int32)
    rs = np.array([0, 5], dtype=np.int32)
    kn = synth.f16_normal((5, Hkv, D), g)
    vn = synth.f16_normal((5, Hkv, D), g)
    k1, v1 = kvcache.append(kp, vp, table, seq_len, rs, kn, vn)
    c1, _ = kvcache.commit(seq_len, np.array([1]))
    assert c1[0] == 12
    kn2 = synth.f16_normal((5, Hkv, D), g)
    k2, _ = kvcache.append(k1, v1, table, c1, rs, kn2, kn2)
    pg, off = kvcache.slot_location(table, 0, 12)
    assert np.array_equal(k2[pg, :, off], kn2[0])
    pg, off = kvcache.slot_location(table, 0, 11)
    assert np.array_equal(k2[pg, :, off], kn[1])


def test_fp_order_and_survival_facts():
    f = json.load(open(os.path.join(GOLD, "fp_order_example.json")))
    a, b = f["a"], f["b"]
    assert (a + b) - b == f["left_assoc"]
    assert a + (b - b) == f["right_assoc"]
    assert abs(100 * f["survive_rate"] ** f["steps"] - f["survive_percent_approx"]) < 0.05


def test_append_writes_each_value_at_its_slot():
    """Element by element: after APPEND, key (j, g, d) of row r sits at
    k[page][g][offset][d] and value (j, g, d) at v[page][g][d][offset] of
    its position's slot; every other cache entry is unchanged."""
    B, Hkv, D = 2, 2, 4
    g, table, kp, vp = _state(B, 3, Hkv, D, 31)
    seq_len = np.array([14, 3], dtype=np.int32)
    rs = np.array([0, 3, 5], dtype=np.int32)
    kn = synth.f16_normal((5, Hkv, D), g)
    vn = synth.f16_normal((5, Hkv, D), g)
    k2, v2 = kvcache.append(kp, vp, table, seq_len, rs, kn, vn)
    touched = set()
    for s in range(B):
        for j in range(int(rs[s + 1] - rs[s])):
            p = int(seq_len[s]) + j
            pg, off = int(table[s][p // 16]), p % 16
            touched.add((pg, off))
            for gg in range(Hkv):
                for d in range(D):
                    assert k2[pg, gg, off, d] == kn[rs[s] + j, gg, d]
                    assert v2[pg, gg, d, off] == vn[rs[s] + j, gg, d]
    for pg in range(kp.shape[0]):
        for off in range(16):
            if (pg, off) not in touched:
                assert np.array_equal(k2[pg, :, off, :], kp[pg, :, off, :])
                assert np.array_equal(v2[pg, :, :, off], vp[pg, :, :, off])


def test_append_skips_rows_it_cannot_place():
    """Hand-listed placements under the skip rules: positions before 0 or
    past the table and pages with ids outside [0, num_pages) are skipped, and
    a block writes at most 8 rows.  Table of 3 pages (48 positions):
      seq 0: seq_len -2, 5 rows  -> rows 2, 3, 4 at positions 0, 1, 2
      seq 1: seq_len 46, 4 rows  -> rows 0, 1 at positions 46, 47
      seq 2: seq_len 14, 4 rows, page index 1 absent -> rows 0, 1 at 14, 15
      seq 3: seq_len 5, 10 rows  -> rows 0..7 at positions 5..12
    Every other cache entry is unchanged."""
    B, Hkv, D = 4, 2, 4
    g, table, kp, vp = _state(B, 3, Hkv, D, 32)
    table[2, 1] = -1
    seq_len = np.array([-2, 46, 14, 5], dtype=np.int32)
    rs = np.array([0, 5, 9, 13, 23], dtype=np.int32)
    kn = synth.f16_normal((23, Hkv, D), g)
    vn = synth.f16_normal((23, Hkv, D), g)
    k2, v2 = kvcache.append(kp, vp, table, seq_len, rs, kn, vn)
    placed = ([(0, j, j - 2) for j in (2, 3, 4)] + [(1, 0, 46), (1, 1, 47)]
              + [(2, 0, 14), (2, 1, 15)] + [(3, j, 5 + j) for j in range(8)])
    touched = set()
    for s, j, p in placed:
        pg, off = int(table[s][p // 16]), p % 16
        touched.add((pg, off))
        assert np.array_equal(k2[pg, :, off, :], kn[rs[s] + j])
        assert np.array_equal(v2[pg, :, :, off], vn[rs[s] + j])
    for pg in range(kp.shape[0]):
        for off in range(16):
            if (pg, off) not in touched:
                assert np.array_equal(k2[pg, :, off, :], kp[pg, :, off, :])
                assert np.array_equal(v2[pg, :, :, off], vp[pg, :, :, off])
