"""decode_attn on the GPU: parity with the oracle, width invariance (row i
of a width-n block vs a width-one call at q_pos + i), NaN-poisoned dead
slots, page-table indirection, ragged batches."""
import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import kvcache as ok
from gpu_util import assert_close, dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def _cache(B, lens, n_max, Hq, Hkv, D, seed, shuffle=True, spare=1):
    """Caches sized for every sequence's length plus a block of n_max."""
    g = synth.rng(seed)
    max_pages = (max(lens) + n_max + 15) // 16 + spare
    table, num_pages = synth.page_table(B, max_pages, g, shuffle=shuffle)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    q = synth.f16_normal((B * n_max, Hq, D), g)
    return g, table, kp, vp, q


def _call(m, q, kp, vp, table, q_pos, rs, scale):
    return host(m.decode_attn(q, kp, vp, table, q_pos, rs, scale))


def _i32(a):
    return dev(np.asarray(a, dtype=np.int32))


def test_small_slice_parity_and_invariance():
    """4 heads (Hq = Hkv = 4), head_dim 64, KV length 128, n = 1..8, row i
    sees 128 + i positions."""
    m = isd()
    L, D, H = 128, 64, 4
    g, table, kp, vp, q = _cache(1, [L], 8, H, H, D, 0, shuffle=False)
    scale = float(np.float32(1 / np.sqrt(D)))
    kd, vd, td = dev(kp), dev(vp), _i32(table)
    qd = dev(q)
    one = []
    for i in range(8):
        one.append(_call(m, qd[i:i + 1], kd, vd, td, _i32([L - 1 + i]), _i32([0, 1]), scale)[0])
    for n in range(1, 9):
        out = _call(m, qd[:n], kd, vd, td, _i32([L - 1]), _i32([0, n]), scale)
        ref = oa.decode_attn(q[:n], kp, vp, table, [L - 1], [0, n], scale)
        assert_close(out, ref, what=f"n={n}")
        for i in range(n):
            assert same_bits(out[i], one[i]), f"n={n} row {i}"


@pytest.mark.parametrize("L", [400, 1600, 8192, 32768])
def test_gqa_width_invariance_and_sampled_parity(L):
    """64 query heads, 8 KV heads, head_dim 128, widths 1..8: every row of a
    width-n block is bit-identical to width one at L + i (32 cases over the
    four lengths); every head of four rows (one per tile) matches the
    oracle."""
    m = isd()
    torch = torch_dev()
    Hq, Hkv, D = 64, 8, 128
    g, table, kp, vp, q = _cache(1, [L], 8, Hq, Hkv, D, L, shuffle=False)
    scale = float(np.float32(1 / np.sqrt(D)))
    kd, vd, td, qd = dev(kp), dev(vp), _i32(table), dev(q)
    one = [_call(m, qd[i:i + 1], kd, vd, td, _i32([L - 1 + i]), _i32([0, 1]), scale)[0]
           for i in range(8)]
    for n in range(1, 9):
        out = _call(m, qd[:n], kd, vd, td, _i32([L - 1]), _i32([0, n]), scale)
        for i in range(n):
            assert same_bits(out[i], one[i]), f"L={L} n={n} row {i}"
    # parity: every head of rows 0, 3, 5 and 7 of the width-8 block, one
    # row in each of the block's four 16-slot tiles (slot = row x 8 + head
    # in the group), so every tile of a run is checked
    out = _call(m, qd, kd, vd, td, _i32([L - 1]), _i32([0, 8]), scale)
    for i in (0, 3, 5, 7):
        sub_q = q[i:i + 1]
        ref = oa.decode_attn(sub_q, kp, vp, table, [L - 1 + i], [0, 1], scale)
        assert_close(out[i], ref[0], what=f"L={L} row {i}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("L", [8192, 32768])
def test_head_dim_64_runs_of_two_and_four_tiles(L):
    """Head size 64 with GQA 64/8: L = 8192 gives 264 units (runs of two
    tiles per work-group), L = 32768 gives 1032 (runs of four, and the
    combine's 64-chunk batches).  Every row of widths 1..8 is bit-identical
    to width one at L + i, rows 0, 3, 5 and 7 of the width-8 block (one per
    tile) match the oracle, and the append form equals the separate append
    then attention."""
    m = isd()
    Hq, Hkv, D = 64, 8, 64
    g, table, kp, vp, q = _cache(1, [L], 8, Hq, Hkv, D, 64 + L, shuffle=True)
    scale = float(np.float32(1 / np.sqrt(D)))
    kd, vd, td, qd = dev(kp), dev(vp), _i32(table), dev(q)
    one = [_call(m, qd[i:i + 1], kd, vd, td, _i32([L - 1 + i]), _i32([0, 1]), scale)[0]
           for i in range(8)]
    for n in (1, 2, 5, 8):
        out = _call(m, qd[:n], kd, vd, td, _i32([L - 1]), _i32([0, n]), scale)
        for i in range(n):
            assert same_bits(out[i], one[i]), f"L={L} n={n} row {i}"
    for i in (0, 3, 5, 7):
        ref = oa.decode_attn(q[i:i + 1], kp, vp, table, [L - 1 + i], [0, 1], scale)
        assert_close(out[i], ref[0], what=f"L={L} row {i}")
    _append_vs_separate([L - 1], [8], Hq, Hkv, D, 64 + L)


@pytest.mark.parametrize("L,Hq,Hkv", [(2000, 32, 2), (32768, 64, 4)])
def test_sixteen_heads_per_group_and_blocks_over_eight_rows(L, Hq, Hkv):
    """The largest head group, Hq / Hkv = 16: a width-8 block is eight
    16-slot tiles (one work-group per tile at L = 2000, runs of four at
    L = 32768).  Widths 1..8 are bit-identical to width one, rows match the
    oracle, and a 10-row block gives its first 8 rows those same bits and
    leaves rows 8 and 9 unwritten."""
    m = isd()
    torch = torch_dev()
    D = 128
    g, table, kp, vp, q = _cache(1, [L], 10, Hq, Hkv, D, L + Hq, shuffle=True)
    scale = float(np.float32(1 / np.sqrt(D)))
    kd, vd, td, qd = dev(kp), dev(vp), _i32(table), dev(q)
    one = [_call(m, qd[i:i + 1], kd, vd, td, _i32([L - 1 + i]), _i32([0, 1]), scale)[0]
           for i in range(8)]
    for n in (1, 3, 8):
        out = _call(m, qd[:n], kd, vd, td, _i32([L - 1]), _i32([0, n]), scale)
        for i in range(n):
            assert same_bits(out[i], one[i]), f"n={n} row {i}"
    for i in (0, 7):
        ref = oa.decode_attn(q[i:i + 1], kp, vp, table, [L - 1 + i], [0, 1], scale)
        assert_close(out[i], ref[0], what=f"row {i}")
    ten = torch.full((10, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    m.decode_attn(qd[:10], kd, vd, td, _i32([L - 1]), _i32([0, 10]), scale, out=ten)
    ten = host(ten)
    assert same_bits(ten[:8], out)
    assert np.isnan(ten[8:]).all()


def test_dead_slots_poisoned_with_nan():
    """Slots past the last row's prefix hold NaN: outputs stay finite and
    bit-identical to the clean cache."""
    m = isd()
    Hq, Hkv, D = 16, 2, 128
    lens = [300, 17, 1000]
    n = 5
    B = 3
    g, table, kp, vp, q = _cache(B, lens, n, Hq, Hkv, D, 9, spare=3)
    q_pos = np.array(lens, dtype=np.int32) - 1
    rs = np.arange(B + 1, dtype=np.int32) * n
    scale = 0.0884
    clean = _call(m, dev(q), dev(kp), dev(vp), _i32(table), _i32(q_pos), _i32(rs), scale)
    kp2, vp2 = kp.copy(), vp.copy()
    live = set()
    for s in range(B):
        for p in range(int(q_pos[s]) + n):
            live.add(ok.slot_location(table, s, p))
    for pg in range(kp.shape[0]):
        for off in range(16):
            if (pg, off) not in live:
                kp2[pg, :, off, :] = np.float16(np.nan)
                vp2[pg, :, :, off] = np.float16(np.nan)
    dirty = _call(m, dev(q), dev(kp2), dev(vp2), _i32(table), _i32(q_pos), _i32(rs), scale)
    assert np.isfinite(dirty).all()
    assert same_bits(clean, dirty)
    ref = oa.decode_attn(q, kp, vp, table, q_pos, rs, scale)
    assert_close(clean, ref)


def test_shuffled_pages_equal_identity_layout():
    m = isd()
    Hq, Hkv, D = 8, 8, 64
    g, table, kp, vp, q = _cache(1, [700], 4, Hq, Hkv, D, 11, shuffle=True)
    ident = np.arange(table.shape[1], dtype=np.int32)[None, :]
    a = _call(m, dev(q[:4]), dev(kp), dev(vp), _i32(table), _i32([699]), _i32([0, 4]), 0.125)
    b = _call(m, dev(q[:4]), dev(kp[table[0]]), dev(vp[table[0]]), _i32(ident), _i32([699]),
              _i32([0, 4]), 0.125)
    assert same_bits(a, b)


def test_ragged_batch_matches_each_sequence_alone():
    """Eight sequences with different lengths and block widths in one call
    equal each sequence run alone and each row run at width one."""
    m = isd()
    Hq, Hkv, D = 64, 8, 128
    g = synth.rng(21)
    lens = [int(v) for v in g.integers(256, 4000, size=8)]
    ns = [int(v) for v in g.integers(1, 9, size=8)]
    B = 8
    max_pages = (max(lens) + 8 + 15) // 16 + 1
    table, num_pages = synth.page_table(B, max_pages, g)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    rs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = synth.f16_normal((int(rs[-1]), Hq, D), g)
    q_pos = np.array(lens, dtype=np.int32) - 1
    kd, vd, td, qd = dev(kp), dev(vp), _i32(table), dev(q)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = _call(m, qd, kd, vd, td, _i32(q_pos), _i32(rs), scale)
    for s in range(B):
        r0, r1 = int(rs[s]), int(rs[s + 1])
        alone = _call(m, qd[r0:r1], kd, vd, _i32(table[s:s + 1]), _i32(q_pos[s:s + 1]),
                      _i32([0, r1 - r0]), scale)
        assert same_bits(out[r0:r1], alone), f"seq {s}"
        i = r1 - r0 - 1
        w1 = _call(m, qd[r1 - 1:r1], kd, vd, _i32(table[s:s + 1]), _i32([q_pos[s] + i]),
                   _i32([0, 1]), scale)
        assert same_bits(out[r1 - 1], w1[0]), f"seq {s} last row"
    ref = oa.decode_attn(q[:int(rs[2])], kp, vp, table[:2], q_pos[:2], rs[:3], scale)
    assert_close(out[:int(rs[2])], ref)


def test_workspace_query_and_too_small():
    m = isd()
    torch = torch_dev()
    import ctypes
    L = m.lib()
    need = ctypes.c_size_t(0)
    assert L.decode_attn(None, None, None, None, 10, 10, None, None, None, 2, 64, 8, 128,
                         ctypes.c_float(0.1), None, ctypes.byref(need), None) == 0
    assert need.value > 0
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    have = ctypes.c_size_t(16)
    q = torch.zeros((2, 64, 128), dtype=torch.float16, device="cuda")
    rc = L.decode_attn(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), 10, 10,
                       q.data_ptr(), q.data_ptr(), q.data_ptr(), 2, 64, 8, 128, ctypes.c_float(0.1),
                       ws.data_ptr(), ctypes.byref(have), None)
    assert rc == -2 and have.value == need.value
    assert L.decode_attn(None, None, None, None, 10, 10, None, None, None, 2, 64, 7, 128,
                         ctypes.c_float(0.1), None, ctypes.byref(need), None) == -1
    assert L.decode_attn(None, None, None, None, 10, 10, None, None, None, 2, 64, 8, 96,
                         ctypes.c_float(0.1), None, ctypes.byref(need), None) == -1


# ------------------------------------------------ append + attention fused

def _append_vs_separate(lens, ns, Hq, Hkv, D, seed, max_pages=None, absent=None):
    """decode_attn_append against kv_commit APPEND then decode_attn: the
    outputs and both caches must be bit-identical."""
    m = isd()
    g = synth.rng(seed)
    B = len(lens)
    if max_pages is None:
        max_pages = (max(lens) + 8 + 15) // 16 + 1
    table, num_pages = synth.page_table(B, max_pages, g)
    if absent is not None:  # (sequence, page index) entries pointing nowhere
        for s, pi in absent:
            table[s, pi] = -1
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    rs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    R = int(rs[-1])
    q = synth.f16_normal((R, Hq, D), g)
    kn = synth.f16_normal((R, Hkv, D), g)
    vn = synth.f16_normal((R, Hkv, D), g)
    q_pos = np.array(lens, dtype=np.int32)
    scale = float(np.float32(1 / np.sqrt(D)))
    td, rd, qd, knd, vnd = _i32(table), _i32(rs), dev(q), dev(kn), dev(vn)
    k1, v1 = dev(kp), dev(vp)
    m.kv_commit(k1, v1, td, _i32(q_pos), _i32(q_pos), row_start=rd, k_new=knd, v_new=vnd)
    out1 = host(m.decode_attn(qd, k1, v1, td, _i32(q_pos), rd, scale))
    k2, v2 = dev(kp), dev(vp)
    out2 = host(m.decode_attn_append(qd, knd, vnd, k2, v2, td, _i32(q_pos), rd, scale))
    assert same_bits(out1, out2)
    assert same_bits(host(k1), host(k2)) and same_bits(host(v1), host(v2))
    assert not same_bits(host(k2), kp)  # the append did write
    return out2


@pytest.mark.parametrize("n", [1, 5, 8])
def test_append_form_equals_append_then_attention(n):
    """One sequence at L = 8192 (264 units: a work-group per tile)."""
    _append_vs_separate([8191], [n], 64, 8, 128, 40 + n)


def test_append_form_ragged_chunk_edges_table_end_absent_pages():
    """Blocks crossing a 256-position chunk edge and a page edge, a block
    running past the table (those rows are not written), an absent page
    under new positions, GQA 16/2 x 128."""
    lens = [253, 1000, 70 * 16 - 3]  # positions 1000.. sit on page index 62
    _append_vs_separate(lens, [8, 3, 6], 16, 2, 128, 44, max_pages=70, absent=[(1, 62)])


def test_append_form_many_units_and_small_heads():
    """2080 units (a work-group per unit with its tiles in order), and
    head size 64 with 4/4 heads."""
    _append_vs_separate([33000, 20500], [7, 4], 64, 8, 128, 45)
    _append_vs_separate([100, 300, 5], [2, 8, 1], 4, 4, 64, 46)


def test_absent_pages_and_positions_outside_the_table_match_oracle():
    """Four sequences: absent pages (ids -1, num_pages, far beyond) inside
    the prefix and on the block's own positions; a block whose positions
    run past the table; a block starting at position -3 (its first three
    rows see nothing); a block whose every visible page is absent.  Outputs
    match the oracle's reading of such entries (no part in the softmax,
    zeros for a row that sees nothing), the append form equals the separate
    append then attention, and width-one calls give the same bits."""
    m = isd()
    Hq, Hkv, D, max_pages = 16, 2, 128, 45
    cap = 16 * max_pages
    g = synth.rng(65)
    lens, ns = [600, cap + 5, -3, 40], [4, 3, 6, 2]
    B = len(lens)
    table, num_pages = synth.page_table(B, max_pages, g)
    for s_, pi, v in ((0, 3, -1), (0, 10, num_pages), (0, 20, 1 << 30), (0, 37, -5),
                      (3, 0, -1), (3, 1, num_pages + 1), (3, 2, -1)):
        table[s_, pi] = v
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    rs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = synth.f16_normal((int(rs[-1]), Hq, D), g)
    q_pos = np.array(lens, dtype=np.int32)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = _call(m, dev(q), dev(kp), dev(vp), _i32(table), _i32(q_pos), _i32(rs), scale)
    ref = oa.decode_attn(q, kp, vp, table, q_pos, rs, scale)
    assert_close(out, ref)
    zero = ~ref.any(axis=(1, 2))
    assert zero.sum() == 5  # rows 0..2 of the block at -3, both rows of the absent one
    assert not out[zero].any()
    for s_ in range(B):  # each row alone at width one
        for i in range(ns[s_]):
            r = int(rs[s_]) + i
            w1 = _call(m, dev(q[r:r + 1]), dev(kp), dev(vp), _i32(table[s_:s_ + 1]),
                       _i32([lens[s_] + i]), _i32([0, 1]), scale)
            assert same_bits(out[r], w1[0]), (s_, i)
    absent = [(s_, pi) for s_ in range(B) for pi in range(max_pages)
              if not 0 <= table[s_, pi] < num_pages]
    _append_vs_separate(lens, ns, Hq, Hkv, D, 65, max_pages=max_pages, absent=absent)
