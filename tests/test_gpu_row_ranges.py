"""Row offsets that break their documented shape, on the GPU.

row_start must be non-decreasing from 0; a call whose offsets are not --
a negative start, a range ending past row_start[B], a decreasing pair, a
sequence that would start before its draft entries -- must still stay
inside the arrays that row_start[B] sizes.  Such a sequence has no rows:
attention and the KV append read and write nothing of it, and the verify
calls report it as not verified (accept length 0, tokens -1; the commit
forms still add accept_len + 1 to its seq_len).  Every other sequence of
the call gives the bits it gives in a well-formed call: the greedy results
are compared with the oracle on the same logits, the sampled ones, the
attention outputs and the caches with a well-formed call holding only the
valid sequences."""
import numpy as np
import pytest

import synth
from oracle import verify as ov
from gpu_util import dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu

# verify layout: B = 7 sequences, R = 9 target rows, R - B = 2 draft entries
#   0: [0, 3)   valid, drafts 0..1
#   1: [3, -2)  decreasing
#   2: [-2, 3)  negative start
#   3: [3, 0)   decreasing
#   4: [0, 12)  first 9 rows inside [0, R), but drafts would start at -4
#   5: [12, 7)  starts past R
#   6: [7, 9)   valid, draft 1
RS_V = [0, 3, -2, 3, 0, 12, 7, 9]
VALID_V = {0: (0, 3, 0), 6: (7, 9, 1)}  # s: (first row, end row, first draft entry)
# a range inside [0, R) whose drafts overrun the R - B entries:
#   B = 3, R = 5: 0: [0, 1) valid; 1: [1, 5) needs drafts 0..2 of 2; 2: [5, 5) empty
RS_V2 = [0, 1, 5, 5]
VALID_V2 = {0: (0, 1, 0)}


def _i32(a):
    return dev(np.asarray(a, dtype=np.int32))


def _well_formed(valid, z, drafts, extra=None):
    """The valid sequences alone as a well-formed batch: (target rows,
    drafts, row_start, their indexes in the original batch)."""
    rows, dr, rs, idx = [], [], [0], []
    for s, (r0, r1, d0) in sorted(valid.items()):
        rows += list(range(r0, r1))
        dr += list(drafts[d0:d0 + (r1 - r0 - 1)])
        rs.append(len(rows))
        idx.append(s)
    return z[rows], np.asarray(dr, dtype=np.int32), np.asarray(rs, dtype=np.int32), idx


def _check_verify(acc, out, valid, B, acc_r, out_r, idx):
    for s in range(B):
        if s in valid:
            i = idx.index(s)
            assert acc[s] == acc_r[i] and np.array_equal(out[s], out_r[i]), f"seq {s}"
        else:
            assert acc[s] == 0 and (out[s] == -1).all(), f"seq {s}"


@pytest.mark.parametrize("layout", ["mixed", "draft_overrun"])
def test_greedy_verify_forms(layout):
    """spec_verify (greedy), spec_verify_commit, spec_verify_margin and
    spec_verify_keys on integer-valued logits (exact ties included)."""
    m = isd()
    rs, valid = (RS_V, VALID_V) if layout == "mixed" else (RS_V2, VALID_V2)
    B, R = len(rs) - 1, rs[-1]
    g = synth.rng(91)
    V = 3000
    z = (g.integers(-40, 40, size=(R, V)) / 4.0).astype(np.float32)
    _, _, t, _ = ov.verify_greedy(z, np.zeros(max(R - B, 1), np.int32),
                                  np.arange(R + 1, dtype=np.int32))
    drafts = g.integers(0, V, size=R - B).astype(np.int32)
    for s, (r0, r1, d0) in valid.items():  # drafts agreeing with the targets for a while
        for j in range(r1 - r0 - 1):
            if j < 1 or g.random() < 0.6:
                drafts[d0 + j] = t[r0 + j]
    zw, dw, rw, idx = _well_formed(valid, z, drafts)
    acc_r, out_r, _, marg_r = ov.verify_greedy(zw, dw, rw)
    zd, dd, rd = dev(z), _i32(drafts), _i32(rs)

    acc, out = m.spec_verify(zd, dd, rd)
    _check_verify(host(acc), host(out), valid, B, acc_r, out_r, idx)

    seq0 = np.arange(100, 100 + B, dtype=np.int32)
    sl, pid = _i32(seq0), _i32(seq0)
    acc, out = m.spec_verify_commit(zd, dd, rd, sl, pid)
    acc = host(acc)
    _check_verify(acc, host(out), valid, B, acc_r, out_r, idx)
    assert np.array_equal(host(sl), seq0 + acc + 1) and np.array_equal(host(pid), seq0 + acc + 1)

    torch = torch_dev()
    margins = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    acc, out, mg, rc = m.spec_verify_margin(zd, dd, rd, 0.5, margins=margins)
    acc, mg, rc = host(acc), host(mg), host(rc)
    _check_verify(acc, host(out), valid, B, acc_r, out_r, idx)
    rows_w = [r for s in sorted(valid) for r in range(valid[s][0], valid[s][1])]
    assert np.array_equal(mg[rows_w], np.asarray(marg_r, dtype=np.float32))
    unowned = sorted(set(range(R)) - set(rows_w))
    assert np.isnan(mg[unowned]).all()  # rows of no valid sequence: not written
    for s in range(B):
        if s not in valid:
            assert rc[s] == -1

    # keys: one per row, carrying the row's greedy token
    key = (np.uint64(0x80000000) << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - t.astype(np.uint64))
    keys = np.stack([key, key - np.uint64(1 << 40)], axis=1)  # the second key never wins
    acc, out = m.spec_verify_keys(dev(keys.view(np.int64)), dd, rd)
    _check_verify(host(acc), host(out), valid, B, acc_r, out_r, idx)


def test_sampled_verify():
    """Rejection sampling (T = 0.8), spec_verify and
    spec_verify_sampled_commit: the valid sequences give the bits of a
    well-formed call holding only them; the others are not verified."""
    m = isd()
    rs, valid = RS_V, VALID_V
    B, R = len(rs) - 1, rs[-1]
    g = synth.rng(92)
    V = 5000
    zt = g.normal(0.0, 3.0, size=(R, V)).astype(np.float32)
    zq = g.normal(0.0, 3.0, size=(R - B, V)).astype(np.float32)
    drafts = g.integers(0, V, size=R - B).astype(np.int32)
    seq_id = np.arange(B, dtype=np.int32) + 40
    pos0 = np.arange(B, dtype=np.int32) * 3 + 500
    acc, out = m.spec_verify(dev(zt), _i32(drafts), _i32(rs), draft_logits=dev(zq),
                             seq_id=_i32(seq_id), pos0=_i32(pos0), temperature=0.8, seed=5)
    zw, dw, rw, idx = _well_formed(valid, zt, drafts)
    qrows = [d0 + j for s, (r0, r1, d0) in sorted(valid.items()) for j in range(r1 - r0 - 1)]
    acc_w, out_w = m.spec_verify(dev(zw), _i32(dw), _i32(rw), draft_logits=dev(zq[qrows]),
                                 seq_id=_i32(seq_id[idx]), pos0=_i32(pos0[idx]),
                                 temperature=0.8, seed=5)
    _check_verify(host(acc), host(out), valid, B, host(acc_w), host(out_w), idx)
    # the commit form: the same results, and accept_len + 1 added everywhere
    sl, pid = _i32(pos0), _i32(pos0)
    acc, out = m.spec_verify_sampled_commit(dev(zt), _i32(drafts), _i32(rs), dev(zq),
                                            _i32(seq_id), sl, pid, 0.8, 5)
    acc = host(acc)
    _check_verify(acc, host(out), valid, B, host(acc_w), host(out_w), idx)
    assert np.array_equal(host(sl), pos0 + acc + 1) and np.array_equal(host(pid), pos0 + acc + 1)


# attention layout: B = 7, R = 11 rows, rows 3..5 owned by no valid sequence
#   0: [0, 3) valid; 1: [3, -2); 2: [-2, 4); 3: [4, 14) first 8 rows end past
#   R; 4: [14, 6); 5: [6, 8) valid; 6: [8, 11) valid
RS_A = [0, 3, -2, 4, 14, 6, 8, 11]
VALID_A = [0, 5, 6]


@pytest.mark.parametrize("append", [False, True])
def test_attention(append):
    """decode_attn / decode_attn_append: rows of valid sequences equal a
    well-formed call holding only them, rows of no valid sequence are not
    written, and the append form writes only the valid sequences' positions."""
    m = isd()
    torch = torch_dev()
    Hq, Hkv, D = 16, 2, 128
    B, R = len(RS_A) - 1, RS_A[-1]
    g = synth.rng(93)
    lens = [int(v) for v in g.integers(100, 900, size=B)]
    max_pages = (max(lens) + 16 + 15) // 16 + 1
    table, num_pages = synth.page_table(B, max_pages, g)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    q = synth.f16_normal((R, Hq, D), g)
    kn = synth.f16_normal((R, Hkv, D), g)
    vn = synth.f16_normal((R, Hkv, D), g)
    q_pos = np.array(lens, dtype=np.int32)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = torch.full((R, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    k1, v1 = dev(kp), dev(vp)
    if append:
        m.decode_attn_append(dev(q), dev(kn), dev(vn), k1, v1, _i32(table), _i32(q_pos),
                             _i32(RS_A), scale, out=out)
    else:
        m.decode_attn(dev(q), k1, v1, _i32(table), _i32(q_pos), _i32(RS_A), scale, out=out)
    rows = [r for s in VALID_A for r in range(RS_A[s], RS_A[s + 1])]
    rw = np.concatenate([[0], np.cumsum([RS_A[s + 1] - RS_A[s] for s in VALID_A])])
    k2, v2 = dev(kp), dev(vp)
    if append:
        ref = m.decode_attn_append(dev(q[rows]), dev(kn[rows]), dev(vn[rows]), k2, v2,
                                   _i32(table[VALID_A]), _i32(q_pos[VALID_A]), _i32(rw), scale)
    else:
        ref = m.decode_attn(dev(q[rows]), k2, v2, _i32(table[VALID_A]), _i32(q_pos[VALID_A]),
                            _i32(rw), scale)
    o = host(out)
    assert same_bits(o[rows], host(ref))
    assert np.isnan(o[[r for r in range(R) if r not in rows]]).all()
    assert same_bits(host(k1), host(k2)) and same_bits(host(v1), host(v2))
    if append:
        assert not same_bits(host(k1), kp)  # the valid sequences did append


def test_kv_append():
    """kv_commit APPEND writes the valid sequences' rows only."""
    m = isd()
    Hkv, D = 2, 64
    B, R = len(RS_A) - 1, RS_A[-1]
    g = synth.rng(94)
    max_pages = 40
    table, num_pages = synth.page_table(B, max_pages, g)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    kn = synth.f16_normal((R, Hkv, D), g)
    vn = synth.f16_normal((R, Hkv, D), g)
    sl = g.integers(0, 600, size=B).astype(np.int32)
    k1, v1 = dev(kp), dev(vp)
    m.kv_commit(k1, v1, _i32(table), _i32(sl), _i32(sl), row_start=_i32(RS_A), k_new=dev(kn),
                v_new=dev(vn))
    rows = [r for s in VALID_A for r in range(RS_A[s], RS_A[s + 1])]
    rw = np.concatenate([[0], np.cumsum([RS_A[s + 1] - RS_A[s] for s in VALID_A])])
    k2, v2 = dev(kp), dev(vp)
    m.kv_commit(k2, v2, _i32(table[VALID_A]), _i32(sl[VALID_A]), _i32(sl[VALID_A]),
                row_start=_i32(rw), k_new=dev(kn[rows]), v_new=dev(vn[rows]))
    assert same_bits(host(k1), host(k2)) and same_bits(host(v1), host(v2))
    assert not same_bits(host(k1), kp)
