"""qgemm_w4_argmax + spec_verify_keys: the lm_head with per-wave-column
argmax keys and the greedy verify from those keys.  The logits are
bit-identical to qgemm_w4's, the keys of a row give exactly the token the
logits give (lowest index among exact ties, also across column boundaries), the
accept lengths, tokens and commit equal spec_verify_commit's on the
logits, a row's keys do not depend on the width, and the keys-only form
(no logits written) writes the same keys."""
import numpy as np
import pytest

import synth
from oracle import qgemm as oq
from oracle import verify as ov
from gpu_util import dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def _i32(a):
    return dev(np.asarray(a, dtype=np.int32))


def _token(keys_row):
    """The index carried by the largest key (complemented in the low bits)."""
    b = int(np.max(keys_row.view(np.uint64)))
    return 0xFFFFFFFF - (b & 0xFFFFFFFF)


def _blocks(ks, rng, V, targets):
    """row_start and drafts for sequences of ks[s] drafts each, agreeing with
    the targets for a uniform number of leading drafts."""
    rs = np.concatenate([[0], np.cumsum(np.asarray(ks) + 1)]).astype(np.int32)
    R = int(rs[-1])
    drafts = np.zeros(R - len(ks), dtype=np.int32)
    for s, k in enumerate(ks):
        d, _ = synth.greedy_drafts(targets[rs[s]:rs[s + 1]], int(k), rng, V,
                                   agree=synth.uniform_agree(0, int(k)))
        drafts[rs[s] - s: rs[s + 1] - s - 1] = d
    return rs, drafts


@pytest.mark.parametrize("V", [300, 3000, 20000, 200000])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_integer_logits_with_ties_match_logits_verify(dt, V):
    """Integer-exact weights and activations: logits are small integers with
    many exact ties, inside and across wave columns; 300, 3000, 20000 and
    200000 rows take four work-group shapes (one row tile per wave, a K
    split over eight waves, three tiles per wave over two, and 5 tiles per
    wave two waves wide, whose 2500 keys per row take the greedy verify
    two rounds of loads), each with a ragged tail."""
    m = isd()
    torch = torch_dev()
    g = synth.rng(500)
    K = 256
    q = g.integers(0, 16, size=(V, K))
    ones = np.ones((V, K // 32), np.float16)
    codes, sm = synth.quant_weights_from(q, ones, (-8 * ones).astype(np.float16))
    B = 3
    ks = [4, 0, 7]
    R = sum(ks) + B
    xi = g.integers(-2, 3, size=(R, K)).astype(np.float32)
    x = xi if dt == "f32" else synth.f32_to_bf16_bits(xi)
    w = m.qgemm_w4_pack(dev(codes), dev(sm))
    xd = dev(x)
    y_ref = host(m.qgemm_w4(w, xd))
    y, keys = m.qgemm_w4_argmax(w, xd)
    assert same_bits(host(y), y_ref)
    kh = host(keys)
    for r in range(R):
        assert _token(kh[r]) == ov.argmax_lowest(y_ref[r].astype(np.float64)), r
    t = [ov.argmax_lowest(r.astype(np.float64)) for r in y_ref]
    rs, drafts = _blocks(ks, g, V, t)
    acc_l, out_l = m.spec_verify(dev(y_ref), _i32(drafts), _i32(rs))
    acc_k, out_k = m.spec_verify_keys(keys, _i32(drafts), _i32(rs))
    assert np.array_equal(host(acc_k), host(acc_l))
    assert np.array_equal(host(out_k), host(out_l))
    # keys only: the same keys without the logits
    y0, keys0 = m.qgemm_w4_argmax(w, xd, logits=False)
    assert y0 is None and np.array_equal(host(keys0), kh)


def test_lm_head_keys_verify_and_commit_equal_logits_path():
    """lm_head 152064 x 5120 (weights drawn on the device), bf16 hidden
    states, two sequences of k = 4 and 7 drafts: y bit-identical to
    qgemm_w4, accept lengths, tokens and the committed seq_len / pos_id equal
    to spec_verify_commit on the logits; every row's keys equal the keys of
    that row computed alone (width invariance)."""
    m = isd()
    torch = torch_dev()
    N, K = 152064, 5120
    w = m.qgemm_w4_pack(*synth.torch_quant_weights(N, K, 41))
    g = synth.rng(42)
    ks = [4, 7]
    R = sum(ks) + len(ks)
    x = dev(synth.activations(R, K, "bf16", g))
    y_ref = m.qgemm_w4(w, x)
    y, keys = m.qgemm_w4_argmax(w, x)
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    for r in (0, 5, R - 1):
        _, k1 = m.qgemm_w4_argmax(w, x[r:r + 1].contiguous(), logits=False)
        assert torch.equal(k1[0], keys[r]), r
    t = [int(v) for v in host(torch.argmax(y_ref, dim=1))]  # first maximum
    rs, drafts = _blocks(ks, g, N, t)
    sl_a = _i32([1000, 2000])
    pid_a = sl_a.clone()
    acc_l, out_l = m.spec_verify_commit(y_ref, _i32(drafts), _i32(rs), sl_a, pid_a)
    sl_b = _i32([1000, 2000])
    pid_b = sl_b.clone()
    acc_k, out_k = m.spec_verify_keys(keys, _i32(drafts), _i32(rs), sl_b, pid_b)
    assert np.array_equal(host(acc_k), host(acc_l))
    assert np.array_equal(host(out_k), host(out_l))
    assert np.array_equal(host(sl_b), host(sl_a)) and np.array_equal(host(pid_b), host(pid_a))


def test_keys_abi_rejects_bad_arguments():
    m = isd()
    torch = torch_dev()
    import ctypes
    L = m.lib()
    w = m.qgemm_w4_pack(*synth.torch_quant_weights(300, 256, 43))
    nk = m.qgemm_w4_argmax_nkeys(w)
    assert nk >= 1
    x = dev(synth.activations(2, 256, "bf16", synth.rng(44)))
    keys = torch.full((2, nk), 7, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    bad = ctypes.c_int(nk + 1)
    assert L.qgemm_w4_argmax(w.codes.data_ptr(), w.scales.data_ptr(), x.data_ptr(), 1, None,
                             300, 256, 2, keys.data_ptr(), ctypes.byref(bad), s) == -1
    good = ctypes.c_int(nk)
    assert L.qgemm_w4_argmax(w.codes.data_ptr(), w.scales.data_ptr(), x.data_ptr(), 1, None,
                             300, 256, 0, keys.data_ptr(), ctypes.byref(good), s) == -1
    assert L.qgemm_w4_argmax(None, None, None, 1, None, 300, 256, 2, None, None, s) == -1
    rs = _i32([0, 2])
    d = _i32([0])
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 9), dtype=torch.int32, device="cuda")
    sl = _i32([5])
    assert L.spec_verify_keys(keys.data_ptr(), nk, d.data_ptr(), rs.data_ptr(), 1, 2,
                              acc.data_ptr(), out.data_ptr(), sl.data_ptr(), None, s) == -1
    assert L.spec_verify_keys(keys.data_ptr(), 0, d.data_ptr(), rs.data_ptr(), 1, 2,
                              acc.data_ptr(), out.data_ptr(), None, None, s) == -1
    torch.cuda.synchronize()
    assert (host(keys) == 7).all() and int(host(sl)[0]) == 5


def test_keys_verify_over_several_load_rounds():
    """spec_verify_keys on synthetic keys with 5000 per row (three rounds of
    the kernel's per-lane key loads, the last one partial): each row's token
    is the one its largest key carries, wherever in the row that key sits
    (the first column, the last, or inside the partial round), with an exact
    tie on the value broken towards the lower index; accept lengths and
    tokens equal the greedy rule applied to those tokens."""
    m = isd()
    torch = torch_dev()
    g = synth.rng(77)
    ks = [4, 0, 7, 2, 1]
    rs = np.concatenate([[0], np.cumsum(np.asarray(ks) + 1)]).astype(np.int32)
    R, nk = int(rs[-1]), 5000
    hi = g.integers(0, 0x7FFFFFFF, size=(R, nk), dtype=np.uint64)
    idx = g.integers(0, 1 << 20, size=(R, nk), dtype=np.uint64)
    keys = (hi << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - idx)
    targets = np.zeros(R, dtype=np.int64)
    spots = [0, nk - 1, 4096, 4500, 2047, 2048]
    for r in range(R):
        col = spots[r % len(spots)] if r < len(spots) else int(g.integers(0, nk))
        t = int(g.integers(0, 1 << 20))
        top = np.uint64(0x80000000)
        keys[r, col] = (top << np.uint64(32)) | np.uint64(0xFFFFFFFF - t)
        # the same value at a higher index elsewhere in the row loses the tie
        other = (col + 1234) % nk
        keys[r, other] = (top << np.uint64(32)) | np.uint64(0xFFFFFFFF - (t + 7))
        targets[r] = t
    drafts = np.zeros(R - len(ks), dtype=np.int32)
    exp_acc, exp_out = [], []
    for s_, k in enumerate(ks):
        tg = targets[rs[s_]:rs[s_ + 1]]
        d, _ = synth.greedy_drafts(tg, int(k), g, 1 << 20, agree=synth.uniform_agree(0, int(k)))
        drafts[rs[s_] - s_: rs[s_ + 1] - s_ - 1] = d
        a, em = ov.greedy_accept(tg, d)
        exp_acc.append(a)
        exp_out.append(em + [-1] * (9 - len(em)))
    kt = dev(keys.view(np.int64))
    acc, out = m.spec_verify_keys(kt, _i32(drafts), _i32(rs))
    assert np.array_equal(host(acc), np.asarray(exp_acc, dtype=np.int32))
    assert np.array_equal(host(out), np.asarray(exp_out, dtype=np.int32))
