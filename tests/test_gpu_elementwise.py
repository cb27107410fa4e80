"""Row-wise layer operations on the GPU against the oracle, and their width
invariance.  Outputs rounded to a 16-bit float are compared element by
element within one unit in the last place of the oracle's value (the fp32
arithmetic on the GPU may round the other way at a half-way point); fp32
outputs that are plain sums are compared bitwise."""
import numpy as np
import pytest

import synth
from oracle import elementwise as ew
from gpu_util import dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def _bf16_host(t):
    b = host(t.contiguous().view(torch_dev().int16)).view(np.uint16)
    return synth.bf16_bits_to_f32(b)


def _f16_host(t):
    return host(t.float())


def _within_ulp(got, ref, mant_bits):
    """|got - ref| <= one ulp of ref in a format with `mant_bits` stored
    mantissa bits (normal range; tiny values get the format's smallest
    normal ulp)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14)))
    ulp = 2.0 ** (e - mant_bits)
    bad = np.abs(got - ref) > ulp
    assert not bad.any(), f"{bad.sum()} elements beyond 1 ulp, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("H", [520, 5120, 100])
def test_embed_rows_exact(H):
    """Rows of 16-byte aligned tables (H % 8 == 0: 16-byte loads) and of
    others (H = 100, and the same table one element past an aligned base:
    single-element loads) equal the table rows exactly; ids outside [0, V)
    give zero rows."""
    m = isd()
    torch = torch_dev()
    g = synth.rng(70 + H)
    V = 300
    table = synth.f32_to_bf16_bits(g.standard_normal((V, H)).astype(np.float32))
    tokens = np.array([0, 299, 5, -1, 300, 17], dtype=np.int32)
    ref = ew.embed(tokens, synth.bf16_bits_to_f32(table)).astype(np.float32)
    h = m.embed_rows(dev(tokens), dev(table).view(torch.bfloat16))
    assert np.array_equal(host(h), ref)
    flat = torch.empty(V * H + 1, dtype=torch.bfloat16, device="cuda")
    flat[1:] = dev(table).view(torch.bfloat16).reshape(-1)
    shifted = flat[1:].view(V, H)
    assert shifted.data_ptr() % 16 != 0
    h2 = m.embed_rows(dev(tokens), shifted)
    assert np.array_equal(host(h2), ref)


@pytest.mark.parametrize("H", [256, 5120, 1000])
def test_add_rmsnorm_parity_and_invariance(H):
    m = isd()
    g = synth.rng(71 + H)
    rows = 8
    h0 = (g.standard_normal((rows, H)) * 3).astype(np.float32)
    d = g.standard_normal((rows, H)).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(H)).astype(np.float32)
    eps = 1e-6
    hd = dev(h0)
    y = m.add_rmsnorm(hd, dev(w), eps, d=dev(d))
    # the residual add is one fp32 addition per element
    assert np.array_equal(host(hd), h0 + d)
    ref = ew.rmsnorm((h0 + d).astype(np.float64), w, eps)
    _within_ulp(_bf16_host(y), ref, 7)
    # without d: normalisation only, h untouched
    h1 = dev(h0)
    y1 = m.add_rmsnorm(h1, dev(w), eps)
    assert np.array_equal(host(h1), h0)
    _within_ulp(_bf16_host(y1), ew.rmsnorm(h0, w, eps), 7)
    # each row alone gives the same bits
    yb = _bf16_host(y)
    for r in range(rows):
        hr = dev(h0[r:r + 1])
        yr = m.add_rmsnorm(hr, dev(w), eps, d=dev(d[r:r + 1]))
        assert same_bits(_bf16_host(yr), yb[r:r + 1]), f"row {r}"


@pytest.mark.parametrize("D,theta", [(128, 1e6), (64, 1e4)])
def test_rope_qkv_parity_ragged_and_invariant(D, theta):
    m = isd()
    g = synth.rng(72 + D)
    Hq, Hkv = 8, 2
    ns = [3, 1, 5]
    rs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    R = int(rs[-1])
    pos = np.array([0, 8191, 32767], dtype=np.int32)
    qkv = g.standard_normal((R, (Hq + 2 * Hkv) * D)).astype(np.float32)
    q, k, v = m.rope_qkv(dev(qkv), dev(rs), dev(pos), Hq, Hkv, D, theta)
    positions = [int(pos[s]) + i for s in range(len(ns)) for i in range(ns[s])]
    qr, kr, vr = ew.rope_qkv(qkv, positions, Hq, Hkv, D, theta)
    _within_ulp(_f16_host(q), qr, 10)
    _within_ulp(_f16_host(k), kr, 10)
    assert np.array_equal(_f16_host(v), vr.astype(np.float16).astype(np.float32))
    # a row evaluated as a single-row block at its own position: same bits
    qb, kb = host(q.view(torch_dev().int16)), host(k.view(torch_dev().int16))
    for s in range(len(ns)):
        for i in range(ns[s]):
            r = int(rs[s]) + i
            q1, k1, _ = m.rope_qkv(dev(qkv[r:r + 1]), dev(np.array([0, 1], np.int32)),
                                   dev(np.array([pos[s] + i], np.int32)), Hq, Hkv, D, theta)
            assert same_bits(host(q1.view(torch_dev().int16)), qb[r:r + 1])
            assert same_bits(host(k1.view(torch_dev().int16)), kb[r:r + 1])


def test_rope_qkv_malformed_offsets():
    """row_start [0, 4, 2, 6] over 8 rows: rows 2 and 3 lie in sequences 0
    and 2 and take sequence 0 (the lowest), rows 4 and 5 sequence 2,
    sequence 1 is empty, rows 6 and 7 lie in no range and are not written.
    Each written row equals a single-row call at its position."""
    m = isd()
    torch = torch_dev()
    g = synth.rng(74)
    Hq, Hkv, D, theta = 4, 2, 64, 1e4
    rows = 8
    rs = np.array([0, 4, 2, 6], dtype=np.int32)
    pos = np.array([10, 500, 3000], dtype=np.int32)
    qkv = g.standard_normal((rows, (Hq + 2 * Hkv) * D)).astype(np.float32)
    q = torch.full((rows, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    k = torch.full((rows, Hkv, D), float("nan"), dtype=torch.float16, device="cuda")
    v = torch.full((rows, Hkv, D), float("nan"), dtype=torch.float16, device="cuda")
    m.rope_qkv(dev(qkv), dev(rs), dev(pos), Hq, Hkv, D, theta, q=q, k=k, v=v)
    qh, kh = host(q.view(torch.int16)), host(k.view(torch.int16))
    for r, p_ in ((0, 10), (1, 11), (2, 12), (3, 13), (4, 3002), (5, 3003)):
        q1, k1, _ = m.rope_qkv(dev(qkv[r:r + 1]), dev(np.array([0, 1], np.int32)),
                               dev(np.array([p_], np.int32)), Hq, Hkv, D, theta)
        assert same_bits(host(q1.view(torch.int16)), qh[r:r + 1]), r
        assert same_bits(host(k1.view(torch.int16)), kh[r:r + 1]), r
    assert torch.isnan(q[6:].float()).all() and torch.isnan(v[6:].float()).all()


def test_silu_mul_parity_and_invariance():
    m = isd()
    g = synth.rng(73)
    rows, F = 8, 17408
    gu = (g.standard_normal((rows, 2 * F)) * 4).astype(np.float32)
    y = m.silu_mul(dev(gu), F)
    _within_ulp(_bf16_host(y), ew.silu_mul(gu, F), 7)
    yb = _bf16_host(y)
    y1 = _bf16_host(m.silu_mul(dev(gu[5:6]), F))
    assert same_bits(y1, yb[5:6])


def test_rowwise_abi_rejects_bad_arguments():
    m = isd()
    L = m.lib()
    assert L.add_rmsnorm(None, None, None, None, 1, 16, 1e-6, None) == -1
    assert L.rope_qkv(None, None, None, 1, 1, 8, 2, 130, 1e4, None, None, None, None) == -1
    assert L.silu_mul(None, None, 1, 8, None) == -1
    assert L.embed_rows(None, None, None, 1, 8, 8, None) == -1
