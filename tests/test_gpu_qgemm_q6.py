"""qgemm_q6 (6-bit super-block weights) on the GPU under the same checks as
the 4-bit product: parity with the oracle, width invariance (memcmp of
every width-n row against the width-one call), prefill widths, garbage in
padding rows, the packed layout read back by the oracle's own reader, and
ABI errors."""
import numpy as np
import pytest

import synth
from oracle import formats
from oracle import qgemm as oq
from gpu_util import assert_close, dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    g = synth.rng(seed)
    return g, synth.quant_weights_q6(N, K, g)


def _pack(m, w):
    ql, qh, sc, d = w
    return m.qgemm_q6_pack(dev(ql), dev(qh), dev(sc), dev(d))


def _run(m, pw, x_d, n):
    return host(m.qgemm_q6(pw, x_d[:n].contiguous()))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_small_slice_parity_all_widths(dt):
    m = isd()
    g, w = _weights(512, 256, 0)
    x = synth.activations(8, 256, dt, g)
    ref = oq.qgemm_q6(*w, x, dt)
    pw, xd = _pack(m, w), dev(x)
    for n in range(1, 9):
        assert_close(_run(m, pw, xd, n), ref[:n], what=f"n={n}")


@pytest.mark.parametrize("N,K,dt", [(1000, 512, "bf16"), (1000, 768, "f32"), (37, 256, "bf16"),
                                    (2049, 1280, "bf16"), (2049, 1280, "f32"), (16400, 256, "bf16"),
                                    (16400, 256, "f32"), (70001, 512, "bf16"),
                                    (70001, 256, "f32")])
def test_ragged_shapes_parity(N, K, dt):
    """Row counts that are not multiples of a tile, every geometry class
    (small, mid, tall and very tall row counts), both activation types."""
    m = isd()
    g, w = _weights(N, K, N + K)
    x = synth.activations(8, K, dt, g)
    ref = oq.qgemm_q6(*w, x, dt)
    pw, xd = _pack(m, w), dev(x)
    for n in (1, 3, 8):
        assert_close(_run(m, pw, xd, n), ref[:n], what=f"n={n}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", [(300, 256), (5120, 5120), (130, 17408)])
def test_integer_exact_bitwise(dt, N, K):
    """d = 1, scales in -3..3, integer x in -4..4: every partial sum is an
    integer below 2^24, so the GPU result must equal the oracle exactly."""
    m = isd()
    g = synth.rng(N + 1)
    q = g.integers(0, 64, size=(N, K))
    sc = g.integers(-3, 4, size=(N, K // 16))
    w = synth.q6_from_codes(q, sc, np.ones((N, K // 256), np.float16))
    xi = g.integers(-4, 5, size=(8, K)).astype(np.float32)
    x = xi if dt == "f32" else synth.f32_to_bf16_bits(xi)
    ref = oq.qgemm_q6(*w, x, dt)
    pw, xd = _pack(m, w), dev(x)
    for n in (1, 5, 8):
        assert np.array_equal(_run(m, pw, xd, n).astype(np.float64), ref[:n])


def test_extreme_codes_and_scales():
    """Codes 0 and 63 with sub-scale -128 and the largest d of the recipe:
    the largest weights the format holds, against the oracle."""
    m = isd()
    g = synth.rng(9)
    N, K = 96, 512
    q = g.integers(0, 64, size=(N, K))
    q[: N // 2, ::2] = 0
    q[N // 2:, 1::2] = 63
    sc = g.integers(-128, 128, size=(N, K // 16))
    sc[:, ::3] = -128
    d = np.full((N, K // 256), 1.9e-4, np.float16)
    w = synth.q6_from_codes(q, sc, d)
    x = synth.activations(8, K, "bf16", g)
    ref = oq.qgemm_q6(*w, x, "bf16")
    assert_close(_run(m, _pack(m, w), dev(x), 8), ref)


DENSE = [(5120, 5120), (34816, 5120), (5120, 17408)]


@pytest.mark.parametrize("N,K", DENSE)
def test_dense_projection_invariance_and_sampled_parity(N, K):
    """Dense projection shapes, bf16 x, widths {1,2,3,4,5,8}: every width-n
    row is bit-identical to the width-one call; sampled output rows match
    the oracle."""
    m = isd()
    g, w = _weights(N, K, 1)
    x = synth.activations(8, K, "bf16", g)
    pw, xd = _pack(m, w), dev(x)
    one = [_run(m, pw, xd[c:c + 1], 1)[0] for c in range(8)]
    for n in (1, 2, 3, 4, 5, 8):
        y = _run(m, pw, xd, n)
        for c in range(n):
            assert same_bits(y[c], one[c]), f"width {n} row {c} differs from width 1"
    rows = np.sort(g.choice(N, size=256, replace=False))
    ref = oq.qgemm_q6(*w, x, "bf16", rows=rows)
    assert_close(_run(m, pw, xd, 8)[:, rows], ref, what=f"{N}x{K}")


def test_lm_head_invariance_and_sampled_parity():
    """The 152064x5120 lm_head in the 6-bit format (weights drawn on the
    device): widths 1..8 bit-identical to width one, sampled rows against
    the oracle."""
    m = isd()
    torch = torch_dev()
    N, K = 152064, 5120
    ql, qh, sc, d = synth.torch_quant_weights_q6(N, K, 11)
    pw = m.qgemm_q6_pack(ql, qh, sc, d)
    g = synth.rng(12)
    x = synth.activations(8, K, "bf16", g)
    xd = dev(x)
    one = [_run(m, pw, xd[c:c + 1], 1)[0] for c in range(8)]
    for n in (2, 5, 8):
        y = _run(m, pw, xd, n)
        for c in range(n):
            assert same_bits(y[c], one[c]), f"width {n} row {c}"
    rows = np.sort(g.choice(N, size=192, replace=False))
    ri = torch.from_numpy(rows).cuda()
    hw = (host(ql[ri]), host(qh[ri]), host(sc[ri]), host(d[ri]).view(np.uint16))
    ref = oq.qgemm_q6(*hw, x, "bf16")
    assert_close(np.stack(one)[:, rows], ref, what="lm_head")


@pytest.mark.parametrize("N,K,dt", [(5120, 5120, "bf16"), (1000, 768, "f32"), (20000, 512, "bf16"),
                                    (20000, 512, "f32"), (70001, 256, "bf16"),
                                    (70001, 256, "f32")])
def test_prefill_widths_equal_single_rows(N, K, dt):
    """Blocks of 16, 17, 100 and 512 rows: every probed row is bit-identical
    to that row evaluated alone, and sampled rows agree with the oracle."""
    m = isd()
    g, w = _weights(N, K, 80 + N)
    pw = _pack(m, w)
    x = synth.activations(512, K, dt, g)
    xd = dev(x)
    probe_rows = [0, 1, 15, 16, 17, 99, 255, 511]
    single = {r: host(m.qgemm_q6(pw, xd[r:r + 1].contiguous())) for r in probe_rows}
    for n in (16, 17, 100, 512):
        y = host(m.qgemm_q6(pw, xd[:n].contiguous()))
        for r in probe_rows:
            if r < n:
                assert same_bits(y[r:r + 1], single[r]), f"n={n} row {r}"
    y = host(m.qgemm_q6(pw, xd))
    sample = [0, 17, 300, 511]
    assert_close(y[sample], oq.qgemm_q6(*w, x[sample], dt))


def test_padding_slots_hold_garbage_rows():
    m = isd()
    g, w = _weights(640, 512, 5)
    x = synth.activations(8, 512, "bf16", g)
    pw = _pack(m, w)
    base = _run(m, pw, dev(x), 3)
    junk = x.copy()
    junk[3:] = 0x7FC0  # NaN bits
    y = host(m.qgemm_q6(pw, dev(junk)[:3]))
    assert same_bits(y, base)


@pytest.mark.parametrize("N,K", [(1, 256), (37, 512), (300, 768)])
def test_pack_layout_bit_exact(N, K):
    """The packed buffer, decoded by the oracle's own reader, gives back the
    row-major inputs exactly, with zero padding rows."""
    m = isd()
    _, w = _weights(N, K, 7 + N)
    pw = _pack(m, w)
    back = formats.unpack_packed_q6(host(pw.packed), N, K)
    for a, b in zip(back, w):
        assert np.array_equal(a, b)


def test_abi_rejects_bad_arguments_without_writing():
    m = isd()
    torch = torch_dev()
    L = m.lib()
    g, w = _weights(64, 256, 3)
    x = dev(synth.activations(8, 256, "bf16", g))
    pw = _pack(m, w)
    p = pw.packed.data_ptr()
    y = torch.full((8, 64), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.qgemm_q6(p, x.data_ptr(), 1, y.data_ptr(), 64, 128, 1, s) == -1   # K % 256
    assert L.qgemm_q6(p, x.data_ptr(), 1, y.data_ptr(), 64, 384, 1, s) == -1
    assert L.qgemm_q6(p, x.data_ptr(), 1, y.data_ptr(), 64, 256, 0, s) == -1
    assert L.qgemm_q6(p, x.data_ptr(), 1, y.data_ptr(), 64, 256, 513, s) == -1
    assert L.qgemm_q6(p, x.data_ptr(), 5, y.data_ptr(), 64, 256, 1, s) == -1
    assert L.qgemm_q6(p + 8, x.data_ptr(), 1, y.data_ptr(), 64, 256, 1, s) == -1
    assert L.qgemm_q6(None, x.data_ptr(), 1, y.data_ptr(), 64, 256, 1, s) == -1
    assert L.qgemm_q6(p, x.data_ptr() + 2, 1, y.data_ptr(), 64, 256, 1, s) == -1
    assert L.qgemm_q6_packed_bytes(64, 320) == 0
    torch.cuda.synchronize()
    assert (host(y) == 7.0).all()
