"""qgemm_w4 on the GPU: parity with the oracle, width invariance (memcmp of
every width-n row against the width-one call), determinism, ABI errors."""
import numpy as np
import pytest

import synth
from oracle import qgemm as oq
from gpu_util import assert_close, dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def _weights(N, K, seed):
    g = synth.rng(seed)
    codes, sm = synth.quant_weights(N, K, g)
    return g, codes, sm


def _run(m, w, x_d, n):
    return host(m.qgemm_w4(w, x_d[:n].contiguous()))


def _pack(m, codes, sm):
    return m.qgemm_w4_pack(dev(codes), dev(sm))


@pytest.mark.parametrize("N,K", [(512, 256), (1024, 256)])
def test_small_slice_fp32_parity_all_widths(N, K):
    """Tiny slice: W 512x256 and the 1024x256 lm_head, fp32 x, n = 1..8."""
    m = isd()
    g, codes, sm = _weights(N, K, 0)
    x = synth.activations(8, K, "f32", g)
    ref = oq.qgemm_w4(codes, sm, x, "f32")
    w, xd = _pack(m, codes, sm), dev(x)
    for n in range(1, 9):
        assert_close(_run(m, w, xd, n), ref[:n], what=f"n={n}")


@pytest.mark.parametrize("N,K,dt", [(1000, 416, "bf16"), (1000, 416, "f32"), (37, 96, "bf16"),
                                    (2049, 1184, "bf16"), (2049, 1184, "f32"), (16400, 160, "bf16"),
                                    (16400, 160, "f32"), (70001, 416, "bf16"),
                                    (70001, 416, "f32")])
def test_ragged_shapes_parity(N, K, dt):
    """Row counts that are not multiples of any tile, K with a partial
    4-block step (K/32 = 13, 3, 37, 5), every row class (small, mid, tall,
    very tall) with both activation types."""
    m = isd()
    g, codes, sm = _weights(N, K, N + K)
    x = synth.activations(8, K, dt, g)
    ref = oq.qgemm_w4(codes, sm, x, dt)
    w, xd = _pack(m, codes, sm), dev(x)
    for n in (1, 3, 8):
        assert_close(_run(m, w, xd, n), ref[:n], what=f"n={n}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", [(300, 256), (5120, 5120), (130, 17408 // 4)])
def test_integer_exact_bitwise(dt, N, K):
    """d = 1, m = -8, integer x: every partial sum is an integer below 2^24,
    so the GPU result must equal the oracle exactly."""
    m = isd()
    g = synth.rng(N)
    q = g.integers(0, 16, size=(N, K))
    codes, sm = synth.quant_weights_from(q, np.ones((N, K // 32), np.float16),
                                         np.full((N, K // 32), -8.0, np.float16))
    xi = g.integers(-4, 5, size=(8, K)).astype(np.float32)
    x = xi if dt == "f32" else synth.f32_to_bf16_bits(xi)
    ref = oq.qgemm_w4(codes, sm, x, dt)
    w, xd = _pack(m, codes, sm), dev(x)
    for n in (1, 5, 8):
        got = _run(m, w, xd, n)
        assert np.array_equal(got.astype(np.float64), ref[:n])


DENSE = [(5120, 5120), (34816, 5120), (5120, 17408)]


@pytest.mark.parametrize("N,K", DENSE)
def test_dense_projection_invariance_and_sampled_parity(N, K):
    """Dense projection shapes, bf16 x, widths {1,2,3,4,5,8}: every width-n
    row is bit-identical to the width-one call on that row alone; sampled
    output rows match the oracle."""
    m = isd()
    torch = torch_dev()
    g, codes, sm = _weights(N, K, 1)
    x = synth.activations(8, K, "bf16", g)
    w, xd = _pack(m, codes, sm), dev(x)
    one = [_run(m, w, xd[c:c + 1], 1)[0] for c in range(8)]
    for n in (1, 2, 3, 4, 5, 8):
        y = _run(m, w, xd, n)
        for c in range(n):
            assert same_bits(y[c], one[c]), f"width {n} row {c} differs from width 1"
    rows = np.sort(g.choice(N, size=1024, replace=False))
    ref = oq.qgemm_w4(codes, sm, x, "bf16", rows=rows)
    y8 = _run(m, w, xd, 8)
    assert_close(y8[:, rows], ref, what=f"{N}x{K}")
    torch.cuda.synchronize()


def test_padding_slots_hold_garbage_rows():
    """The activation rows after row n in memory hold NaN/huge garbage: the
    width-n result must not change."""
    m = isd()
    torch = torch_dev()
    g, codes, sm = _weights(640, 512, 5)
    x = synth.activations(8, 512, "bf16", g)
    w = _pack(m, codes, sm)
    base = _run(m, w, dev(x), 3)
    junk = x.copy()
    junk[3:] = 0x7FC0  # NaN bits
    buf = dev(junk)
    y = host(m.qgemm_w4(w, buf[:3]))
    assert same_bits(y, base)
    torch.cuda.synchronize()


def test_run_twice_identical():
    m = isd()
    g, codes, sm = _weights(34816, 5120, 2)
    x = synth.activations(8, 5120, "bf16", g)
    w, xd = _pack(m, codes, sm), dev(x)
    a = _run(m, w, xd, 8)
    b = _run(m, w, xd, 8)
    assert same_bits(a, b)


def test_abi_rejects_bad_arguments_without_writing():
    m = isd()
    torch = torch_dev()
    L = m.lib()
    g, codes, sm = _weights(64, 64, 3)
    x = dev(synth.activations(8, 64, "bf16", g))
    w = _pack(m, codes, sm)
    cd, sd = w.codes, w.scales
    y = torch.full((8, 64), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.qgemm_w4(cd.data_ptr(), sd.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 64, 48, 1, s) == -1
    assert L.qgemm_w4(cd.data_ptr(), sd.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 64, 64, 513, s) == -1
    assert L.qgemm_w4(cd.data_ptr(), sd.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 64, 64, 0, s) == -1
    assert L.qgemm_w4(cd.data_ptr(), sd.data_ptr(), x.data_ptr(), 5, y.data_ptr(), 64, 64, 1, s) == -1
    assert L.qgemm_w4(cd.data_ptr() + 1, sd.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 64, 64, 1, s) == -1
    assert L.qgemm_w4(None, sd.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 64, 64, 1, s) == -1
    torch.cuda.synchronize()
    assert (host(y) == 7.0).all()


@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (300, 416), (64, 512), (1000, 160)])
def test_pack_layout_bit_exact(N, K):
    """The packed layout, decoded by the oracle's own reader, gives back the
    row-major codes and scales exactly, with zero padding."""
    from oracle import formats
    m = isd()
    g, codes, sm = _weights(N, K, 7 + N)
    w = _pack(m, codes, sm)
    c2, s2 = formats.unpack_packed(host(w.codes), host(w.scales), N, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sm)


# ------------------------------------------------------ prefill widths

@pytest.mark.parametrize("N,K,dt", [(5120, 5120, "bf16"), (1000, 416, "bf16"), (300, 256, "f32"),
                                    (20000, 512, "bf16"), (70001, 256, "bf16"), (5120, 1024, "f32"),
                                    (20000, 512, "f32"), (70001, 256, "f32")])
def test_prefill_widths_equal_single_rows(N, K, dt):
    """Blocks of 16, 17, 64, 100 and 512 rows (slot groups of 16, ragged last
    group) in every row class (small, mid, tall and very tall): every row is
    bit-identical to that row evaluated alone, and sampled rows agree with
    the oracle."""
    m = isd()
    g, codes, sm = _weights(N, K, 80 + N)
    w = _pack(m, codes, sm)
    x = synth.activations(512, K, dt, g)
    xd = dev(x)
    probe_rows = [0, 1, 15, 16, 17, 63, 99, 255, 511]
    single = {r: host(m.qgemm_w4(w, xd[r:r + 1].contiguous())) for r in probe_rows}
    for n in (16, 17, 64, 100, 512):
        y = host(m.qgemm_w4(w, xd[:n].contiguous()))
        for r in probe_rows:
            if r < n:
                assert same_bits(y[r:r + 1], single[r]), f"n={n} row {r}"
    y = host(m.qgemm_w4(w, xd))
    sample = probe_rows[:4] + [300, 511]
    ref = oq.qgemm_w4(codes, sm, x[sample], dt)
    assert_close(y[sample], ref)
