"""spec_verify_noalloc (the library's own device scratch as workspace)
against spec_verify (a caller-owned workspace) through the C ABI: two calls
in a row, the second with a smaller input, in both modes, must give the
same accept lengths and tokens bit for bit.  The scratch keeps the previous
call's contents, so the second call also shows that nothing in it depends
on what the scratch held before."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, isd, torch_dev

pytestmark = pytest.mark.gpu


def _i32(a):
    return dev(np.asarray(a, dtype=np.int32))


def _case(seed, B, k, V):
    g = synth.rng(seed)
    n = k + 1
    rs = (np.arange(B + 1) * n).astype(np.int32)
    zt = (g.standard_normal((B * n, V)) * 3).astype(np.float32)
    zd = (zt.reshape(B, n, V)[:, :k].reshape(B * k, V)
          + g.standard_normal((B * k, V)) * 0.5).astype(np.float32)
    drafts = synth.gumbel_draws(zd, 0.8, g)
    seq_id = g.permutation(1000)[:B].astype(np.int32)
    pos0 = g.integers(256, 16384, size=B).astype(np.int32)
    return zt, zd, drafts, rs, seq_id, pos0


@pytest.mark.parametrize("temperature", [0.8, 0.0])
def test_noalloc_equals_workspace_call_twice(temperature):
    m = isd()
    torch = torch_dev()
    # a large call, then a smaller one over the scratch the first one left
    for seed, (B, k, V) in ((60, (8, 7, 152064)), (61, (3, 4, 32000))):
        zt, zd, drafts, rs, seq_id, pos0 = _case(seed, B, k, V)
        args = dict(draft_logits=dev(zd), seq_id=_i32(seq_id), pos0=_i32(pos0),
                    temperature=temperature, seed=11)
        zt_d, dr_d, rs_d = dev(zt), _i32(drafts), _i32(rs)
        acc_w, out_w = m.spec_verify(zt_d, dr_d, rs_d, **args)
        acc_s, out_s = m.spec_verify_noalloc(zt_d, dr_d, rs_d, **args)
        torch.cuda.synchronize()
        print(f"noalloc T={temperature} B={B} k={k} V={V}: accept {host(acc_s).tolist()}")
        assert np.array_equal(host(acc_s), host(acc_w)), (seed, temperature)
        assert np.array_equal(host(out_s), host(out_w)), (seed, temperature)


def test_noalloc_rejects_beyond_its_scratch():
    m = isd()
    torch = torch_dev()
    V = 152064
    zt = torch.zeros((4, V), dtype=torch.float32, device="cuda")
    rs = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    dr = torch.zeros(3, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="ISD_ENOSPC"):
        m.spec_verify_noalloc(zt, dr, rs, max_rows=4000)


@pytest.mark.parametrize("temperature", [0.8, 0.0])
def test_noalloc_under_graph_capture(temperature):
    """The callers it is for: the call captured in a HIP graph (it allocates
    nothing and records no memset) and replayed three times, with an eager
    call on other inputs between the replays that leaves its own contents
    in the shared scratch; every replay gives the workspace call's bits."""
    m = isd()
    torch = torch_dev()
    zt, zd, drafts, rs, seq_id, pos0 = _case(62, 4, 5, 32000)
    B = len(rs) - 1
    args = dict(draft_logits=dev(zd), seq_id=_i32(seq_id), pos0=_i32(pos0),
                temperature=temperature, seed=13)
    zt_d, dr_d, rs_d = dev(zt), _i32(drafts), _i32(rs)
    acc_w, out_w = m.spec_verify(zt_d, dr_d, rs_d, **args)
    acc_w, out_w = host(acc_w), host(out_w)
    ozt, ozd, odr, ors, osid, opos = _case(63, 6, 7, 70000)
    other = (dev(ozt), _i32(odr), _i32(ors))
    oargs = dict(draft_logits=dev(ozd), seq_id=_i32(osid), pos0=_i32(opos),
                 temperature=temperature, seed=5)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, 9), dtype=torch.int32, device="cuda")
    m.spec_verify_noalloc(zt_d, dr_d, rs_d, accept_len=acc, out_tokens=out, **args)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        m.spec_verify_noalloc(zt_d, dr_d, rs_d, accept_len=acc, out_tokens=out, **args)
    for r in range(3):
        acc.fill_(-5)
        out.fill_(-5)
        m.spec_verify_noalloc(*other, **oargs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), acc_w), (temperature, r)
        assert np.array_equal(host(out), out_w), (temperature, r)
