"""A whole verify pass captured in a HIP graph and replayed: every replay,
with eager work and synchronisations in between, must reproduce the eager
pass bit for bit (the kernels use no memset nodes and keep no state)."""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, isd, same_bits, torch_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_pass():
    m = isd()
    torch = torch_dev()
    g = synth.rng(50)
    V, K, n, Hq, Hkv, D, L = 4096, 512, 5, 16, 2, 128, 700
    codes, sm = synth.quant_weights(V, K, g)
    w = m.qgemm_w4_pack(dev(codes), dev(sm))
    x = dev(synth.activations(n, K, "bf16", g))
    max_pages = (L + n + 15) // 16 + 1
    table, num_pages = synth.page_table(1, max_pages, g)
    kp, vp = synth.kv_pages(num_pages, Hkv, D, g)
    kd, vd = dev(kp), dev(vp)
    td = dev(table)
    q = dev(synth.f16_normal((n, Hq, D), g))
    kn = dev(synth.f16_normal((n, Hkv, D), g))
    vn = dev(synth.f16_normal((n, Hkv, D), g))
    rs = dev(np.array([0, n], np.int32))
    seq0 = dev(np.array([L - 1], np.int32))
    seq_len, pos_id = seq0.clone(), seq0.clone()
    drafts = dev(g.integers(0, V, size=n - 1).astype(np.int32))
    zd = dev((g.standard_normal((n - 1, V)) * 3).astype(np.float32))
    sid = dev(np.array([1], np.int32))
    y = torch.empty((n, V), dtype=torch.float32, device="cuda")
    att = torch.empty((n, Hq, D), dtype=torch.float32, device="cuda")
    ws_a = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    ws_v = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    acc = torch.empty(1, dtype=torch.int32, device="cuda")
    toks = torch.empty((1, 9), dtype=torch.int32, device="cuda")
    acc2 = torch.empty(1, dtype=torch.int32, device="cuda")
    toks2 = torch.empty((1, 9), dtype=torch.int32, device="cuda")

    def step():
        seq_len.copy_(seq0)
        pos_id.copy_(seq0)
        m.kv_commit(kd, vd, td, seq_len, pos_id, row_start=rs, k_new=kn, v_new=vn)
        m.decode_attn(q, kd, vd, td, pos_id, rs, 0.0884, out=att, ws=ws_a)
        m.qgemm_w4(w, x, y=y)
        m.spec_verify(y, drafts, rs, accept_len=acc, out_tokens=toks, ws=ws_v)
        m.spec_verify(y, drafts, rs, draft_logits=zd, seq_id=sid, pos0=pos_id, temperature=0.8,
                      seed=3, accept_len=acc2, out_tokens=toks2, ws=ws_v)
        m.kv_commit(kd, vd, td, seq_len, pos_id, accept_len=acc)

    def snapshot():
        torch.cuda.synchronize()
        return [host(t).copy() for t in (att, y, acc, toks, acc2, toks2, seq_len, pos_id, kd, vd)]

    step()
    ref = snapshot()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for r in range(3):
        # eager work between replays that touches the same buffers
        att.fill_(float("nan"))
        y.zero_()
        toks.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, ref):
            assert same_bits(a, b), f"replay {r}"
