"""The end-to-end property on a synthetic multi-layer target: speculative
greedy decoding emits exactly the tokens of serial greedy decoding and
leaves exactly the same key/value cache, at a small shape and at the dense
shapes (5120 hidden, GQA 64/8 x 128, 34816 gate+up, 17408 down, vocabulary
152064).  The small model's logits are also checked against the oracle's
forward pass of the same weights."""
import numpy as np
import pytest

import synth
from gpu_util import host, isd, torch_dev

pytestmark = pytest.mark.gpu

TINY = dict(L=2, H=256, Hq=4, Hkv=2, D=64, F=512, V=1024)
DENSE = dict(L=2, H=5120, Hq=64, Hkv=8, D=128, F=17408, V=152064)


def _target(shape, seed, max_pages):
    torch = torch_dev()
    from invariant_speculative_decoding_amd.synthetic_target import SyntheticTarget, TargetConfig
    cfg = TargetConfig(**shape)
    w = synth.torch_target_weights(cfg.L, cfg.H, cfg.Hq, cfg.Hkv, cfg.D, cfg.F, cfg.V, seed)
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(2 * max_pages, generator=g)[:max_pages].to(torch.int32)
    t = SyntheticTarget(cfg, w, max_pages, page_table=table.view(1, -1).cuda(),
                        num_pages=2 * max_pages)
    return cfg, w, t


def _host_weights(w):
    torch = torch_dev()

    def q(pair):
        c, sm = pair
        return host(c), host(sm).view(np.uint16)

    return {
        "layers": [{"qkv": q(l["qkv"]), "o": q(l["o"]), "gu": q(l["gu"]), "down": q(l["down"]),
                    "attn_norm": host(l["attn_norm"]), "mlp_norm": host(l["mlp_norm"])}
                   for l in w["layers"]],
        "embed": host(w["embed"].view(torch.int16)).view(np.uint16),
        "final_norm": host(w["final_norm"]),
        "lm_head": q(w["lm_head"]),
    }


def _cache(t, length):
    """Keys and values of positions 0..length-1, [L][pos][Hkv][D] (fp16 bits)."""
    torch = torch_dev()
    table = host(t.table)[0]
    pos = np.arange(length)
    pg, off = table[pos // 16], pos % 16
    ks = [host(kp.view(torch.int16))[pg, :, off, :] for kp in t.kp]
    vs = [host(vp.view(torch.int16))[pg, :, :, off] for vp in t.vp]
    return ks, vs


def test_tiny_model_logits_match_oracle():
    from oracle.model import OracleTarget
    torch = torch_dev()
    cfg, w, t = _target(TINY, 90, max_pages=8)
    ref = OracleTarget(cfg, _host_weights(w))
    g = synth.rng(91)
    toks = g.integers(0, cfg.V, size=13).astype(np.int32)
    for lo, hi in ((0, 8), (8, 13)):  # a block from an empty cache, then one over it
        z = host(t.forward(torch.tensor(toks[lo:hi], device="cuda")))
        zr = ref.forward(toks[lo:hi], lo)
        err = np.abs(z - zr).max() / np.abs(zr).max()
        assert err <= 2e-2, f"block {lo}:{hi}: relative max error {err:.2e}"
        t.commit(torch.tensor([hi - lo - 1], dtype=torch.int32, device="cuda"))


def _corrupting_drafter(reference, p_agree, seed, V):
    g = np.random.default_rng(seed)

    def draft(out, k):
        d = []
        for j in range(k):
            i = len(out) + j
            if i < len(reference) and g.random() < p_agree:
                d.append(reference[i])
            else:
                d.append(int(g.integers(0, V)))
        return d

    return draft


def _spec_equals_serial(shape, seed, T, k, max_pages, prompt_len):
    from invariant_speculative_decoding_amd.synthetic_target import (serial_decode,
                                                                     speculative_decode)
    g = synth.rng(seed)
    prompt = g.integers(0, shape["V"], size=prompt_len).astype(np.int32)
    _, _, ts = _target(shape, seed, max_pages)
    serial = serial_decode(ts, prompt, T)
    _, _, tp = _target(shape, seed, max_pages)
    spec, accepts = speculative_decode(tp, prompt, T, _corrupting_drafter(serial, 0.7, seed, shape["V"]), k)
    assert spec == serial, f"first difference at token {next(i for i in range(T) if spec[i] != serial[i])}"
    assert max(accepts) > 0 and min(accepts) < k  # drafts were both accepted and rejected
    n = min(int(host(ts.seq_len)[0]), int(host(tp.seq_len)[0]))
    assert n >= prompt_len - 1 + T - 1
    ks, vs = _cache(ts, n)
    kp, vp = _cache(tp, n)
    for li in range(shape["L"]):
        assert np.array_equal(ks[li], kp[li]) and np.array_equal(vs[li], vp[li]), f"layer {li}"
    return accepts


@pytest.mark.parametrize("k", [4, 7])
def test_tiny_speculative_equals_serial(k):
    _spec_equals_serial(TINY, 92 + k, T=40, k=k, max_pages=8, prompt_len=11)


def test_dense_speculative_equals_serial():
    _spec_equals_serial(DENSE, 95, T=24, k=4, max_pages=4, prompt_len=9)
