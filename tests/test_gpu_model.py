"""The end-to-end property on a synthetic multi-layer target: speculative
greedy decoding emits exactly the tokens of serial greedy decoding and
leaves exactly the same key/value cache, at a small shape and at the dense
shapes (5120 hidden, GQA 64/8 x 128, 34816 gate+up, 17408 down, vocabulary
152064).  Every operation of the small model's layers, and of one layer
at the dense shapes, is checked against the oracle's value of that
operation on the GPU's own inputs, and the small model's logits against
the oracle's whole forward pass of the same weights."""
import numpy as np
import pytest

import synth
from gpu_util import assert_close, assert_rounded, host, isd, torch_dev

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


def _host_weights(w, embed=True):
    torch = torch_dev()

    def q(pair):
        c, sm = pair
        return host(c), host(sm).view(np.uint16)

    return {
        "layers": [{"qkv": q(l["qkv"]), "o": q(l["o"]), "gu": q(l["gu"]), "down": q(l["down"]),
                    "attn_norm": host(l["attn_norm"]), "mlp_norm": host(l["mlp_norm"])}
                   for l in w["layers"]],
        "embed": host(w["embed"].view(torch.int16)).view(np.uint16) if embed else None,
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


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _cache64(t, length):
    """The GPU's keys and values of positions 0..length-1 as fp64,
    [L][pos][Hkv][D]."""
    ks, vs = _cache(t, length)
    return ([k.view(np.float16).astype(np.float64) for k in ks],
            [v.view(np.float16).astype(np.float64) for v in vs])


OUT_OF = {"qkv": "qkv", "o": "o", "gu": "gu", "down": "delta", "lm_head": "logits"}
# outputs stored in 16 bits: correctly rounded from the exact value
ROUNDED = {"x": "bf16", "x2": "bf16", "mm": "bf16", "xf": "bf16",
           "q": "fp16", "k": "fp16", "v": "fp16"}


def _check_ops(ref, trace, t, start, rows=None, what=""):
    """Every operation of every layer against the oracle's value of that
    operation on the GPU's own inputs (teacher forcing): fp32 outputs
    within max-abs error 2e-3 x max|ref|, 16-bit outputs correctly rounded
    up to the fp32 error before rounding (assert_rounded).  Returns the
    largest error per operation name (relative to max|ref| for fp32
    outputs, in half ulps for 16-bit ones)."""
    n = trace[0]["x"].shape[0]
    Ks, Vs = _cache64(t, start + n)
    worst = {}
    for li, rec in enumerate(trace):
        g = {k: _f64(v) for k, v in rec.items() if v is not None}
        last = li == len(trace) - 1
        r = ref.step_from(None if last else li, g, start,
                          None if last else Ks[li], None if last else Vs[li], rows=rows)
        cols = {OUT_OF[p]: c for p, c in (rows or {}).items()}
        for name, val in r.items():
            got = g[name] if name not in cols else g[name][:, cols[name]]
            got = got.reshape(val.shape)
            tag = f"{what} layer {'final' if last else li} {name}"
            if name in ROUNDED:
                e = assert_rounded(got, val, ROUNDED[name], what=tag)
            else:
                e = assert_close(got, val, what=tag)
            worst[name] = max(worst.get(name, 0.0), e)
    return worst


def test_tiny_model_operations_match_oracle():
    """Each operation of the 2-layer tiny model against the oracle's value
    of that operation, fed the GPU's own rounded inputs (bf16 activations,
    fp16 q/k/v, the GPU's cache): fp32 outputs at max-abs error <= 2e-3 x
    max|ref|, bf16 and fp16 outputs correctly rounded; and the logits of
    the whole forward against the oracle's forward."""
    from oracle.model import OracleTarget
    torch = torch_dev()
    cfg, w, t = _target(TINY, 90, max_pages=8)
    hw = _host_weights(w)
    ref = OracleTarget(cfg, hw)
    g = synth.rng(91)
    toks = g.integers(0, cfg.V, size=13).astype(np.int32)
    worst, e2e = {}, []
    for lo, hi in ((0, 8), (8, 13)):  # a block from an empty cache, then one over it
        trace = []
        z = _f64(t.forward(torch.tensor(toks[lo:hi], device="cuda"), trace=trace))
        for k, v in _check_ops(ref, trace, t, lo, what=f"block {lo}:{hi}").items():
            worst[k] = max(worst.get(k, 0.0), v)
        zr = ref.forward(toks[lo:hi], lo)
        e2e.append(float(np.abs(z - zr).max() / np.abs(zr).max()))
        t.commit(torch.tensor([hi - lo - 1], dtype=torch.int32, device="cuda"))
    print("tiny model, largest relative error per operation:",
          {k: f"{v:.2e}" for k, v in sorted(worst.items())})
    print("tiny model, end-to-end logits relative error per block:", [f"{e:.2e}" for e in e2e])
    # The whole forward is not held to the per-operation bound: every bf16
    # and fp16 rounding point rounds the GPU's fp32 value, the oracle the
    # exact one, and the few elements within that difference of a half-way
    # point round to neighbouring values; the attention's fp16 weights
    # (about 1e-4 relative on its output) seed such differences in the
    # residual stream.  Measured on this model: 1.9e-3 and 2.2e-3 of
    # max|ref|.  This bound only guards the composition.
    assert max(e2e) <= 5e-3, e2e


def test_dense_layer_operations_match_oracle():
    """One layer at the dense shapes (5120 hidden, GQA 64/8 x 128, 34816
    gate+up, 17408 down, vocabulary 152064) after an 8-token prefill, a
    5-row verify block: every operation against the oracle on the GPU's own
    inputs, the projections and the lm_head on 256 sampled output rows
    each, the row-wise operations and attention in full: fp32 outputs at
    max-abs error <= 2e-3 x max|ref|, bf16 and fp16 outputs correctly
    rounded."""
    from oracle.model import OracleTarget
    torch = torch_dev()
    shape = dict(DENSE, L=1)
    cfg, w, t = _target(shape, 96, max_pages=4)
    hw = _host_weights(w, embed=False)  # the per-operation check needs no embedding
    ref = OracleTarget(cfg, hw)
    g = synth.rng(97)
    toks = g.integers(0, cfg.V, size=14).astype(np.int32)
    t.forward(torch.tensor(toks[:8], device="cuda"))
    t.commit(torch.tensor([7], dtype=torch.int32, device="cuda"))
    nq = (cfg.Hq + 2 * cfg.Hkv) * cfg.D
    rows = {"qkv": np.sort(g.choice(nq, 256, replace=False)),
            "o": np.sort(g.choice(cfg.H, 256, replace=False)),
            "gu": np.sort(g.choice(2 * cfg.F, 256, replace=False)),
            "down": np.sort(g.choice(cfg.H, 256, replace=False)),
            "lm_head": np.sort(g.choice(cfg.V, 256, replace=False))}
    trace = []
    t.forward(torch.tensor(toks[8:13], device="cuda"), trace=trace)
    worst = _check_ops(ref, trace, t, 8, rows=rows, what="dense")
    print("dense layer, largest relative error per operation:",
          {k: f"{v:.2e}" for k, v in sorted(worst.items())})


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
