"""Pin of the oracle's synthetic target (CPU only): its attention, which the
forward pass evaluates with its own loop over a list cache, is checked
against the paged decode-attention oracle (itself pinned against a
pure-Python brute force) on the same rounded queries, keys and values; the
rest of the layer is the row-wise oracle operations, each pinned in
test_oracle_elementwise.py."""
import types

import numpy as np

import synth
from oracle import attention, elementwise as ew, formats
from oracle.model import OracleTarget, round_bf16, round_f16, round_f32


def _weights(H, Hq, Hkv, D, F, V, g):
    def qw(N, K):
        return synth.quant_weights(N, K, g)
    layer = {"qkv": qw((Hq + 2 * Hkv) * D, H), "o": qw(H, Hq * D), "gu": qw(2 * F, H),
             "down": qw(H, F), "attn_norm": 1.0 + 0.1 * g.standard_normal(H),
             "mlp_norm": 1.0 + 0.1 * g.standard_normal(H)}
    return {"layers": [layer],
            "embed": synth.f32_to_bf16_bits(g.standard_normal((V, H)).astype(np.float32)),
            "final_norm": 1.0 + 0.1 * g.standard_normal(H), "lm_head": qw(V, H)}


def test_model_attention_matches_paged_decode_attention():
    H, Hq, Hkv, D, F, V = 64, 4, 2, 16, 64, 40
    cfg = types.SimpleNamespace(H=H, Hq=Hq, Hkv=Hkv, D=D, F=F, V=V, eps=1e-6, theta=1e4)
    g = synth.rng(5)
    w = _weights(H, Hq, Hkv, D, F, V, g)
    tokens = [3, 17, 29, 5, 11]
    n = len(tokens)
    got = OracleTarget(cfg, w).forward(tokens, 0)

    lw = w["layers"][0]
    h = ew.embed(tokens, formats.bf16_to_f64(w["embed"]))
    x = round_bf16(ew.rmsnorm(h, lw["attn_norm"], cfg.eps))
    qkv = x @ formats.dequant(*lw["qkv"]).T
    q, k, v = ew.rope_qkv(qkv, list(range(n)), Hq, Hkv, D, cfg.theta)
    q, k, v = round_f16(q), round_f16(k), round_f16(v)
    # the block's keys and values on one 16-position page, identity table
    kp = np.zeros((1, Hkv, 16, D), dtype=np.float16)
    vp = np.zeros((1, Hkv, D, 16), dtype=np.float16)
    for i in range(n):
        kp[0, :, i, :] = k[i]
        vp[0, :, :, i] = v[i]
    att = attention.decode_attn(q.astype(np.float16), kp, vp, np.zeros((1, 1), np.int32),
                                np.array([0]), np.array([0, n]), float(D) ** -0.5)
    o = round_f32(att.reshape(n, Hq * D)) @ formats.dequant(*lw["o"]).T
    h = h + o
    x2 = round_bf16(ew.rmsnorm(h, lw["mlp_norm"], cfg.eps))
    mm = round_bf16(ew.silu_mul(x2 @ formats.dequant(*lw["gu"]).T, F))
    h = h + mm @ formats.dequant(*lw["down"]).T
    ref = round_bf16(ew.rmsnorm(h, w["final_norm"], cfg.eps)) @ formats.dequant(*w["lm_head"]).T
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9 * np.abs(ref).max())


def test_step_from_reproduces_each_operation():
    """The per-operation form: fed the rounded intermediates of a layer
    computed step by step from the pinned pieces (paged decode attention,
    row-wise operations, dense dequantised products), every output equals
    that step's exact value, and a projection over chosen rows equals those
    columns of the whole product."""
    H, Hq, Hkv, D, F, V = 64, 4, 2, 16, 64, 40
    cfg = types.SimpleNamespace(H=H, Hq=Hq, Hkv=Hkv, D=D, F=F, V=V, eps=1e-6, theta=1e4)
    g = synth.rng(6)
    w = _weights(H, Hq, Hkv, D, F, V, g)
    lw = w["layers"][0]
    start, n = 3, 4
    pos = list(range(start, start + n))
    h_in = g.standard_normal((n, H))
    delta_in = g.standard_normal((n, H))
    h = h_in + delta_in
    x_ex = ew.rmsnorm(h, lw["attn_norm"], cfg.eps)
    x = round_bf16(x_ex)
    qkv = x @ formats.dequant(*lw["qkv"]).T
    q_ex, k_ex, v_ex = ew.rope_qkv(qkv, pos, Hq, Hkv, D, cfg.theta)
    q, k, v = round_f16(q_ex), round_f16(k_ex), round_f16(v_ex)
    # cache: `start` earlier positions, then the block's own rows
    Kc = np.concatenate([round_f16(g.standard_normal((start, Hkv, D))), k])
    Vc = np.concatenate([round_f16(g.standard_normal((start, Hkv, D))), v])
    kp = np.zeros((1, Hkv, 16, D), dtype=np.float16)
    vp = np.zeros((1, Hkv, D, 16), dtype=np.float16)
    for p in range(start + n):
        kp[0, :, p, :] = Kc[p]
        vp[0, :, :, p] = Vc[p]
    att_ex = attention.decode_attn(q.astype(np.float16), kp, vp, np.zeros((1, 1), np.int32),
                                   np.array([start]), np.array([0, n]), float(D) ** -0.5)
    att = round_f32(att_ex)
    o = att.reshape(n, Hq * D) @ formats.dequant(*lw["o"]).T
    h2 = round_f32(h + o)
    x2_ex = ew.rmsnorm(h2, lw["mlp_norm"], cfg.eps)
    x2 = round_bf16(x2_ex)
    gu = x2 @ formats.dequant(*lw["gu"]).T
    mm_ex = ew.silu_mul(gu, F)
    mm = round_bf16(mm_ex)
    delta = mm @ formats.dequant(*lw["down"]).T
    gpu = {"h_in": h_in, "delta_in": delta_in, "h": h, "x": x, "qkv": qkv, "q": q, "k": k,
           "v": v, "att": att, "o": o, "h2": h2, "x2": x2, "gu": gu, "mm": mm, "delta": delta}
    ref = OracleTarget(cfg, w).step_from(0, gpu, start, Kc, Vc)
    want = {"h": h, "x": x_ex, "qkv": qkv, "q": q_ex, "k": k_ex, "v": v_ex, "att": att_ex,
            "o": o, "h2": h + o, "x2": x2_ex, "gu": gu, "mm": mm_ex, "delta": delta}
    for name, val in want.items():
        np.testing.assert_allclose(ref[name], val, rtol=1e-12, atol=1e-12, err_msg=name)
    rows = {"qkv": [5, 0, 31], "gu": [127, 64], "down": [1], "o": [63, 2]}
    sub = OracleTarget(cfg, w).step_from(0, gpu, start, Kc, Vc, rows=rows)
    out_of = {"qkv": "qkv", "o": "o", "gu": "gu", "down": "delta"}
    for name, r in rows.items():
        np.testing.assert_allclose(sub[out_of[name]], want[out_of[name]][:, r], rtol=1e-12,
                                   atol=1e-12, err_msg=name)
    # the final norm and the lm_head
    xf_ex = ew.rmsnorm(h, w["final_norm"], cfg.eps)
    xf = round_bf16(xf_ex)
    fin = OracleTarget(cfg, w).step_from(None, {"h_in": h_in, "delta_in": delta_in, "h": h,
                                                 "xf": xf}, start, rows={"lm_head": [7, 39]})
    np.testing.assert_allclose(fin["xf"], xf_ex, rtol=1e-12)
    np.testing.assert_allclose(fin["logits"], (xf @ formats.dequant(*w["lm_head"]).T)[:, [7, 39]],
                               rtol=1e-12, atol=1e-12)
