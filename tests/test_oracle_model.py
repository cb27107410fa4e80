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
