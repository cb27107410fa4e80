"""Forward pass of the synthetic decoder-only target (oracle; test
infrastructure).

The composition the library runs layer by layer (see the layer operations
in ``elementwise``): pre-norm attention and SiLU-gated MLP blocks around
4-bit projections, with the residual stream kept unrounded.  The values
the method stores in reduced precision are rounded here at the same
points: activations entering a projection are bf16 (rounded to nearest
even from the exact normalised value), queries, keys and values are fp16,
the attention output enters its projection as fp32, and the gated MLP
product is bf16.  Everything else is fp64.

It backs the end-to-end check that speculative decoding reproduces serial
decoding (ramgpt.org, "When Lossless Speculation Stops Being Lossless on
Blackwell", section "A Better Backend Test Matrix": end-to-end greedy
generation equivalence): the oracle pins the composition of a small model,
the equivalence itself is a property of the GPU outputs.
"""
from __future__ import annotations

import numpy as np

from . import elementwise as ew
from . import formats


def round_bf16(x):
    """Nearest bf16 value (ties to even) of fp64 values, returned as fp64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)  # 8 significant bits


def round_f16(x):
    """Nearest fp16 value of fp64 values, returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


class OracleTarget:
    """Weights as host arrays: per layer (codes, scale_min) of qkv, o, gu and
    down, the two norm weights; the bf16 embedding table (bits), the final
    norm and the lm_head (codes, scale_min).  Keeps its own fp16 key/value
    cache per layer, one entry per committed or appended position."""

    def __init__(self, cfg, weights):
        self.cfg = cfg
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({
                "qkv": formats.dequant(*lw["qkv"]),
                "o": formats.dequant(*lw["o"]),
                "gu": formats.dequant(*lw["gu"]),
                "down": formats.dequant(*lw["down"]),
                "attn_norm": np.asarray(lw["attn_norm"], dtype=np.float64),
                "mlp_norm": np.asarray(lw["mlp_norm"], dtype=np.float64),
            })
        self.embed = formats.bf16_to_f64(weights["embed"])
        self.final_norm = np.asarray(weights["final_norm"], dtype=np.float64)
        self.lm_head = formats.dequant(*weights["lm_head"])
        self.K = [[] for _ in self.layers]  # per layer: list of [Hkv][D] per position
        self.V = [[] for _ in self.layers]

    def forward(self, tokens, start: int):
        """Logits [n][V] of a block whose row i sits at position start + i
        and sees positions 0 .. start + i; the cache must hold exactly the
        positions before `start` (the block's entries are appended)."""
        c = self.cfg
        n = len(tokens)
        positions = [start + i for i in range(n)]
        h = ew.embed(tokens, self.embed)
        delta = None
        for li, lw in enumerate(self.layers):
            assert len(self.K[li]) == start
            if delta is not None:
                h = h + delta
            x = round_bf16(ew.rmsnorm(h, lw["attn_norm"], c.eps))
            qkv = x @ lw["qkv"].T
            q, k, v = ew.rope_qkv(qkv, positions, c.Hq, c.Hkv, c.D, c.theta)
            q, k, v = round_f16(q), round_f16(k), round_f16(v)
            for i in range(n):
                self.K[li].append(k[i])
                self.V[li].append(v[i])
            Kc = np.stack(self.K[li])  # [pos][Hkv][D]
            Vc = np.stack(self.V[li])
            grp = c.Hq // c.Hkv
            att = np.zeros((n, c.Hq, c.D))
            for i in range(n):
                vis = start + i + 1
                for hq in range(c.Hq):
                    g = hq // grp
                    s = (Kc[:vis, g, :] @ q[i, hq]) * (float(c.D) ** -0.5)
                    p = np.exp(s - s.max())
                    att[i, hq] = (p / p.sum()) @ Vc[:vis, g, :]
            o = round_f32(att.reshape(n, c.Hq * c.D)) @ lw["o"].T
            h = h + o
            x2 = round_bf16(ew.rmsnorm(h, lw["mlp_norm"], c.eps))
            gu = x2 @ lw["gu"].T
            mm = round_bf16(ew.silu_mul(gu, c.F))
            delta = mm @ lw["down"].T
        h = h + delta
        xf = round_bf16(ew.rmsnorm(h, self.final_norm, c.eps))
        return xf @ self.lm_head.T

    def truncate(self, length: int):
        """Roll the caches back to `length` positions."""
        for li in range(len(self.layers)):
            del self.K[li][length:]
            del self.V[li][length:]
