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
    cache per layer, one entry per committed or appended position.  A
    matrix is dequantised when first used whole (``forward``); ``step_from``
    may dequantise only the rows it is asked for."""

    def __init__(self, cfg, weights):
        self.cfg = cfg
        self.raw = []
        self.layers = []
        for lw in weights["layers"]:
            self.raw.append({k: lw[k] for k in ("qkv", "o", "gu", "down")})
            self.layers.append({
                "attn_norm": np.asarray(lw["attn_norm"], dtype=np.float64),
                "mlp_norm": np.asarray(lw["mlp_norm"], dtype=np.float64),
            })
        self.raw_embed = weights["embed"]
        self._embed = None
        self.final_norm = np.asarray(weights["final_norm"], dtype=np.float64)
        self.raw_lm = weights["lm_head"]
        self._full = {}
        self.K = [[] for _ in self.layers]  # per layer: list of [Hkv][D] per position
        self.V = [[] for _ in self.layers]

    @property
    def embed(self):
        """The embedding table in fp64 (converted on first use)."""
        if self._embed is None:
            self._embed = formats.bf16_to_f64(self.raw_embed)
        return self._embed

    def _pair(self, li, name):
        return self.raw_lm if name == "lm_head" else self.raw[li][name]

    def weight(self, li, name):
        """The whole dequantised matrix (fp64), kept after the first use."""
        key = (li, name) if name != "lm_head" else name
        if key not in self._full:
            self._full[key] = formats.dequant(*self._pair(li, name))
        return self._full[key]

    def proj(self, x, li, name, rows=None):
        """x @ W.T in fp64 (x exact), over the given output rows of W only."""
        if rows is None:
            return np.asarray(x, dtype=np.float64) @ self.weight(li, name).T
        codes, sm = self._pair(li, name)
        w = formats.dequant(np.asarray(codes)[rows], np.asarray(sm)[rows])
        return np.asarray(x, dtype=np.float64) @ w.T

    def attention(self, q, Kc, Vc, start: int):
        """Causal attention of block rows q [n][Hq][D] over cached keys and
        values Kc, Vc [pos][Hkv][D]: row i sees positions 0 .. start + i
        (plain softmax in fp64)."""
        c = self.cfg
        n = q.shape[0]
        grp = c.Hq // c.Hkv
        att = np.zeros((n, c.Hq, c.D))
        for i in range(n):
            vis = start + i + 1
            for hq in range(c.Hq):
                g = hq // grp
                s = (Kc[:vis, g, :] @ q[i, hq]) * (float(c.D) ** -0.5)
                p = np.exp(s - s.max())
                att[i, hq] = (p / p.sum()) @ Vc[:vis, g, :]
        return att

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
            qkv = self.proj(x, li, "qkv")
            q, k, v = ew.rope_qkv(qkv, positions, c.Hq, c.Hkv, c.D, c.theta)
            q, k, v = round_f16(q), round_f16(k), round_f16(v)
            for i in range(n):
                self.K[li].append(k[i])
                self.V[li].append(v[i])
            att = self.attention(q, np.stack(self.K[li]), np.stack(self.V[li]), start)
            o = self.proj(round_f32(att.reshape(n, c.Hq * c.D)), li, "o")
            h = h + o
            x2 = round_bf16(ew.rmsnorm(h, lw["mlp_norm"], c.eps))
            gu = self.proj(x2, li, "gu")
            mm = round_bf16(ew.silu_mul(gu, c.F))
            delta = self.proj(mm, li, "down")
        h = h + delta
        xf = round_bf16(ew.rmsnorm(h, self.final_norm, c.eps))
        return self.proj(xf, None, "lm_head")

    def step_from(self, li, g, start: int, Kc=None, Vc=None, rows=None):
        """Every operation of layer li (li = None: the final norm and the
        lm_head) evaluated in fp64 on the inputs the GPU gave that operation,
        so that each GPU output can be compared with the exact value of its
        own operation, without the rounding differences of earlier
        operations carried along.  `g` maps names to the GPU's arrays (as
        fp64): "h_in" (residual before the layer's addition), "delta_in"
        (the addition, absent for the first layer), "h" (residual after it),
        "x", "qkv", "q", "k", "v", "att", "o", "h2", "x2", "gu", "mm",
        "delta"; for li = None "h_in", "delta_in", "h", "xf", "logits".
        Kc, Vc: the GPU's cache [pos][Hkv][D] of this layer through the
        block.  `rows` maps a projection name to the output rows to compute
        (all when absent).  Returns a dict with the exact (unrounded) value
        of each GPU output under the same name; projections restricted to
        rows give only those columns."""
        c = self.cfg
        rows = rows or {}
        r = {}
        n = g["h_in"].shape[0]
        d = g.get("delta_in")
        r["h"] = g["h_in"] + d if d is not None else g["h_in"]
        if li is None:
            r["xf"] = ew.rmsnorm(g["h"], self.final_norm, c.eps)
            r["logits"] = self.proj(g["xf"], None, "lm_head", rows.get("lm_head"))
            return r
        lw = self.layers[li]
        positions = [start + i for i in range(n)]
        r["x"] = ew.rmsnorm(g["h"], lw["attn_norm"], c.eps)
        r["qkv"] = self.proj(g["x"], li, "qkv", rows.get("qkv"))
        r["q"], r["k"], r["v"] = ew.rope_qkv(g["qkv"], positions, c.Hq, c.Hkv, c.D, c.theta)
        r["att"] = self.attention(g["q"], Kc, Vc, start)
        r["o"] = self.proj(g["att"].reshape(n, c.Hq * c.D), li, "o", rows.get("o"))
        r["h2"] = g["h"] + g["o"]
        r["x2"] = ew.rmsnorm(g["h2"], lw["mlp_norm"], c.eps)
        r["gu"] = self.proj(g["x2"], li, "gu", rows.get("gu"))
        r["mm"] = ew.silu_mul(g["gu"], c.F)
        r["delta"] = self.proj(g["mm"], li, "down", rows.get("down"))
        return r

    def truncate(self, length: int):
        """Roll the caches back to `length` positions."""
        for li in range(len(self.layers)):
            del self.K[li][length:]
            del self.V[li][length:]
