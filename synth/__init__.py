"""Seeded synthetic inputs for the verify path.

This module only draws random numbers and lays them out in the storage
formats the library and the oracle both accept.  It holds none of the
method's arithmetic: no dequantisation, no products, no softmax, no
argmax, no accept rule, no slot-to-page mapping.  Quantities that depend
on the method's results (drafts that agree with the target's argmax,
planted near-ties) are built by the callers from results they computed
themselves; the helpers here only take those results as plain inputs.

Storage formats produced here:

* 4-bit block weights: ``codes`` is ``uint8[N][K/2]`` (element ``2t`` of a
  row in the low nibble of byte ``t``, element ``2t+1`` in the high nibble),
  ``scale_min`` is ``uint16[N][K/32][2]`` holding the raw fp16 bits of the
  block scale ``d`` and block minimum ``m`` (``w = d*q + m``).
* 6-bit super-block weights: ``ql`` is ``uint8[N][K/2]`` (the low four
  bits of each code, element ``2t`` in the low nibble of byte ``t``),
  ``qh`` is ``uint8[N][K/4]`` (the high two bits, element ``4t+i`` in bits
  ``2i, 2i+1`` of byte ``t``), ``sc`` is ``int8[N][K/16]`` (one scale per
  16-value sub-block) and ``d`` is ``uint16[N][K/256]`` holding the fp16
  bits of one scale per 256-value super-block
  (``w = d * sc * (q - 32)``, ``q`` in 0..63).
* bf16 values travel as raw ``uint16`` bits (the upper half of an fp32,
  rounded to nearest-even).
* fp16 values travel as ``numpy.float16`` arrays (or their ``uint16`` view).
* The key cache is ``f16[num_pages][Hkv][16][D]`` and the value cache is
  ``f16[num_pages][Hkv][D][16]``; a page table ``int32[B][max_pages]`` names
  the page that holds positions ``16p .. 16p+15`` of a sequence.
"""
from __future__ import annotations

import numpy as np

PAGE = 16  # positions per KV page


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 / fp16

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- weights

def quant_weights(N: int, K: int, g: np.random.Generator,
                  d_lo: float = 0.005, d_hi: float = 0.02,
                  codes_fill: int | None = None):
    """Random 4-bit block weights: codes uniform in 0..15, d ~ U(d_lo, d_hi)
    rounded to fp16, m = fp16(-8*d) (exact: a power-of-two multiple).

    Returns (codes uint8[N][K//2], scale_min uint16[N][K//32][2]).
    """
    assert K % 32 == 0
    if codes_fill is None:
        q = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    else:
        q = np.full((N, K), codes_fill, dtype=np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    d = g.uniform(d_lo, d_hi, size=(N, K // 32)).astype(np.float16)
    m = (-8.0 * d.astype(np.float64)).astype(np.float16)
    sm = np.empty((N, K // 32, 2), dtype=np.uint16)
    sm[..., 0] = d.view(np.uint16)
    sm[..., 1] = m.view(np.uint16)
    return codes, sm


def quant_weights_from(q: np.ndarray, d: np.ndarray, m: np.ndarray):
    """Pack explicit codes q[N][K] (0..15) and fp16 d, m [N][K//32]."""
    q = np.asarray(q, dtype=np.uint8)
    assert q.max(initial=0) < 16
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sm = np.empty(d.shape + (2,), dtype=np.uint16)
    sm[..., 0] = np.asarray(d, dtype=np.float16).view(np.uint16)
    sm[..., 1] = np.asarray(m, dtype=np.float16).view(np.uint16)
    return codes, sm


def q6_from_codes(q: np.ndarray, sc: np.ndarray, d: np.ndarray):
    """Lay out explicit 6-bit codes q[N][K] (0..63), int8 sub-block scales
    sc[N][K//16] and fp16 super-block scales d[N][K//256] in the storage
    format.  Returns (ql, qh, sc int8, d uint16 bits)."""
    q = np.asarray(q, dtype=np.uint8)
    assert q.max(initial=0) < 64 and q.shape[1] % 256 == 0
    lo, hi = q & 0x0F, q >> 4
    ql = (lo[:, 0::2] | (lo[:, 1::2] << 4)).astype(np.uint8)
    qh = (hi[:, 0::4] | (hi[:, 1::4] << 2) | (hi[:, 2::4] << 4) | (hi[:, 3::4] << 6)).astype(np.uint8)
    return (ql, qh, np.asarray(sc, dtype=np.int8),
            np.asarray(d, dtype=np.float16).view(np.uint16))


def quant_weights_q6(N: int, K: int, g: np.random.Generator,
                     d_lo: float = 6.2e-5, d_hi: float = 1.9e-4):
    """Random 6-bit super-block weights: codes uniform in 0..63, sub-block
    scales uniform over the whole int8 range, d ~ U(d_lo, d_hi) rounded to
    fp16 (normal fp16 values).  Returns (ql, qh, sc, d) as ``q6_from_codes``."""
    assert K % 256 == 0
    q = g.integers(0, 64, size=(N, K), dtype=np.uint8)
    sc = g.integers(-128, 128, size=(N, K // 16)).astype(np.int8)
    d = g.uniform(d_lo, d_hi, size=(N, K // 256)).astype(np.float16)
    return q6_from_codes(q, sc, d)


# ---------------------------------------------------------------- activations

def activations(n: int, K: int, dtype: str, g: np.random.Generator):
    """x[n][K] drawn N(0,1) in fp32; returned as fp32 or as bf16 bits."""
    x = g.standard_normal((n, K), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def f16_normal(shape, g: np.random.Generator, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape) * std).astype(np.float16)


# ---------------------------------------------------------------- paged cache

def page_table(B: int, max_pages: int, g: np.random.Generator,
               shuffle: bool = True, num_pages: int | None = None):
    """Give each sequence max_pages distinct pages out of a pool.

    With shuffle, page ids are a seeded permutation of the pool; without,
    sequence s owns pages s*max_pages .. s*max_pages+max_pages-1 in order
    (an identity table for B == 1).
    """
    total = B * max_pages
    if num_pages is None:
        num_pages = total
    assert num_pages >= total
    ids = g.permutation(num_pages)[:total] if shuffle else np.arange(total)
    return ids.reshape(B, max_pages).astype(np.int32), num_pages


def kv_pages(num_pages: int, Hkv: int, D: int, g: np.random.Generator):
    """Fill whole key and value caches with N(0,1) fp16 values."""
    k = f16_normal((num_pages, Hkv, PAGE, D), g)
    v = f16_normal((num_pages, Hkv, D, PAGE), g)
    return k, v


# ---------------------------------------------------------------- drafts

def greedy_drafts(targets, k: int, g: np.random.Generator, V: int,
                  agree=None):
    """Drafts d_1..d_k for a greedy verify block.

    ``targets[j]`` is the target's choice after input j (j = 0..k), computed
    by the caller.  The first ``a`` drafts copy targets[0..a-1]; d_{a+1} is
    uniform over the vocabulary minus targets[a]; later drafts are uniform.
    ``agree`` is either an int or a callable drawing it from ``g``.
    """
    a = agree(g) if callable(agree) else int(agree)
    a = max(0, min(k, a))
    d = g.integers(0, V, size=k).astype(np.int64)
    d[:a] = np.asarray(targets[:a])
    if a < k:
        r = int(g.integers(0, V - 1))
        t = int(targets[a])
        d[a] = r if r < t else r + 1
    return d.astype(np.int32), a


def geometric_agree(p: float, k: int):
    """Number of leading drafts that agree: each further draft keeps agreeing
    with probability p until the first miss, truncated at k
    (so P(a >= j) = p**j)."""
    def draw(g: np.random.Generator) -> int:
        a = 0
        while a < k and g.random() < p:
            a += 1
        return a
    return draw


def uniform_agree(lo: int, hi: int):
    def draw(g: np.random.Generator) -> int:
        return int(g.integers(lo, hi + 1))
    return draw


def gumbel_draws(draft_logits: np.ndarray, temperature: float,
                 g: np.random.Generator) -> np.ndarray:
    """Draft tokens a drafter would sample from its own logits at the given
    temperature (Gumbel-max on fp64 logits).  This is the drafter's side of
    the step, not the verifier's."""
    z = np.asarray(draft_logits, dtype=np.float64) / temperature
    u = g.random(z.shape)
    gum = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
    return np.argmax(z + gum, axis=-1).astype(np.int32)


# ---------------------------------------------------------------- on-device

def torch_quant_weights(N: int, K: int, seed: int, device="cuda",
                        d_lo: float = 0.005, d_hi: float = 0.02):
    """Same distribution as ``quant_weights`` drawn directly on the device
    with a seeded torch generator (for large benchmark matrices): uniform
    code bytes (two uniform nibbles), d ~ U(d_lo, d_hi) rounded to fp16,
    m = fp16(-8 d).  Returns (codes uint8[N][K/2], scale_min int16[N][K/32][2]
    holding the fp16 bits)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=gen)
    d = (torch.rand((N, K // 32), device=device, generator=gen, dtype=torch.float64)
         * (d_hi - d_lo) + d_lo).to(torch.float16)
    m = (-8.0 * d.to(torch.float64)).to(torch.float16)
    sm = torch.stack([d, m], dim=-1).contiguous().view(torch.int16)
    return codes, sm


def torch_quant_weights_q6(N: int, K: int, seed: int, device="cuda",
                           d_lo: float = 6.2e-5, d_hi: float = 1.9e-4):
    """Same distribution as ``quant_weights_q6`` drawn on the device with a
    seeded torch generator: uniform ql and qh bytes (uniform codes), uniform
    int8 sub-block scales, d ~ U(d_lo, d_hi) rounded to fp16.  Returns (ql,
    qh uint8, sc int8, d int16 holding the fp16 bits)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    ql = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=device, generator=gen)
    qh = torch.randint(0, 256, (N, K // 4), dtype=torch.uint8, device=device, generator=gen)
    sc = torch.randint(-128, 128, (N, K // 16), dtype=torch.int8, device=device, generator=gen)
    d = (torch.rand((N, K // 256), device=device, generator=gen, dtype=torch.float64)
         * (d_hi - d_lo) + d_lo).to(torch.float16)
    return ql, qh, sc, d.view(torch.int16)


def torch_normal(shape, seed: int, dtype, device="cuda", std: float = 1.0):
    """N(0, std^2) fp32 draws on the device, rounded to ``dtype``
    (torch.float16 / torch.bfloat16 round to nearest even)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(shape, device=device, generator=gen, dtype=torch.float32) * std
    return x.to(dtype)


def torch_target_weights(L: int, H: int, Hq: int, Hkv: int, D: int, F: int, V: int, seed: int,
                         device="cuda"):
    """Random weights of a synthetic decoder-only target, drawn on the
    device: per layer the 4-bit matrices qkv [(Hq + 2 Hkv) D][H], o
    [H][Hq D], gate+up [2F][H] and down [H][F] (row-major codes and fp16
    scale/min, as ``torch_quant_weights``) and RMS-norm weights 1 +
    0.1 N(0,1) (fp32); a bf16 N(0,1) embedding table [V][H], a final norm
    weight and a 4-bit lm_head [V][H].  Seeds are derived from `seed`."""
    import torch
    layers = []
    for li in range(L):
        s0 = seed + 100 * (li + 1)
        layers.append({
            "qkv": torch_quant_weights((Hq + 2 * Hkv) * D, H, s0 + 1, device),
            "o": torch_quant_weights(H, Hq * D, s0 + 2, device),
            "gu": torch_quant_weights(2 * F, H, s0 + 3, device),
            "down": torch_quant_weights(H, F, s0 + 4, device),
            "attn_norm": 1.0 + 0.1 * torch_normal((H,), s0 + 5, torch.float32, device),
            "mlp_norm": 1.0 + 0.1 * torch_normal((H,), s0 + 6, torch.float32, device),
        })
    return {
        "layers": layers,
        "embed": torch_normal((V, H), seed + 7, torch.bfloat16, device),
        "final_norm": 1.0 + 0.1 * torch_normal((H,), seed + 8, torch.float32, device),
        "lm_head": torch_quant_weights(V, H, seed + 9, device),
    }
