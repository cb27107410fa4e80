"""A synthetic decoder-only target model run entirely through the library's
calls, and the two decoding loops whose outputs must agree byte for byte:
serial greedy decoding (one token per pass) and speculative decoding
(verify passes of a block of drafted tokens).

The pages' end-to-end test is exactly this comparison: deterministic
speculative output must match non-speculative decoding, token for token
(ramgpt.org, "When Lossless Speculation Stops Being Lossless on
Blackwell", sections "Why Tiny Numerical Differences Can Change Entire
Answers", "A Better Backend Test Matrix" and "This Changes How Speculative
Decoding Should Be Benchmarked"; tokenstrom.com, "'Lossless,' but not
quite", section "What the measurements show": 43 of 50 outputs differed).

Layer (pre-norm, residual stream in fp32):
    x   = rmsnorm(h) (bf16)                        add_rmsnorm
    qkv = W_qkv x                                  qgemm_w4 (bf16 activations)
    q,k,v = split + rotary embedding (fp16)        rope_qkv
    append k, v at the block's positions, then     decode_attn_append
    a   = causal attention over the paged cache      (kv_commit APPEND + decode_attn)
    h  += W_o a                                    qgemm_w4 (fp32 activations), add_rmsnorm
    x   = rmsnorm(h)                               add_rmsnorm
    h  += W_down (silu(W_g x) * W_u x)             qgemm_w4, silu_mul, qgemm_w4, add_rmsnorm
then logits = W_lm rmsnorm(h) with each row's argmax keys (qgemm_w4_argmax),
and the decoding loops verify from those keys and commit the accepted rows
in one launch (spec_verify_keys).  Python only sequences the calls and
slices views; every arithmetic step is a library kernel.  One sequence per call
(B = 1), blocks of at most 8 rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

import invariant_speculative_decoding_amd as isd


@dataclass(frozen=True)
class TargetConfig:
    L: int
    H: int
    Hq: int
    Hkv: int
    D: int
    F: int
    V: int
    theta: float = 1e6
    eps: float = 1e-6


class SyntheticTarget:
    """Weights (as produced by ``synth.torch_target_weights``) packed once,
    a paged KV cache per layer over one page table, and the sequence state
    (seq_len = positions in the cache, pos_id = position of the next
    block's first row; the two are equal between passes)."""

    def __init__(self, cfg: TargetConfig, weights, max_pages: int, page_table=None,
                 num_pages=None, device="cuda"):
        self.cfg = cfg
        c = cfg
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({
                "qkv": isd.qgemm_w4_pack(*lw["qkv"]),
                "o": isd.qgemm_w4_pack(*lw["o"]),
                "gu": isd.qgemm_w4_pack(*lw["gu"]),
                "down": isd.qgemm_w4_pack(*lw["down"]),
                "attn_norm": lw["attn_norm"].contiguous(),
                "mlp_norm": lw["mlp_norm"].contiguous(),
            })
        self.embed = weights["embed"].contiguous()
        self.final_norm = weights["final_norm"].contiguous()
        self.lm_head = isd.qgemm_w4_pack(*weights["lm_head"])
        if page_table is None:
            page_table = torch.arange(max_pages, dtype=torch.int32, device=device).view(1, -1)
        self.table = page_table
        P = int(num_pages if num_pages is not None else page_table.max().item() + 1)
        self.kp = [torch.zeros((P, c.Hkv, isd.PAGE, c.D), dtype=torch.float16, device=device)
                   for _ in range(c.L)]
        self.vp = [torch.zeros((P, c.Hkv, c.D, isd.PAGE), dtype=torch.float16, device=device)
                   for _ in range(c.L)]
        self.seq_len = torch.zeros(1, dtype=torch.int32, device=device)
        self.pos_id = torch.zeros(1, dtype=torch.int32, device=device)
        self.scale = float(c.D) ** -0.5
        self.ws_attn = None
        self.device = device

    def forward(self, tokens, trace=None) -> torch.Tensor:
        """Logits [n][V] of a block of n <= 8 rows at positions pos_id ..
        pos_id + n - 1; the block's keys and values are appended to the
        cache (not committed).  With a list `trace`, copies of every
        operation's input and output are appended to it, one dict per layer
        and one for the final norm and lm_head (names as the layer table in
        the module docstring: h_in, delta_in, h, x, qkv, q, k, v, att, o,
        h2, x2, gu, mm, delta; h_in, delta_in, h, xf, logits)."""
        c = self.cfg
        n = tokens.numel()
        rs = torch.tensor([0, n], dtype=torch.int32, device=self.device)
        h = isd.embed_rows(tokens, self.embed)
        delta = None

        def keep(rec, **kw):
            if trace is not None:
                rec.update({k: (None if v is None else v.clone()) for k, v in kw.items()})

        for li, lw in enumerate(self.layers):
            rec = {}
            keep(rec, h_in=h, delta_in=delta)
            x = isd.add_rmsnorm(h, lw["attn_norm"], c.eps, d=delta)
            qkv = isd.qgemm_w4(lw["qkv"], x)
            q, k, v = isd.rope_qkv(qkv, rs, self.pos_id, c.Hq, c.Hkv, c.D, c.theta)
            if self.ws_attn is None:
                self.ws_attn = torch.empty(64 << 20, dtype=torch.uint8, device=self.device)
            # the block's keys and values are appended at pos_id (= seq_len:
            # the commit keeps the two equal) inside the attention launches
            att = isd.decode_attn_append(q, k, v, self.kp[li], self.vp[li], self.table,
                                         self.pos_id, rs, self.scale, ws=self.ws_attn)
            keep(rec, h=h, x=x, qkv=qkv, q=q, k=k, v=v, att=att)
            o = isd.qgemm_w4(lw["o"], att.view(n, c.Hq * c.D))
            x2 = isd.add_rmsnorm(h, lw["mlp_norm"], c.eps, d=o)
            gu = isd.qgemm_w4(lw["gu"], x2)
            mm = isd.silu_mul(gu, c.F)
            delta = isd.qgemm_w4(lw["down"], mm)
            keep(rec, o=o, h2=h, x2=x2, gu=gu, mm=mm, delta=delta)
            if trace is not None:
                trace.append(rec)
        rec = {}
        keep(rec, h_in=h, delta_in=delta)
        xf = isd.add_rmsnorm(h, self.final_norm, c.eps, d=delta)
        # the logits (bit-identical to qgemm_w4's) and each row's argmax keys
        z, self.keys = isd.qgemm_w4_argmax(self.lm_head, xf)
        keep(rec, h=h, xf=xf, logits=z)
        if trace is not None:
            trace.append(rec)
        return z

    def commit(self, accept_len: torch.Tensor):
        """Keep the block's first accept_len + 1 rows in the cache."""
        isd.kv_commit(self.kp[0], self.vp[0], self.table, self.seq_len, self.pos_id,
                      accept_len=accept_len)

    def prefill(self, prompt):
        """Runs all prompt tokens but the last through the model in blocks
        of up to 8 and commits them; returns the last prompt token."""
        toks = [int(t) for t in prompt]
        body = toks[:-1]
        for i in range(0, len(body), 8):
            blk = torch.tensor(body[i:i + 8], dtype=torch.int32, device=self.device)
            self.forward(blk)
            self.commit(torch.tensor([blk.numel() - 1], dtype=torch.int32, device=self.device))
        return toks[-1]


def serial_decode(target: SyntheticTarget, prompt, T: int):
    """Greedy decoding one token per pass; returns the T generated tokens."""
    last = target.prefill(prompt)
    out = []
    rs = torch.tensor([0, 1], dtype=torch.int32, device=target.device)
    no_drafts = torch.zeros(1, dtype=torch.int32, device=target.device)
    while len(out) < T:
        target.forward(torch.tensor([last], dtype=torch.int32, device=target.device))
        # the target's token from the lm_head's argmax keys, committed in the
        # same launch
        acc, toks = isd.spec_verify_keys(target.keys, no_drafts, rs, seq_len=target.seq_len,
                                         pos_id=target.pos_id)
        last = int(toks[0, 0].item())
        out.append(last)
    return out


def speculative_decode(target: SyntheticTarget, prompt, T: int, drafter, k: int):
    """Greedy speculative decoding: each pass verifies the last token plus
    k drafted tokens, accepts the longest agreeing prefix and emits the
    correction (or bonus) token.  `drafter(generated_so_far, k)` returns k
    token ids.  Returns (the first T generated tokens, accepted counts)."""
    last = target.prefill(prompt)
    out, accepts = [], []
    rs = torch.tensor([0, k + 1], dtype=torch.int32, device=target.device)
    while len(out) < T:
        d = [int(t) for t in drafter(out, k)]
        blk = torch.tensor([last] + d, dtype=torch.int32, device=target.device)
        target.forward(blk)
        acc, toks = isd.spec_verify_keys(target.keys, blk[1:].contiguous(), rs,
                                         seq_len=target.seq_len, pos_id=target.pos_id)
        a = int(acc.item())
        em = [int(t) for t in toks[0, : a + 1].tolist()]
        out.extend(em)
        accepts.append(a)
        last = em[-1]
    return out[:T], accepts
