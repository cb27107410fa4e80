"""Eager launches of one kernel, for hardware-counter collection.

    python invariant_speculative_decoding_amd/probe.py lm_head [--reps R]
        qgemm_w4 on a 152064 x 5120 4-bit matrix (bf16 activations) at
        widths 1..8, R launches each.
    python invariant_speculative_decoding_amd/probe.py copy [--mib M] [--reps R]
        R device-to-device copies of an M MiB buffer (a plain streaming
        kernel of known size, used to calibrate byte counters).
    python invariant_speculative_decoding_amd/probe.py attn [--L L] [--n N] [--reps R]
        decode_attn, GQA 64/8 x 128, one sequence whose row 0 sees L
        positions on shuffled 16-token pages, width N, R launches.
    python invariant_speculative_decoding_amd/probe.py proj [--N N] [--K K] [--n n] [--reps R]
        qgemm_w4 on one N x K 4-bit matrix at width n, R launches.

Run under a profiler, e.g. rocprofv3 --pmc FETCH_SIZE; prints only a
one-line summary of what it launched.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["lm_head", "copy", "attn", "proj"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--L", type=int, default=8192)
    ap.add_argument("--n", type=int, default=1)
    ap.add_argument("--N", type=int, default=5120)
    ap.add_argument("--K", type=int, default=5120)
    args = ap.parse_args()
    import torch

    import invariant_speculative_decoding_amd as m
    import synth
    if args.what == "lm_head":
        N, K = 152064, 5120
        w = m.qgemm_w4_pack(*synth.torch_quant_weights(N, K, 1237))
        x = synth.torch_normal((8, K), 1247, torch.bfloat16)
        y = torch.empty((8, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for n in range(1, 9):
            for _ in range(args.reps):
                m.qgemm_w4(w, x[:n], y=y[:n])
        torch.cuda.synchronize()
        print(f"probe lm_head: {8 * args.reps} qgemm_w4 launches, N={N} K={K}, widths 1..8")
    elif args.what == "attn":
        Hq, Hkv, D, n, L = 64, 8, 128, args.n, args.L
        max_pages = (L + n - 1 + 15) // 16 + 1
        npg = 2 * max_pages
        kp = synth.torch_normal((npg, Hkv, 16, D), 1, torch.float16)
        vp = synth.torch_normal((npg, Hkv, D, 16), 2, torch.float16)
        q = synth.torch_normal((n, Hq, D), 3, torch.float16)
        g = torch.Generator().manual_seed(4)
        table = torch.randperm(npg, generator=g)[:max_pages].to(torch.int32).view(1, -1).cuda()
        qp = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
        rs = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        out = torch.empty((n, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(args.reps):
            m.decode_attn(q, kp, vp, table, qp, rs, float(D) ** -0.5, out=out, ws=ws)
        torch.cuda.synchronize()
        print(f"probe attn: {args.reps} decode_attn launches, L={L} n={n}")
    elif args.what == "proj":
        N, K, n = args.N, args.K, args.n
        w = m.qgemm_w4_pack(*synth.torch_quant_weights(N, K, 1337))
        x = synth.torch_normal((n, K), 1347, torch.bfloat16)
        y = torch.empty((n, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(args.reps):
            m.qgemm_w4(w, x, y=y)
        torch.cuda.synchronize()
        print(f"probe proj: {args.reps} qgemm_w4 launches, N={N} K={K} n={n}")
    else:
        nb = args.mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"probe copy: {args.reps} copies of {args.mib} MiB")


if __name__ == "__main__":
    main()
