"""Eager launches of one kernel, for hardware-counter collection.

    python invariant_speculative_decoding_amd/probe.py lm_head [--reps R]
        qgemm_w4 on a 152064 x 5120 4-bit matrix (bf16 activations) at
        widths 1..8, R launches each.
    python invariant_speculative_decoding_amd/probe.py copy [--mib M] [--reps R]
        R device-to-device copies of an M MiB buffer (a plain streaming
        kernel of known size, used to calibrate byte counters).

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
    ap.add_argument("what", choices=["lm_head", "copy"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--mib", type=int, default=1024)
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
