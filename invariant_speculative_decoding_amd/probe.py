"""Eager launches of one kernel, for hardware-counter collection.

    python invariant_speculative_decoding_amd/probe.py lm_head [--reps R] [--fmt w4|q6] [--argmax]
        qgemm_w4 (or qgemm_q6) on a 152064 x 5120 4-bit (6-bit) matrix, bf16
        activations, at widths 1..8, R launches each; with --argmax the
        4-bit product runs as qgemm_w4_argmax (logits and argmax keys).
    python invariant_speculative_decoding_amd/probe.py copy [--mib M] [--reps R]
        R device-to-device copies of an M MiB buffer (a plain streaming
        kernel of known size, used to calibrate byte counters).
    python invariant_speculative_decoding_amd/probe.py attn [--L L] [--n N] [--reps R]
        decode_attn, GQA 64/8 x 128, one sequence whose row 0 sees L
        positions on shuffled 16-token pages, width N, R launches.
    python invariant_speculative_decoding_amd/probe.py proj [--N N] [--K K] [--n n] [--reps R]
                                                           [--fmt w4|q6]
        qgemm_w4 (or qgemm_q6) on one N x K matrix at width n, R launches.
    python invariant_speculative_decoding_amd/probe.py verify [--reps R] [--margin]
        spec_verify at T = 0.8 and spec_verify_commit (greedy) on
        N(0, 3) logits over a 152064-entry vocabulary, one sequence at
        widths 1..8 (uniformly drawn drafts), R launches of each per width;
        with --margin also spec_verify_margin (threshold 1e-3).
    python invariant_speculative_decoding_amd/probe.py model [--T T] [--k k]
        The synthetic 2-layer target at the dense shapes (5120 hidden, GQA
        64/8 x 128, 34816 gate+up, 17408 down, vocabulary 152064): a
        64-token prompt, T tokens of serial greedy decoding, then the same
        T tokens by speculative decoding with k drafts per pass (each draft
        the serial token with probability 0.7, else a random id); checks
        that both emit the same tokens and prints the passes and accepted
        drafts.
    python invariant_speculative_decoding_amd/probe.py step [--reps R] [--rounds N]
        The ragged batched sampled step: 8 sequences at committed lengths
        U{256..16384}, k = 4 drafts each, V = 32000 at T = 0.8; append +
        attention, sampled verify and commit captured as one graph and
        replayed R * N times (lengths restored before each); prints the
        median step time, algorithmic GB/s and tokens/s.

Run under a profiler, e.g. rocprofv3 --pmc FETCH_SIZE; prints only a
one-line summary of what it launched.  With --timed, the lm_head and proj
launches are captured in one HIP graph per width, replayed --rounds times,
and timed with HIP events on the capturing stream; the summary line then
gives the average microseconds per launch, the algorithmic GB/s
(weights at their format's bytes per weight, plus activations and
outputs) and the TFLOP/s of the 2 N K n multiply-adds.
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
    ap.add_argument("what", choices=["lm_head", "copy", "attn", "proj", "verify", "model", "step"])
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--L", type=int, default=8192)
    ap.add_argument("--n", type=int, default=1)
    ap.add_argument("--N", type=int, default=5120)
    ap.add_argument("--K", type=int, default=5120)
    ap.add_argument("--fmt", choices=["w4", "q6"], default="w4")
    ap.add_argument("--timed", action="store_true")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--margin", action="store_true")
    ap.add_argument("--argmax", action="store_true")
    ap.add_argument("--T", type=int, default=32)
    ap.add_argument("--k", type=int, default=4)
    args = ap.parse_args()
    import torch

    import invariant_speculative_decoding_amd as m
    import synth

    def packed(N, K, seed):
        if args.fmt == "q6":
            return m.qgemm_q6_pack(*synth.torch_quant_weights_q6(N, K, seed)), m.qgemm_q6
        w = m.qgemm_w4_pack(*synth.torch_quant_weights(N, K, seed))
        if args.argmax:
            keys = torch.empty((512, m.qgemm_w4_argmax_nkeys(w)), dtype=torch.int64, device="cuda")

            def qgemm_w4_argmax(w, x, y):
                return m.qgemm_w4_argmax(w, x, y=y, keys=keys[:x.shape[0]])
            return w, qgemm_w4_argmax
        return w, m.qgemm_w4

    def bytes_per_weight():
        return 0.625 if args.fmt == "w4" else 0.75 + 1.0 / 16 + 2.0 / 256

    def run_widths(name, f, w, x, y, widths, N, K):
        if not args.timed:
            for n in widths:
                for _ in range(args.reps):
                    f(w, x[:n], y=y[:n])
            torch.cuda.synchronize()
            print(f"probe {name}: {len(widths) * args.reps} {f.__name__} launches, N={N} K={K}, "
                  f"widths {widths[0]}..{widths[-1]}")
            return
        st = torch.cuda.Stream()
        for n in widths:
            f(w, x[:n], y=y[:n])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                for _ in range(args.reps):
                    f(w, x[:n], y=y[:n])
            with torch.cuda.stream(st):
                g.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(args.rounds):
                    g.replay()
                e1.record(st)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (args.rounds * args.reps)
            b = N * K * bytes_per_weight() + n * K * 2 + n * N * 4
            print(f"probe {name} {args.fmt} N={N} K={K} n={n}: {us:.2f} us/launch, "
                  f"{b / us / 1e3:.1f} GB/s, {2.0 * N * K * n / us / 1e6:.2f} TFLOP/s", flush=True)
            del g

    if args.what == "lm_head":
        N, K = 152064, 5120
        w, f = packed(N, K, 1237)
        x = synth.torch_normal((8, K), 1247, torch.bfloat16)
        y = torch.empty((8, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        run_widths("lm_head", f, w, x, y, list(range(1, 9)), N, K)
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
        w, f = packed(N, K, 1337)
        x = synth.torch_normal((n, K), 1347, torch.bfloat16)
        y = torch.empty((n, N), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        run_widths("proj", f, w, x, y, [n], N, K)
    elif args.what == "verify":
        V = 152064
        zt = synth.torch_normal((8, V), 21, torch.float32, std=3.0)
        zd = synth.torch_normal((7, V), 22, torch.float32, std=3.0)
        g = torch.Generator().manual_seed(23)
        drafts = torch.randint(0, V, (7,), generator=g, dtype=torch.int32).cuda()
        seq_id = torch.zeros(1, dtype=torch.int32, device="cuda")
        pos0 = torch.full((1,), 8191, dtype=torch.int32, device="cuda")
        ws_s = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
        ws_g = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for n in range(1, 9):
            rs = torch.tensor([0, n], dtype=torch.int32, device="cuda")
            d = drafts[:max(n - 1, 1)]
            for _ in range(args.reps):
                m.spec_verify(zt[:n], d, rs, draft_logits=zd[:max(n - 1, 1)], seq_id=seq_id,
                              pos0=pos0, temperature=0.8, seed=7, ws=ws_s)
                sl = torch.full((1,), 8191, dtype=torch.int32, device="cuda")
                pid = sl.clone()
                m.spec_verify_commit(zt[:n], d, rs, sl, pid, ws=ws_g)
                if args.margin:
                    m.spec_verify_margin(zt[:n], d, rs, 1e-3, ws=ws_g)
        torch.cuda.synchronize()
        print(f"probe verify: {8 * args.reps} sampled and {8 * args.reps} greedy verify calls"
              f"{' (and margin)' if args.margin else ''}, V={V}")
    elif args.what == "model":
        import numpy as np
        from invariant_speculative_decoding_amd.synthetic_target import (
            SyntheticTarget, TargetConfig, serial_decode, speculative_decode)
        cfg = TargetConfig(L=2, H=5120, Hq=64, Hkv=8, D=128, F=17408, V=152064)
        w = synth.torch_target_weights(cfg.L, cfg.H, cfg.Hq, cfg.Hkv, cfg.D, cfg.F, cfg.V, 31)
        max_pages = (64 + args.T + 8 * (args.k + 1) + 15) // 16 + 1
        g = torch.Generator().manual_seed(32)
        table = torch.randperm(2 * max_pages, generator=g)[:max_pages].to(torch.int32)
        prompt = np.random.default_rng(33).integers(0, cfg.V, size=64)

        def target():
            return SyntheticTarget(cfg, w, max_pages, page_table=table.view(1, -1).cuda(),
                                   num_pages=2 * max_pages)

        ref = serial_decode(target(), prompt, args.T)
        rng = np.random.default_rng(34)

        def drafter(out, k):
            i = len(out)
            return [ref[i + j] if i + j < len(ref) and rng.random() < 0.7
                    else int(rng.integers(0, cfg.V)) for j in range(k)]

        spec, acc = speculative_decode(target(), prompt, args.T, drafter, args.k)
        torch.cuda.synchronize()
        assert spec == ref, "speculative output differs from serial"
        print(f"probe model: prompt 64, serial {args.T} passes; speculative {len(acc)} passes of "
              f"{args.k + 1} rows, {sum(acc)} drafts accepted, {sum(acc) + len(acc)} tokens "
              f"(first {args.T} equal to serial)", flush=True)
    elif args.what == "step":
        # Ragged batched sampled step: 8 sequences at committed lengths
        # U{256..16384} on shuffled 16-token pages, GQA 64/8 x 128, k = 4
        # drafts each (40 rows), V = 32000 at T = 0.8 with target logits
        # N(0, 3) and draft logits target + N(0, 0.5), drafts drawn from the
        # draft distribution.  One step = append + attention, sampled
        # verify, commit; the committed lengths are restored before every
        # step (outside the timed events).
        import numpy as np
        B, Hq, Hkv, D, k, V, T = 8, 64, 8, 128, 4, 32000, 0.8
        n = k + 1
        R = B * n
        g = np.random.default_rng(41)
        C = g.integers(256, 16385, size=B).astype(np.int32)
        max_pages = (int(C.max()) + n + 15) // 16 + 1
        npg = B * max_pages
        perm = torch.randperm(npg, generator=torch.Generator().manual_seed(42))
        table = perm.view(B, max_pages).to(torch.int32).cuda()
        kp = synth.torch_normal((npg, Hkv, 16, D), 43, torch.float16)
        vp = synth.torch_normal((npg, Hkv, D, 16), 44, torch.float16)
        q = synth.torch_normal((R, Hq, D), 45, torch.float16)
        kn = synth.torch_normal((R, Hkv, D), 46, torch.float16)
        vn = synth.torch_normal((R, Hkv, D), 47, torch.float16)
        zt = synth.torch_normal((R, V), 48, torch.float32, std=3.0)
        zd = (zt.view(B, n, V)[:, :k].reshape(B * k, V)
              + synth.torch_normal((B * k, V), 49, torch.float32, std=0.5)).contiguous()
        pq = torch.softmax(zd.cpu().double() / T, dim=1)
        drafts = torch.multinomial(pq, 1, generator=torch.Generator().manual_seed(50))
        drafts = drafts.view(-1).to(torch.int32).cuda()
        rs = (torch.arange(B + 1, dtype=torch.int32) * n).cuda()
        seq_id = torch.arange(B, dtype=torch.int32, device="cuda")
        sl0 = torch.from_numpy(C).cuda()
        sl, pid = sl0.clone(), sl0.clone()
        out = torch.empty((R, Hq, D), dtype=torch.float32, device="cuda")
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        toks = torch.empty((B, m.MAX_OUT), dtype=torch.int32, device="cuda")
        ws_a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        ws_v = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        scale = float(np.float32(1 / np.sqrt(D)))

        def reset():
            sl.copy_(sl0)
            pid.copy_(sl0)

        def step():
            m.decode_attn_append(q, kn, vn, kp, vp, table, pid, rs, scale, out=out, ws=ws_a)
            m.spec_verify(zt, drafts, rs, draft_logits=zd, seq_id=seq_id, pos0=pid,
                          temperature=T, seed=7, accept_len=acc, out_tokens=toks, ws=ws_v)
            m.kv_commit(kp, vp, table, sl, pid, accept_len=acc)

        for _ in range(2):
            reset()
            step()
        torch.cuda.synchronize()
        emitted = int(acc.sum().item()) + B
        st = torch.cuda.Stream()
        gs, gr = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs, stream=st):
            step()
        with torch.cuda.graph(gr, stream=st):
            reset()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.rounds * args.reps)]
        with torch.cuda.stream(st):
            for e0, e1 in ev:
                gr.replay()
                e0.record(st)
                gs.replay()
                e1.record(st)
        torch.cuda.synchronize()
        us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        kv = int(((C.astype(np.int64) + n) * Hkv * D * 2 * 2).sum())
        b = kv + R * Hq * D * (2 + 4) + R * Hkv * D * 2 * 2 * 2 + (R + B * k) * V * 4
        print(f"probe step: B={B} L=U{{256..16384}} (sum {int(C.sum())}) k={k} V={V} T={T}: "
              f"{us:.2f} us/step (median of {len(ev)}), {b / 1e6:.1f} MB algorithmic, "
              f"{b / us / 1e3:.1f} GB/s ({b / us / 1e3 / 8000:.3f} of 8 TB/s), "
              f"{emitted} tokens emitted per step, {emitted / us * 1e6:.0f} tokens/s", flush=True)
        del gs, gr
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
