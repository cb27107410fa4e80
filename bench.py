"""Benchmark of the batch-invariant verify pass on one MI355X.

One timed step = one verify pass at every width n = 1..8 (k = n - 1 drafts)
of a single sequence, each pass running the whole hot path on synthetic,
seeded, HBM-resident inputs:

    kv_commit APPEND   n rows of K/V (8 kv-heads x 128) into 16-token pages
    decode_attn        GQA 64/8 x 128, row 0 sees L = 8192 positions
    qgemm_w4           5120x5120, 34816x5120, 5120x17408 (4-bit, bf16 x)
    qgemm_w4           lm_head 152064x5120 -> logits [n][152064]
    spec_verify        greedy accept-prefix on the logits
    spec_verify        rejection sampling (T = 0.8) on the logits against
                       synthetic drafter logits
    kv_commit COMMIT   keep the accepted prefix

`value` is the pass's algorithmic HBM bytes (weights at 0.625 B each, KV,
activations, logits read once and written once) divided by the measured
time, over all widths.  Per-op times come from HIP events recorded on the
stream the kernels run on.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-pass weight GB/s (% HBM peak) at widths 1–8; width-invariance pass rate"
PEAK_GBS = 8000.0

V = 152064
HID = 5120
PROJ = [(5120, 5120), (34816, 5120), (5120, 17408)]
LM = (V, HID)
HQ, HKV, D = 64, 8, 128
L = 8192  # positions seen by row 0
T_SAMPLE = 0.8
WIDTHS = list(range(1, 9))


def weight_bytes(N, K):
    return N * K // 2 + N * (K // 32) * 4


def pass_bytes(n):
    """Algorithmic HBM bytes of one verify pass at width n."""
    w = sum(weight_bytes(N, K) for N, K in PROJ) + weight_bytes(*LM)
    act = sum(n * K * 2 + n * N * 4 for N, K in PROJ + [LM])
    kv = (L + n - 1) * HKV * D * 2 * 2 + n * HQ * D * (2 + 4)
    app = n * HKV * D * 2 * 2 * 2  # read new rows, write pages
    verify = n * V * 4 + (n * V * 4 + (n - 1) * V * 4)  # greedy read; sampled reads
    return w + act + kv + app + verify, w


class Workload:
    def __init__(self, torch, m, seed=1234):
        import synth
        self.t, self.m = torch, m
        dev = "cuda"
        self.W = []
        self.raw = []  # row-major weights (the oracle's input for the CPU baseline)
        for i, (N, K) in enumerate(PROJ + [LM]):
            self.raw.append(synth.torch_quant_weights(N, K, seed + i, dev))
            self.W.append(m.qgemm_w4_pack(*self.raw[-1]))
        self.X = [synth.torch_normal((8, K), seed + 10 + i, torch.bfloat16)
                  for i, (N, K) in enumerate(PROJ + [LM])]
        self.Y = [torch.empty((8, N), dtype=torch.float32, device=dev) for N, K in PROJ + [LM]]
        # paged cache: one sequence, capacity for L + 8 positions, shuffled pages
        self.max_pages = (L + 8 + 15) // 16 + 1
        g = torch.Generator(device="cpu")
        g.manual_seed(seed + 20)
        self.num_pages = 4 * self.max_pages
        self.table = torch.randperm(self.num_pages, generator=g)[: self.max_pages].to(
            torch.int32).view(1, -1).to(dev)
        self.kp = synth.torch_normal((self.num_pages, HKV, 16, D), seed + 21, torch.float16)
        self.vp = synth.torch_normal((self.num_pages, HKV, D, 16), seed + 22, torch.float16)
        self.kn = synth.torch_normal((8, HKV, D), seed + 23, torch.float16)
        self.vn = synth.torch_normal((8, HKV, D), seed + 24, torch.float16)
        self.q = synth.torch_normal((8, HQ, D), seed + 25, torch.float16)
        self.attn_out = torch.empty((8, HQ, D), dtype=torch.float32, device=dev)
        self.seq0 = torch.tensor([L - 1], dtype=torch.int32, device=dev)
        self.seq_len = self.seq0.clone()
        self.pos_id = self.seq0.clone()
        self.row_start = {n: torch.tensor([0, n], dtype=torch.int32, device=dev) for n in WIDTHS}
        self.seq_id = torch.tensor([3], dtype=torch.int32, device=dev)
        # drafter logits for sampling: target-like N(0, 3) values
        self.zd = synth.torch_normal((7, V), seed + 26, torch.float32, std=3.0)
        self.acc = torch.empty(1, dtype=torch.int32, device=dev)
        self.toks = torch.empty((1, 9), dtype=torch.int32, device=dev)
        self.acc2 = torch.empty(1, dtype=torch.int32, device=dev)
        self.toks2 = torch.empty((1, 9), dtype=torch.int32, device=dev)
        self.ws_attn = torch.empty(32 << 20, dtype=torch.uint8, device=dev)
        self.ws_ver = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        self.drafts = {}
        self.sdrafts = {}
        self.scale = float(np.float32(1.0 / np.sqrt(D)))

    def make_drafts(self, rng):
        """Greedy drafts agreeing with the target's (GPU) choices for a
        truncated geometric(0.7) count; sampling drafts uniform."""
        import synth
        t = self.t
        for n in WIDTHS:
            z = self.m.qgemm_w4(self.W[3], self.X[3][:n])
            tk = z.argmax(dim=1).cpu().numpy()
            d, _ = synth.greedy_drafts(tk, n - 1, rng, V, agree=synth.geometric_agree(0.7, n - 1))
            self.drafts[n] = t.tensor(np.append(d, 0).astype(np.int32), device="cuda")
            self.sdrafts[n] = t.tensor(rng.integers(0, V, size=max(n - 1, 1)).astype(np.int32),
                                       device="cuda")

    def verify_pass(self, n, ev=None):
        m, t = self.m, self.t
        rec = (lambda k: ev[k].record()) if ev is not None else (lambda k: None)
        self.seq_len.copy_(self.seq0)  # steady state: every pass starts at L - 1
        self.pos_id.copy_(self.seq0)
        rs = self.row_start[n]
        rec(0)
        m.kv_commit(self.kp, self.vp, self.table, self.seq_len, self.pos_id, row_start=rs,
                    k_new=self.kn[:n], v_new=self.vn[:n])
        rec(1)
        m.decode_attn(self.q[:n], self.kp, self.vp, self.table, self.pos_id, rs, self.scale,
                      out=self.attn_out[:n], ws=self.ws_attn)
        rec(2)
        for i in range(3):
            m.qgemm_w4(self.W[i], self.X[i][:n], y=self.Y[i][:n])
        rec(3)
        z = m.qgemm_w4(self.W[3], self.X[3][:n], y=self.Y[3][:n])
        rec(4)
        m.spec_verify(z, self.drafts[n], rs, accept_len=self.acc, out_tokens=self.toks,
                      ws=self.ws_ver)
        m.spec_verify(z, self.sdrafts[n], rs, draft_logits=self.zd[: max(n - 1, 1)],
                      seq_id=self.seq_id, pos0=self.pos_id, temperature=T_SAMPLE, seed=7,
                      accept_len=self.acc2, out_tokens=self.toks2, ws=self.ws_ver)
        rec(5)
        m.kv_commit(self.kp, self.vp, self.table, self.seq_len, self.pos_id, accept_len=self.acc)
        rec(6)


def invariance_check(t, m, w: Workload):
    """memcmp of every width-n row against the width-one evaluation of that
    row, for the four matrices and attention.  Returns (identical, checked)."""
    ok = tot = 0
    for i in range(4):
        pw = w.W[i]
        one = [m.qgemm_w4(pw, w.X[i][c:c + 1].contiguous()).cpu() for c in range(8)]
        for n in WIDTHS:
            y = m.qgemm_w4(pw, w.X[i][:n].contiguous()).cpu()
            for c in range(n):
                tot += 1
                ok += int(t.equal(y[c].view(t.int32), one[c][0].view(t.int32)))
    rs1 = t.tensor([0, 1], dtype=t.int32, device="cuda")
    one = []
    for i in range(8):
        qp = t.tensor([L - 1 + i], dtype=t.int32, device="cuda")
        one.append(m.decode_attn(w.q[i:i + 1].contiguous(), w.kp, w.vp, w.table, qp, rs1,
                                 w.scale).cpu())
    for n in WIDTHS:
        out = m.decode_attn(w.q[:n].contiguous(), w.kp, w.vp, w.table, w.seq0, w.row_start[n],
                            w.scale).cpu()
        for i in range(n):
            tot += 1
            ok += int(t.equal(out[i].view(t.int32), one[i][0].view(t.int32)))
    return ok, tot


def cpu_baseline(w: Workload, budget_s: float = 20.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    a width-8 verify pass restricted to a slice of every weight matrix's
    rows, one kv-head group of attention, and greedy verify of the sampled
    logits.  Rate = the sample's algorithmic bytes / its time."""
    from oracle import attention as oa
    from oracle import qgemm as oq
    from oracle import verify as ov
    n = 8
    frac_rows = 2048
    t0 = time.perf_counter()
    nbytes = 0
    for i, (N, K) in enumerate(PROJ + [LM]):
        codes, sm = w.raw[i]
        rows = min(N, frac_rows)
        c = codes[:rows].cpu().numpy()
        s = sm[:rows].cpu().numpy().view(np.uint16)
        x = w.X[i][:n].view(w.t.int16).cpu().numpy().view(np.uint16)
        z = oq.qgemm_w4(c, s, x, "bf16")
        nbytes += weight_bytes(rows, K) + n * K * 2 + n * rows * 4
        if time.perf_counter() - t0 > budget_s:
            break
    ov.verify_greedy(z, np.zeros(n - 1, np.int32), np.array([0, n]))
    nbytes += n * z.shape[1] * 4
    # attention: kv-head 0 (8 query heads) at L for the n rows
    kp = w.kp.cpu().numpy()
    vp = w.vp.cpu().numpy()
    q = w.q[:n].cpu().numpy().copy()
    q[:, 8:] = 0
    table = w.table.cpu().numpy()
    kp1 = kp[:, :1]
    vp1 = vp[:, :1]
    oa.decode_attn(q[:, :8], kp1, vp1, table, [L - 1], [0, n], w.scale)
    nbytes += (L + n - 1) * D * 2 * 2
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"width-8 pass on the first {frac_rows} rows of each of the four weight "
                      f"matrices, greedy verify of the sampled logits, one kv-head group of "
                      f"attention at L={L}; {nbytes/1e6:.1f} MB algorithmic in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-invariance", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verify path here is built and timed on a "
              "single MI355X (no multi-GPU path exists); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_speculative_decoding_amd as m
    m.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = Workload(torch, m)
    w.make_drafts(np.random.default_rng(5))
    inv_ok, inv_tot = (0, 0) if args.no_invariance else invariance_check(torch, m, w)

    nev = 7
    for _ in range(args.warmup):
        for n in WIDTHS:
            w.verify_pass(n)
    torch.cuda.synchronize()

    events = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
                  for _ in range(args.steps)] for n in WIDTHS}
    tok = 0
    t0 = time.perf_counter()
    for s in range(args.steps):
        for n in WIDTHS:
            w.verify_pass(n, events[n][s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # tokens emitted per pass (the inputs are the same every step)
    emitted = {}
    for n in WIDTHS:
        w.verify_pass(n)
        emitted[n] = int(w.acc.item()) + 1

    ops = ["kv_append", "decode_attn", "qgemm_proj", "qgemm_lm_head", "spec_verify", "kv_commit"]
    per_w = []
    tot_bytes = tot_w = 0
    tot_ms = 0.0
    lm_ms = []
    op_ms = {o: 0.0 for o in ops}
    for n in WIDTHS:
        ms = [sum(events[n][s][i].elapsed_time(events[n][s][i + 1]) for s in range(args.steps))
              / args.steps for i in range(nev - 1)]
        pm = sum(events[n][s][0].elapsed_time(events[n][s][-1]) for s in range(args.steps)) / args.steps
        b, wb = pass_bytes(n)
        tot_bytes += b
        tot_w += wb
        tot_ms += pm
        lm_ms += [events[n][s][3].elapsed_time(events[n][s][4]) for s in range(args.steps)]
        for o, v in zip(ops, ms):
            op_ms[o] += v / len(WIDTHS)
        per_w.append({"n": n, "us": round(pm * 1e3, 2), "GBps": round(b / (pm * 1e-3) / 1e9, 1),
                      "lm_head_us": round(ms[3] * 1e3, 2), "attn_us": round(ms[1] * 1e3, 2),
                      "proj_us": round(ms[2] * 1e3, 2), "verify_us": round(ms[4] * 1e3, 2)})
    t1 = per_w[0]["us"]
    for p in per_w:
        p["t_over_t1"] = round(p["us"] / t1, 3)
    value = tot_bytes / (tot_ms * 1e-3) / 1e9
    lm_avg_s = float(np.mean(lm_ms)) * 1e-3
    lm_bytes = np.mean([weight_bytes(*LM) + n * HID * 2 + n * V * 4 for n in WIDTHS])
    achieved = lm_bytes / lm_avg_s / 1e9
    ms_step = tot_ms  # one step = the eight passes

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "verify pass at widths 1..8 (k = 0..7 drafts), one sequence: "
                        "kv append, GQA 64/8x128 decode attention at L=8192, 4-bit qgemm "
                        "5120x5120 + 34816x5120 + 5120x17408, 4-bit lm_head 152064x5120, greedy "
                        "and sampled (T=0.8) spec_verify, kv commit",
            "widths": WIDTHS,
            "weights_bytes_per_pass": int(tot_w / len(WIDTHS)),
        },
        "frac_of_hbm_peak": round(value / PEAK_GBS, 4),
        "weight_GBps": round(tot_w / (tot_ms * 1e-3) / 1e9, 1),
        "invariance": {"identical_rows": inv_ok, "checked_rows": inv_tot,
                       "rate": (inv_ok / inv_tot) if inv_tot else None},
        "tokens_per_s": round(sum(emitted.values()) / (tot_ms * 1e-3), 1),
        "emitted_per_pass": [emitted[n] for n in WIDTHS],
        "per_width": per_w,
        "op_avg_us": {o: round(v * 1e3, 2) for o, v in op_ms.items()},
        "wall_s_timed": round(wall, 4),
        "roofline": {"kernel": "qgemm_w4 (lm_head 152064x5120)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                     "avg_us": round(lm_avg_s * 1e6, 2), "bytes_per_launch": int(lm_bytes)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
