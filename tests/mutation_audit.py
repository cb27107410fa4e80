"""Mutation audit of the oracle (test infrastructure, run by hand; not
collected by pytest).

Each entry below plants one plausible mistake in a copy of an oracle module
(a dropped term, a wrong sign, index, offset, layout or constant) and runs
the CPU test suite on that copy; the audit passes when every planted mistake
makes some test fail.  Nothing here touches the repository's own files.

    python tests/mutation_audit.py [index ...]
"""
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

M = [
 ("formats", "q[:, 0::2] = c & 0x0F\n    q[:, 1::2] = c >> 4", "q[:, 0::2] = c >> 4\n    q[:, 1::2] = c & 0x0F", "nibble order swapped"),
 ("formats", "(d[:, :, None] * qb + m[:, :, None])", "(d[:, :, None] * qb)", "minimum dropped"),
 ("formats", "(d[:, :, None] * qb + m[:, :, None])", "(d[:, :, None] * qb - m[:, :, None])", "minimum sign"),
 ("formats", "d = f16_to_f64(sm[..., 0])\n    m = f16_to_f64(sm[..., 1])", "d = f16_to_f64(sm[..., 1])\n    m = f16_to_f64(sm[..., 0])", "scale/min swapped"),
 ("formats", "(b.astype(np.uint32) << np.uint32(16))", "(b.astype(np.uint32) << np.uint32(15))", "bf16 shift"),
 ("formats", "e = [pb[b] & 15 for b in range(4)] + [pb[b] >> 4 for b in range(4)]", "e = [pb[b] >> 4 for b in range(4)] + [pb[b] & 15 for b in range(4)]", "packed nibble halves"),
 ("formats", "sm[16 * T + i, 4 * S + j, :] = sp[T, S, i, j, :]", "sm[16 * T + i, 4 * S + j, :] = sp[T, S, i, 3 - j, :]", "packed scale block order"),
 ("formats", "return np.asarray(x, dtype=np.float32).astype(np.float64)", "return np.asarray(x, dtype=np.float16).astype(np.float64)", "f32 activations narrowed"),
 ("formats", "hi[:, i::4] = (h >> (2 * i)) & 3", "hi[:, i::4] = (h >> (2 * (3 - i))) & 3", "q6 high-bit order"),
 ("formats", "return lo + 16 * hi", "return lo + 8 * hi", "q6 high-bit weight"),
 ("formats", "(q.reshape(N, K // 16, 16) - 32.0)", "(q.reshape(N, K // 16, 16) - 31.0)", "q6 offset"),
 ("formats", "per_sub = (dd[:, :, None] * s.reshape(N, K // 256, 16))", "per_sub = (dd[:, :, None] * np.abs(s).reshape(N, K // 256, 16))", "q6 sub-scale sign"),
 ("formats", "sc[16 * T:16 * T + 16, 8 * S + 2 * p + h] = srec[:, h, p] - 128", "sc[16 * T:16 * T + 16, 8 * S + 2 * p + h] = srec[:, p % 2, 2 * h + p // 2] - 128", "q6 packed sub-scale order"),
 ("qgemm", "out[:, s:s + sel.size] = xs @ W.T\n    return out\n\n\ndef qgemm_q6", "out[:, s:s + sel.size] = xs[::-1] @ W.T\n    return out\n\n\ndef qgemm_q6", "activation rows reversed"),
 ("attention", "m = int(np.searchsorted(pos, int(q_pos[s]) + i + 1))", "m = int(np.searchsorted(pos, int(q_pos[s]) + i))", "visible length off by one"),
 ("attention", "sc = scale * (Kv @ q[r, h])", "sc = (Kv @ q[r, h])", "scale dropped"),
 ("attention", "                h = g * grp + hh\n                sc = scale", "                h = hh * Hkv + g\n                sc = scale", "GQA head mapping"),
 ("attention", "out[r, h] = (w / w.sum()) @ Vv", "out[r, h] = (w / w.max()) @ Vv", "normaliser"),
 ("attention", "K[p] = f16_to_f64(k_pages[pg, g, off, :])", "K[p] = f16_to_f64(k_pages[pg, g, (off + 1) % PAGE, :])", "key slot offset"),
 ("attention", "V[p] = f16_to_f64(v_pages[pg, g, :, off])", "V[p] = f16_to_f64(v_pages[pg, g, :, (off + 1) % PAGE])", "value slot offset"),
 ("attention", "return int(page_table[s][p // PAGE]), p % PAGE", "return int(page_table[0][p // PAGE]), p % PAGE", "page table row"),
 ("attention", "            if 0 <= int(page_table[s][p // PAGE]) < num_pages]", "            if int(page_table[s][p // PAGE]) < num_pages]", "negative page ids present"),
 ("attention", "range(max(0, min(end, cap)))", "range(max(0, end))", "positions past the table"),
 ("attention", "a_old = np.exp(M - Mn) if M", "a_old = np.exp(Mn - M) if M", "LSE rescale sign"),
 ("attention", "A = A * a_old + ac * np.exp(mc - Mn)", "A = A + ac * np.exp(mc - Mn)", "LSE numerator rescale dropped"),
 ("verify", "return int(np.flatnonzero(zz == best)[0])", "return int(np.flatnonzero(zz == best)[-1])", "tie-break highest index"),
 ("verify", "zz = np.where(np.isnan(z), -np.inf, z)", "zz = np.where(np.isnan(z), np.inf, z)", "NaN wins"),
 ("verify", "return float(z[-1] - z[-2])", "return float(z[-1] - z[-3])", "margin second index"),
 ("verify", "return a, [int(v) for v in drafts[:a]] + [int(targets[a])]", "return a, [int(v) for v in drafts[:a]] + [int(targets[min(a + 1, k)])]", "correction token row"),
 ("verify", "while a < k and int(drafts[a]) == int(targets[a]):", "while a < k - 1 and int(drafts[a]) == int(targets[a]):", "accept bound"),
 ("verify", "d = np.asarray(drafts)[r0 - s: r0 - s + k]", "d = np.asarray(drafts)[r0: r0 + k]", "ragged draft offset"),
 ("verify", "for j in range(int(accept_len[s]) + 1):", "for j in range(int(accept_len[s])):", "recheck rows range"),
 ("verify", "x = np.asarray(z, dtype=np.float64) / float(temperature)", "x = np.asarray(z, dtype=np.float64) * float(temperature)", "temperature inverted"),
 ("verify", "v = int(np.searchsorted(c, t, side=\"right\"))", "v = int(np.searchsorted(c, t, side=\"left\"))", "inverse CDF side"),
 ("verify", "    r = np.maximum(0.0, p - q)\n    if r.sum() == 0.0:\n        r = p\n    c = np.cumsum(r)", "    r = np.maximum(0.0, q - p)\n    if r.sum() == 0.0:\n        r = p\n    c = np.cumsum(r)", "residual sign (vectorised)"),
 ("verify", "ratio = np.where(q[x] > 0, p[x] / np.where(q[x] > 0, q[x], 1.0), np.inf)", "ratio = np.where(p[x] > 0, q[x] / np.where(p[x] > 0, p[x], 1.0), np.inf)", "ratio inverted (vectorised)"),
 ("verify", "u = philox.uniform(seed, sid, p0 + j - 1, philox.STREAM_ACCEPT)", "u = philox.uniform(seed, sid, p0 + j, philox.STREAM_ACCEPT)", "accept uniform position"),
 ("verify", "u = philox.uniform(seed, sid, p0 + j - 1, philox.STREAM_ACCEPT)", "u = philox.uniform(seed, sid, p0 + j - 1, philox.STREAM_SAMPLE)", "accept uniform stream"),
 ("verify", "            if 0 <= x < len(p):\n", "            if x < len(p):\n", "draft id below the vocabulary accepted"),
 ("verify", "                r = np.maximum(0.0, p - q)\n                if r.sum() == 0.0:\n                    r = p\n                u2", "                r = p\n                if r.sum() == 0.0:\n                    r = p\n                u2", "residual replaced by p"),
 ("verify", "p = softmax(zt[r0 + k], temperature)", "p = softmax(zt[r0 + k - 1], temperature)", "bonus row"),
 ("verify", "q = softmax(zd[r0 - s + a], temperature)", "q = softmax(zd[r0 + a], temperature)", "draft logit row"),
 ("verify", "ratio = p[x] / q[x] if q[x] > 0 else np.inf", "ratio = q[x] / p[x] if p[x] > 0 else np.inf", "ratio inverted"),
 ("verify", "u2 = philox.uniform(seed, sid, p0 + k, philox.STREAM_SAMPLE)", "u2 = philox.uniform(seed, sid, p0 + k - 1, philox.STREAM_SAMPLE)", "bonus uniform position"),
 ("philox", "WEYL1 = 0xBB67AE85", "WEYL1 = 0xBB67AE84", "Weyl constant"),
 ("philox", "for rnd in range(10):", "for rnd in range(9):", "round count"),
 ("philox", "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0", "c0, c1, c2, c3 = hi1 ^ c1 ^ k1, lo1, hi0 ^ c3 ^ k0, lo0", "round keys swapped"),
 ("philox", "return (w0 >> 8) * 2.0 ** -24", "return (w0 & 0xFFFFFF) * 2.0 ** -24", "uniform low bits"),
 ("philox", "w0 = philox4x32_10((pos, seq, stream, 0),", "w0 = philox4x32_10((seq, pos, stream, 0),", "counter order"),
 ("kvcache", "            p = int(seq_len[s]) + j\n", "            p = int(seq_len[s]) + j + 1\n", "append position"),
 ("kvcache", "np.asarray(accept_len, dtype=np.int64) + 1", "np.asarray(accept_len, dtype=np.int64)", "commit drops correction token"),
 ("kvcache", "v_pages[pg, :, :, off] = v_new[rs[s] + j]", "v_pages[pg, :, :, off] = v_new[rs[s] + j][:, ::-1]", "value dims reversed"),
 ("kvcache", "            if not 0 <= p < cap:\n", "            if p < 0:\n", "append past the table"),
 ("kvcache", "            if not 0 <= pg < num_pages:\n", "            if pg >= num_pages:\n", "append to an absent page"),
 ("kvcache", "range(min(rs[s + 1] - rs[s], MAX_ROWS))", "range(rs[s + 1] - rs[s])", "append row cap"),
 ("elementwise", "return h / np.sqrt(ms + eps) * w", "return h / (np.sqrt(ms) + eps) * w", "rmsnorm eps placement"),
 ("elementwise", "ms = np.mean(h * h, axis=-1, keepdims=True)", "ms = np.mean(np.abs(h), axis=-1, keepdims=True) ** 2", "rmsnorm mean of squares"),
 ("elementwise", "x2 * c + x1 * s", "x2 * c - x1 * s", "rope sign"),
 ("elementwise", "theta ** (-2.0 * i / D)", "theta ** (-1.0 * i / D)", "rope frequency"),
 ("elementwise", "k = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(R, Hkv, D)", "k = qkv[:, (Hq + Hkv) * D:].reshape(R, Hkv, D)", "k/v split"),
 ("elementwise", "return g / (1.0 + np.exp(-g)) * u", "return g / (1.0 + np.exp(g)) * u", "silu sign"),
 ("elementwise", "if 0 <= int(t) < V:", "if 0 <= int(t) <= V and int(t) < V + 1 and int(t) != 0 or int(t) == 0:", "embed id 0 / range"),
 ("model", "return np.ldexp(np.round(m * 256.0) / 256.0, e)", "return np.ldexp(np.floor(m * 256.0) / 256.0, e)", "bf16 rounding truncates"),
 ("model", "s = (Kc[:vis, g, :] @ q[i, hq]) * (float(c.D) ** -0.5)", "s = (Kc[:vis, g, :] @ q[i, hq])", "model attention scale"),
 ("verify", "(w > 0) & (c > lo_t)", "(c > lo_t)", "draw candidates admit zero weights"),
 ("verify", "lo_t, hi_t = (u - tol) * S, (u + tol) * S", "lo_t, hi_t = (u - tol) * S, u * S", "draw candidate window one-sided"),
 ("model", 'r["h2"] = g["h"] + g["o"]', 'r["h2"] = g["h_in"] + g["o"]', "per-op residual from layer input"),
 ("model", 'r["x"] = ew.rmsnorm(g["h"], lw["attn_norm"], c.eps)', 'r["x"] = ew.rmsnorm(g["h"], lw["mlp_norm"], c.eps)', "per-op attention norm weight"),
 ("model", "w = formats.dequant(np.asarray(codes)[rows], np.asarray(sm)[rows])", "w = formats.dequant(np.asarray(codes)[rows], np.asarray(sm)[::-1][rows])", "per-op row subset scales"),
]

def main():
    only = sys.argv[1:]
    dst = os.path.join(tempfile.mkdtemp(prefix="oracle_mut_"), "repo")
    os.makedirs(dst)
    skip = shutil.ignore_patterns("__pycache__", "*.so", ".pytest_cache")
    for name in ("oracle", "synth", "tests", "include", "invariant_speculative_decoding_amd"):
        shutil.copytree(os.path.join(ROOT, name), os.path.join(dst, name), ignore=skip)
    for name in ("pytest.ini", "bench.py", "__graft_entry__.py"):
        shutil.copy(os.path.join(ROOT, name), dst)
    def suite():
        # test_abi.py needs the built library, which the copy leaves out
        return subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-x", "-q",
                               "-p", "no:cacheprovider", "--ignore=tests/test_abi.py"],
                              cwd=dst, capture_output=True, text=True, timeout=900)

    base = suite()
    if base.returncode != 0:  # a mutation only counts as caught if the clean copy passes
        print(base.stdout[-2000:])
        raise SystemExit("the unmutated copy fails its CPU tests")
    survived = 0
    for i, (mod, old, new, what) in enumerate(M):
        if only and str(i) not in only:
            continue
        path = os.path.join(dst, "oracle", mod + ".py")
        src = open(path).read()
        if src.count(old) != 1:
            print(f"{i:2d} {mod:12s} {what:40s} PATTERN NOT UNIQUE", flush=True)
            survived += 1
            continue
        open(path, "w").write(src.replace(old, new))
        p = suite()
        open(path, "w").write(src)
        failed = [l.split(" ")[1] for l in p.stdout.splitlines() if l.startswith(("FAILED", "ERROR"))]
        caught = p.returncode != 0
        survived += not caught
        print(f"{i:2d} {mod:12s} {what:40s} {'caught by ' + failed[0] if failed else ('caught' if caught else 'SURVIVED')}",
              flush=True)
    shutil.rmtree(os.path.dirname(dst))
    print(f"{survived} mutation(s) survived")
    return 1 if survived else 0


if __name__ == "__main__":
    sys.exit(main())
