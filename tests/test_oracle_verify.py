"""Pins for the oracle's argmax, greedy accept, Philox and rejection-
sampling rule (CPU only)."""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import philox, verify

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ greedy

def test_greedy_hand_example():
    g = _gold("greedy_hand_example.json")
    z = np.array(g["logits"], dtype=np.float32)
    t = [verify.argmax_lowest(r) for r in z]
    assert t == g["targets"]
    for c in g["cases"]:
        a, em = verify.greedy_accept(t, c["drafts"])
        assert a == c["accept_len"] and em == c["emitted"]
        rs = np.array([0, 4])
        acc, out, _, _ = verify.verify_greedy(z, np.array(c["drafts"]), rs)
        assert acc[0] == c["accept_len"]
        assert list(out[0, :len(em)]) == em and (out[0, len(em):] == -1).all()


def test_argmax_is_numpy_first_occurrence():
    g = synth.rng(0)
    for _ in range(200):
        z = g.integers(-3, 4, size=g.integers(1, 50)).astype(np.float32)
        assert verify.argmax_lowest(z) == int(np.argmax(z))


def test_argmax_nan_never_wins_and_signed_zero_ties():
    assert verify.argmax_lowest([np.nan, 1.0, 0.5]) == 1
    assert verify.argmax_lowest([-0.0, 0.0, -1.0]) == 0
    assert verify.argmax_lowest([0.0, -0.0]) == 0


def test_greedy_generator_gives_exact_accept_lengths():
    g = synth.rng(1)
    V, k = 50, 4
    for _ in range(300):
        t = g.integers(0, V, size=k + 1)
        d, a = synth.greedy_drafts(t, k, g, V, agree=synth.uniform_agree(0, k))
        got, em = verify.greedy_accept(t, d)
        assert got == a and em[-1] == t[a]


@pytest.mark.parametrize("k,expect", [(4, 2.7731), (7, 3.1412)])
def test_geometric_agree_closed_form(k, expect):
    """E[a+1] = (1 - 0.7^(k+1)) / 0.3 for truncated geometric agreement."""
    assert abs((1 - 0.7 ** (k + 1)) / 0.3 - expect) < 1e-4
    g = synth.rng(2)
    draw = synth.geometric_agree(0.7, k)
    a = np.array([draw(g) for _ in range(200000)])
    assert abs((a + 1).mean() - expect) < 0.02


# ------------------------------------------------------------------ philox

def test_philox_known_answers():
    for c in _gold("philox_kat.json")["cases"]:
        ctr = [int(v, 16) for v in c["counter"]]
        key = [int(v, 16) for v in c["key"]]
        assert list(philox.philox4x32_10(ctr, key)) == [int(v, 16) for v in c["out"]]


def _torch_include():
    try:
        import torch
        inc = os.path.join(os.path.dirname(torch.__file__), "include")
    except Exception:
        return None
    hdr = os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")
    return inc if os.path.exists(hdr) else None


@pytest.mark.skipif(shutil.which("g++") is None or _torch_include() is None,
                    reason="needs g++ and torch's C++ headers")
def test_philox_matches_independent_implementation(tmp_path):
    """torch ships its own host-compilable Philox4x32-10; its key is the
    seed and its counter is (offset lo, offset hi, subsequence lo, hi)."""
    src = tmp_path / "ph.cpp"
    src.write_text(
        "#include <ATen/core/PhiloxRNGEngine.h>\n#include <cstdio>\n#include <cstdlib>\n"
        "int main(int c, char** v){ for(int i=1;i+3<c+1;i+=3){"
        " at::philox_engine e(strtoull(v[i],0,0), strtoull(v[i+1],0,0), strtoull(v[i+2],0,0));"
        " unsigned a=e(); unsigned b=e(); unsigned d=e(); unsigned f=e();"
        " printf(\"%u %u %u %u\\n\", a, b, d, f);} }\n")
    exe = tmp_path / "ph"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", _torch_include(), str(src), "-o", str(exe)],
                   check=True)
    g = synth.rng(3)
    cases = []
    for _ in range(64):
        seed = int(g.integers(0, 2 ** 63)) * 2 + int(g.integers(0, 2))
        pos, seq, stream = int(g.integers(0, 2 ** 32)), int(g.integers(0, 2 ** 32)), int(g.integers(0, 4))
        cases.append((seed, pos, seq, stream))
    args = []
    for seed, pos, seq, stream in cases:
        args += [str(seed), str(stream), str(pos | (seq << 32))]
    out = subprocess.run([str(exe)] + args, check=True, capture_output=True, text=True).stdout
    for (seed, pos, seq, stream), line in zip(cases, out.strip().split("\n")):
        want = [int(v) for v in line.split()]
        got = philox.philox4x32_10((pos, seq, stream, 0), (seed & 0xFFFFFFFF, seed >> 32))
        assert list(got) == want
        assert philox.uniform(seed, seq, pos, stream) == (want[0] >> 8) * 2.0 ** -24


def test_philox_uniformity_and_stream_independence():
    n = 40000
    u0 = np.array([philox.uniform(4, 3, p, 0) for p in range(n)])
    u1 = np.array([philox.uniform(4, 3, p, 1) for p in range(n)])
    for u in (u0, u1):
        assert u.min() >= 0 and u.max() < 1
        h, _ = np.histogram(u, bins=20, range=(0, 1))
        assert stats.chisquare(h).pvalue > 1e-3
    assert abs(np.corrcoef(u0, u1)[0, 1]) < 0.03


# ------------------------------------------------------------------ sampling

def test_sampled_hand_example():
    g = _gold("sampled_hand_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    for c in g["cases"]:
        tok, acc = verify.accept_or_resample(p, q, np.array([c["x"]]), np.array([c["u"]]),
                                             np.array([c["u2"]]))
        assert int(tok[0]) == c["token"] and bool(acc[0]) == c["accepted"]
    assert abs(np.minimum(p, q).sum() - g["accept_probability"]) < 1e-15


def test_monte_carlo_reproduces_target_distribution():
    """x ~ q, then the rule: emitted tokens follow p (16-token vocabulary,
    10^6 trials), and the acceptance rate is sum min(p, q)."""
    g = synth.rng(16)
    V, T = 16, 10 ** 6
    p = g.dirichlet(np.ones(V) * 0.7)
    q = g.dirichlet(np.ones(V) * 0.7)
    x = g.choice(V, size=T, p=q)
    tok, acc = verify.accept_or_resample(p, q, x, g.random(T), g.random(T))
    f = np.bincount(tok, minlength=V)
    assert stats.chisquare(f, p * T).pvalue > 1e-3
    sigma = np.sqrt(p * (1 - p) / T)
    assert (np.abs(f / T - p) < 5 * sigma + 1e-12).all()
    ra = np.minimum(p, q).sum()
    assert abs(acc.mean() - ra) < 5 * np.sqrt(ra * (1 - ra) / T)


def test_equal_distributions_always_accept():
    g = synth.rng(17)
    p = g.dirichlet(np.ones(10))
    x = g.choice(10, size=5000, p=p)
    _, acc = verify.accept_or_resample(p, p, x, g.random(5000), g.random(5000))
    assert acc.all()


def test_draft_outside_target_support_always_rejects():
    g = synth.rng(18)
    p = np.array([0.4, 0.6, 0.0, 0.0])
    q = np.array([0.0, 0.0, 1.0, 0.0])
    tok, acc = verify.accept_or_resample(p, q, np.full(20000, 2), g.random(20000), g.random(20000))
    assert not acc.any()
    f = np.bincount(tok, minlength=4) / 20000
    assert abs(f[0] - 0.4) < 0.02 and f[2] == 0 and f[3] == 0


def test_sampled_draft_ids_outside_the_vocabulary_are_never_accepted():
    """A draft id outside [0, V) decides exactly as an in-range token to
    which the target gives probability 0 (a logit of -inf): rejected at its
    position, and the token drawn there from the same residual."""
    g = synth.rng(23)
    B, k, V, T, seed = 4, 3, 30, 0.8, 99
    zt = (g.standard_normal((B * (k + 1), V)) * 3).astype(np.float64)
    zd = (g.standard_normal((B * k, V)) * 3).astype(np.float64)
    rs = np.arange(B + 1) * (k + 1)
    seq_id, pos0 = np.array([1, 2, 3, 4]), np.array([10, 20, 30, 40])
    x0 = 7
    drafts = g.integers(0, V, size=B * k)
    drafts[drafts == x0] = x0 + 1
    bad = drafts.copy()
    for s, j, v in ((0, 0, -1), (1, 1, V), (2, 2, V + 1000), (3, 0, -(1 << 31))):
        zt[s * (k + 1) + j, x0] = -np.inf
        drafts[s * k + j] = x0
        bad[s * k + j] = v
    acc, out, rec = verify.verify_sampled(zt, zd, drafts, rs, seq_id, pos0, T, seed)
    acc_b, out_b, rec_b = verify.verify_sampled(zt, zd, bad, rs, seq_id, pos0, T, seed)
    assert np.array_equal(acc, acc_b) and np.array_equal(out, out_b)
    assert (acc <= np.array([0, 1, 2, 0])).all()  # rejected at the planted position at the latest


def test_verify_sampled_matches_stepwise_rule():
    """The batched sequential verify equals stepping accept_or_resample by
    hand with the Philox uniforms of each (sequence, position, stream)."""
    g = synth.rng(19)
    B, k, V, T, seed = 3, 4, 40, 0.8, 1234
    zt = (g.standard_normal((B * (k + 1), V)) * 3).astype(np.float32)
    zd = (zt.reshape(B, k + 1, V)[:, :k].reshape(B * k, V)
          + g.standard_normal((B * k, V)) * 0.5).astype(np.float32)
    drafts = synth.gumbel_draws(zd, T, g)
    rs = np.arange(B + 1) * (k + 1)
    seq_id = np.array([7, 0, 3])
    pos0 = np.array([100, 5, 77])
    acc, out, _ = verify.verify_sampled(zt, zd, drafts, rs, seq_id, pos0, T, seed)
    for s in range(B):
        em = []
        for j in range(1, k + 1):
            p = verify.softmax(zt[s * (k + 1) + j - 1], T)
            qd = verify.softmax(zd[s * k + j - 1], T)
            u = philox.uniform(seed, int(seq_id[s]), int(pos0[s]) + j - 1, 0)
            u2 = philox.uniform(seed, int(seq_id[s]), int(pos0[s]) + j - 1, 1)
            tok, ok = verify.accept_or_resample(p, qd, np.array([drafts[s * k + j - 1]]),
                                                np.array([u]), np.array([u2]))
            em.append(int(tok[0]))
            if not ok[0]:
                break
        else:
            p = verify.softmax(zt[s * (k + 1) + k], T)
            u2 = philox.uniform(seed, int(seq_id[s]), int(pos0[s]) + k, 1)
            em.append(verify.inverse_cdf(p, u2)[0])
        assert acc[s] == len(em) - 1
        assert list(out[s, :len(em)]) == em


# ---------------------------------------------------------- margin re-check

def test_recheck_rows_hand_example():
    """Two sequences: rows 0..2 (k = 2) and rows 3..6 (k = 3).  Margins
    chosen by hand; the re-check looks only at rows 0..a of each sequence."""
    margins = np.array([0.5, 2e-4, 3.0,      # seq 0
                        1.0, 0.8, 5e-4, 0.0])  # seq 1
    rs = [0, 3, 7]
    # seq 0 accepts 2 -> rows 0..2 checked, row 1 is the first below 1e-3;
    # seq 1 accepts 1 -> rows 0..1 checked, none below 1e-3
    assert list(verify.recheck_rows(margins, rs, [2, 1], 1e-3)) == [1, -1]
    # seq 0 accepts 0 -> only row 0; seq 1 accepts 3 -> row 2 (5e-4) first
    assert list(verify.recheck_rows(margins, rs, [0, 3], 1e-3)) == [-1, 2]
    # an exact tie (margin 0) is below any positive threshold
    assert list(verify.recheck_rows(margins, rs, [0, 3], 1e-9)) == [-1, 3]
    # threshold 0 flags nothing
    assert list(verify.recheck_rows(margins, rs, [2, 3], 0.0)) == [-1, -1]


def test_top2_margin_matches_brute_force():
    g = np.random.default_rng(11)
    for V in (2, 3, 17, 1000):
        z = g.standard_normal(V).astype(np.float32)
        z[g.integers(0, V)] = z.max()  # sometimes an exact tie
        best = max(z)
        rest = list(z)
        rest.remove(best)
        assert verify.top2_margin(z) == float(best) - float(max(rest))


def test_greedy_ragged_batch_hand_example():
    """Two sequences in one call (k = 2 and k = 1): drafts are packed
    sequence after sequence, k_s per sequence, while target rows are k_s + 1
    per sequence.  Argmaxes by construction: rows 0..2 -> 1, 2, 3 (sequence
    0), rows 3..4 -> 0, 3 (sequence 1)."""
    V = 4
    z = np.zeros((5, V), dtype=np.float32)
    for r, t in enumerate([1, 2, 3, 0, 3]):
        z[r, t] = 1.0
    rs = np.array([0, 3, 5])
    drafts = np.array([1, 0, 0])  # sequence 0: [1, 0]; sequence 1: [0]
    acc, out, t_all, _ = verify.verify_greedy(z, drafts, rs)
    assert list(t_all) == [1, 2, 3, 0, 3]
    # sequence 0 accepts draft 1 (= target 1), rejects 0 (target 2): emits 1, 2
    # sequence 1 accepts draft 0 (= target 0) and takes the bonus target 3
    assert list(acc) == [1, 1]
    assert list(out[0, :2]) == [1, 2] and (out[0, 2:] == -1).all()
    assert list(out[1, :2]) == [0, 3] and (out[1, 2:] == -1).all()


def test_softmax_temperature_closed_form():
    """softmax(z / T): z = (0, ln 3) at T = 1/2 gives weights 1 : 9; at
    T = 2 it gives 1 : sqrt(3)."""
    z = np.array([0.0, math.log(3.0)])
    np.testing.assert_allclose(verify.softmax(z, 0.5), [0.1, 0.9], rtol=1e-14)
    r3 = math.sqrt(3.0)
    np.testing.assert_allclose(verify.softmax(z, 2.0), [1 / (1 + r3), r3 / (1 + r3)], rtol=1e-14)


def test_inverse_cdf_step_boundary():
    """The draw is the smallest v whose cumulative weight exceeds u * S
    strictly: with four equal weights, u = k/4 lands exactly on a step and
    selects entry k."""
    w = np.ones(4)
    for k in range(4):
        v, gap = verify.inverse_cdf(w, k / 4)
        assert v == k and gap == 0.0
    v, _ = verify.inverse_cdf(w, 0.3)
    assert v == 1
    # zero-weight entries are never drawn, even at their step
    v, _ = verify.inverse_cdf(np.array([0.0, 2.0, 0.0, 2.0]), 0.5)
    assert v == 3


def test_draw_candidates_window():
    """The candidates of a draw are the entries a threshold within tol * S
    selects: one entry away from any step, both neighbours at a step, zero
    weights never, and the last positive entry when the window reaches S."""
    w = np.ones(4)
    assert verify.draw_candidates(w, 0.3, 1e-5) == (1,)
    assert verify.draw_candidates(w, 0.5, 1e-5) == (1, 2)
    assert verify.draw_candidates(w, 0.5 + 2e-5, 1e-5) == (2,)
    assert verify.draw_candidates(w, 0.5 - 2e-5, 1e-5) == (1,)
    # inside the window on either side of a step: both neighbours
    assert verify.draw_candidates(w, 0.5 - 5e-6, 1e-5) == (1, 2)
    assert verify.draw_candidates(w, 0.5 + 5e-6, 1e-5) == (1, 2)
    assert verify.draw_candidates(w, 0.0, 1e-5) == (0,)
    # zero weights between positive ones are skipped at the shared step
    z = np.array([1.0, 0.0, 0.0, 1.0])
    assert verify.draw_candidates(z, 0.5, 1e-3) == (0, 3)
    # a threshold near S reaches the last positive entry only
    assert verify.draw_candidates(np.array([1.0, 1.0, 0.0]), 1.0 - 1e-7, 1e-5) == (1,)
    # the drawn entry itself is always a candidate
    g = np.random.default_rng(3)
    for _ in range(200):
        p = g.random(50) * (g.random(50) < 0.7)
        if p.sum() == 0:
            continue
        u = float(g.random())
        v, _ = verify.inverse_cdf(p, u)
        assert v in verify.draw_candidates(p, u, 1e-5)
