"""Helpers for the GPU tests: moving seeded numpy inputs to the device,
comparing against the oracle at the stated tolerance, and memcmp."""
from __future__ import annotations

import numpy as np
import pytest

TOL = 2e-3  # max-abs error <= TOL * max|ref| for floating-point outputs


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch


def isd():
    """The HIP library binding; fails (never falls back) when unavailable."""
    import invariant_speculative_decoding_amd as m
    m.lib()
    return m


def dev(a):
    """numpy -> contiguous GPU tensor (uint16 travels as int16 bits)."""
    torch = torch_dev()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def assert_close(got, ref, tol=TOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} * max|ref| {scale:.3e}"
    return err / scale if scale else 0.0


def half_ulp(x, fmt):
    """Half a unit in the last place of the 16-bit format (bf16: 8
    significant bits, no subnormals below 2^-126; fp16: 11 significant bits,
    subnormal spacing 2^-24) at the magnitude of each value of x."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    mant, emin = (8, -126) if fmt == "bf16" else (11, -14)
    e = np.floor(np.log2(np.where(x > 0, x, 2.0 ** emin)))
    e = np.maximum(e, emin)
    return np.ldexp(0.5, (e - (mant - 1)).astype(np.int64))


def assert_rounded(got, exact, fmt, slack=4e-6, what=""):
    """A 16-bit GPU output must be the exact value correctly rounded, up to
    the GPU's fp32 error before the rounding: |got - exact| <= half an ulp
    of got + slack * |exact| (the slack lets a value within fp32 error of a
    half-way point round either way).  Returns the largest error in half
    ulps."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    assert got.shape == exact.shape, (got.shape, exact.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = np.abs(got - exact)
    lim = half_ulp(got, fmt) + slack * np.abs(exact)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} values not correctly rounded, e.g. "
                           f"got {got[bad][0]!r} exact {exact[bad][0]!r}")
    return float((err / half_ulp(got, fmt)).max())


def same_bits(a, b) -> bool:
    """memcmp of two arrays (any dtype)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.tobytes() == b.tobytes()


def greedy_compare(acc, out, acc_r, out_r, margins, rs, tie=1e-3):
    """Near-tie exclusion for greedy verify: a row whose oracle top-2 margin
    is below ``tie`` may flip under fp32 rounding.  Emitted tokens are
    compared up to the first near-tie row among rows 0..a_oracle; accept
    lengths only when no near-tie row lies in rows 0..min(a_gpu, a_oracle).
    Returns the number of sequences with an exclusion."""
    excluded = 0
    for s in range(len(acc)):
        r0 = int(rs[s])
        near = [j for j in range(int(acc_r[s]) + 1) if margins[r0 + j] < tie]
        if near:
            excluded += 1
            j0 = near[0]
            assert list(out[s, :j0]) == list(out_r[s, :j0]), f"seq {s}"
            lim = min(int(acc[s]), int(acc_r[s]))
            if not any(margins[r0 + j] < tie for j in range(lim + 1)):
                assert acc[s] == acc_r[s]
        else:
            assert acc[s] == acc_r[s], f"seq {s}: {acc[s]} vs {acc_r[s]}"
            assert np.array_equal(out[s], out_r[s]), f"seq {s}"
    return excluded


def sampled_compare(acc, out, acc_r, out_r, records, counts=None):
    """Comparison of rejection sampling with the oracle.

    An accept test whose uniform lies within 1e-5 (relative) of its
    threshold may go the other way in fp32: such a sequence is compared up
    to that decision only and counted as an exclusion.  A draw (residual or
    bonus) whose threshold lies within 1e-5 S of a cumulative step is still
    checked: the accept length and every earlier token exactly, and the
    drawn token must be one of the oracle's candidates for thresholds within
    that window (``oracle.verify.draw_candidates``); `counts["near_draws"]`
    counts them.  Every other sequence is compared exactly.  Returns the
    number of exclusions."""
    excl = 0
    for s in range(len(acc)):
        amb = [i for i, r in enumerate(records[s]) if r[3]]
        if not amb:
            assert acc[s] == acc_r[s] and np.array_equal(out[s], out_r[s]), f"seq {s}"
            continue
        kind, j = records[s][amb[0]][0], records[s][amb[0]][1]
        if kind == "accept":
            excl += 1
            assert list(out[s, :j - 1]) == list(out_r[s, :j - 1]), f"seq {s}"
        else:
            # a draw ends the sequence's decisions: it is the last record
            assert amb[0] == len(records[s]) - 1
            assert acc[s] == acc_r[s], f"seq {s}: {acc[s]} vs {acc_r[s]}"
            assert list(out[s, :j - 1]) == list(out_r[s, :j - 1]), f"seq {s}"
            cand = records[s][amb[0]][4]
            assert int(out[s, j - 1]) in cand, f"seq {s}: {out[s, j - 1]} not in {cand}"
            assert (out[s, j:] == -1).all(), f"seq {s}"
            if counts is not None:
                counts["near_draws"] = counts.get("near_draws", 0) + 1
    return excl
