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


def sampled_compare(acc, out, acc_r, out_r, records):
    """Exclusion for rejection sampling: a decision whose uniform lies within
    1e-5 of its threshold (relative), or a draw within 1e-5 of a CDF step,
    may go the other way in fp32.  Each sequence is compared in full when it
    has no such decision, else up to the first one.  Returns the number of
    sequences with an exclusion."""
    excl = 0
    for s in range(len(acc)):
        amb = [i for i, r in enumerate(records[s]) if r[3]]
        if not amb:
            assert acc[s] == acc_r[s] and np.array_equal(out[s], out_r[s]), f"seq {s}"
        else:
            excl += 1
            upto = records[s][amb[0]][1] - 1  # tokens decided before it
            assert list(out[s, :upto]) == list(out_r[s, :upto]), f"seq {s}"
    return excl
