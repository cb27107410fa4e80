"""Philox4x32-10 (oracle; test infrastructure).

The counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11): a 128-bit counter is mixed with
a 64-bit key by ten rounds, each multiplying two counter words by fixed
constants and exchanging the halves of the products with the other words
and the key; the key is advanced by two Weyl constants between rounds.

The accept rule needs one uniform per decision, keyed so that a decision's
random number depends only on (seed, sequence, position, purpose) and never
on how sequences are batched (proofoftech.org, "'Lossless' speculative
decoding is a property of the math, not your deployment.", section
"Distribution-preserving is not bitwise-reproducible": reproducible output
must be engineered, not assumed).  The key is (seed low word, seed high
word); the counter is (position, sequence id, stream, 0) with stream 0 for
the accept test and stream 1 for the residual or bonus sample; the uniform
is ``(w0 >> 8) * 2**-24`` from the first output word.
"""
from __future__ import annotations

MASK = 0xFFFFFFFF
MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85

STREAM_ACCEPT = 0
STREAM_SAMPLE = 1


def philox4x32_10(counter, key):
    """Four 32-bit output words for a 4-word counter and 2-word key."""
    c0, c1, c2, c3 = (int(v) & MASK for v in counter)
    k0, k1 = (int(v) & MASK for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + WEYL0) & MASK
            k1 = (k1 + WEYL1) & MASK
        p0 = MUL0 * c0
        p1 = MUL1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform(seed: int, seq: int, pos: int, stream: int) -> float:
    """u in [0, 1) with 24 random bits, as an exact fp64 value."""
    w0 = philox4x32_10((pos, seq, stream, 0), (seed & MASK, (seed >> 32) & MASK))[0]
    return (w0 >> 8) * 2.0 ** -24
