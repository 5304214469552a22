"""Philox4x32-10 counter-based generator (oracle side; test infrastructure only).

Written from its published definition: J. Salmon, M. Moraes, R. Dror, D. Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11, section 4 (Philox-4x32
with 10 rounds). One round maps the counter (c0, c1, c2, c3) with key (k0, k1):
    (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2       (32x32 -> 64-bit products)
    c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
and the key is bumped by the Weyl constants between rounds.

Stream layout used by the acceptance walk: key = (seed_lo, seed_hi), counter =
(trial_lo, round, step, trial_hi); one call per uniform, u = (out0 >> 8) * 2**-24.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Scalar reference: ctr 4 ints, key 2 ints -> 4 ints."""
    c0, c1, c2, c3 = (int(x) & MASK for x in ctr)
    k0, k1 = (int(x) & MASK for x in key)
    for r in range(10):
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK, lo1, (hi0 ^ c3 ^ k1) & MASK, lo0
        if r < 9:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
    return c0, c1, c2, c3


def philox_batch(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised over uint64 arrays of counter words (values < 2**32)."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK
    c1 = np.asarray(c1, dtype=np.uint64) & MASK
    c2 = np.asarray(c2, dtype=np.uint64) & MASK
    c3 = np.asarray(c3, dtype=np.uint64) & MASK
    k0 = np.uint64(k0 & MASK)
    k1 = np.uint64(k1 & MASK)
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    mask = np.uint64(MASK)
    for r in range(10):
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & mask, lo1, (hi0 ^ c3 ^ k1) & mask, lo0
        if r < 9:
            k0 = (k0 + np.uint64(W0)) & mask
            k1 = (k1 + np.uint64(W1)) & mask
    return c0, c1, c2, c3


def uniform(seed: int, trial: int, rnd: int, step: int) -> float:
    """The walk's uniform in [0, 1) for (trial, round, step)."""
    out = philox4x32_10((trial & MASK, rnd, step, (trial >> 32) & MASK), (seed & MASK, (seed >> 32) & MASK))
    return (out[0] >> 8) * (2.0 ** -24)
