"""Inputs on which an offset-code dot product loses the error bound.

Every weight sits at its format's zero code except one unit step per block (the
same position in every block of a row), and x is 1 everywhere except a small value
eps at those positions.  Then y = nb * d * (+-1) * eps and S = sum |w x| = nb * |d| *
eps are tiny, while sum |x| over the zero weights is nb * 31: a kernel that carries
an offset on every code (or factors a block bias out of its sum) rounds sums of
size ~ sum |x| and misses the bound by orders of magnitude.  Zero codes: Q8_0 q = 0,
Q4_0 n = 8, Q5_0 u = 16; Q4_1 n = 8 and Q5_1 u = 16 with the bias m = -n d (so
that d u + m = 0).  The bytes come from the oracle's packers; the layouts follow
"EdgeRunner Core Architecture", sections 1.3 and 3.1 (reading R19 for the fields
of Q4_1 / Q5_0 / Q5_1).
"""
from __future__ import annotations

import numpy as np

import oracle

ZERO = {oracle.FMT_Q8_0: 0, oracle.FMT_Q4_0: 8, oracle.FMT_Q5_0: 16, oracle.FMT_Q4_1: 8, oracle.FMT_Q5_1: 16}
# Positions of the one nonzero weight per block: both nibble halves, the ends of a
# block, and both sides of the 16-weight boundary.
POSITIONS = (5, 21, 0, 31, 16, 15)
EPS = (1e-1, 1e-2, 1e-3, 1e-4)


def codes(fmt: int, M: int, K: int):
    """(codes [M][K], d16 [M][K/32], m16 [M][K/32] or None): row r has code
    ZERO + s_r, s_r = +1 for even r and -1 for odd r, at POSITIONS[r % 6] of every
    block, and the zero code elsewhere; d = 2^-7."""
    nb = K // 32
    c = np.full((M, K), ZERO[fmt], dtype=np.int64)
    for r in range(M):
        p = POSITIONS[r % len(POSITIONS)]
        c[r, p::32] += 1 if r % 2 == 0 else -1
    d16 = np.full((M, nb), 2.0 ** -7, dtype=np.float16)
    m16 = None
    if fmt in (oracle.FMT_Q4_1, oracle.FMT_Q5_1):
        m16 = (-ZERO[fmt] * d16.astype(np.float64)).astype(np.float16)
    return c, d16, m16


def weights(fmt: int, M: int, K: int) -> np.ndarray:
    """Raw block bytes of codes(fmt, M, K)."""
    c, d16, m16 = codes(fmt, M, K)
    if fmt == oracle.FMT_Q8_0:
        return oracle.pack_q8_0(c, d16)
    if fmt == oracle.FMT_Q4_0:
        return oracle.pack_q4_0(c, d16)
    if fmt == oracle.FMT_Q4_1:
        return oracle.pack_q4_1(c, d16, m16)
    if fmt == oracle.FMT_Q5_0:
        return oracle.pack_q5_0(c, d16)
    return oracle.pack_q5_1(c, d16, m16)


def activations(N: int, K: int) -> np.ndarray:
    """x [N][K] fp32: 1 everywhere, EPS[n % 4] at every position in POSITIONS."""
    x = np.ones((N, K), dtype=np.float32)
    for n in range(N):
        for p in POSITIONS:
            x[n, p::32] = EPS[n % len(EPS)]
    return x
