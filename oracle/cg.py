"""Real-basis Clebsch-Gordan coupling tensors c[m_in, m_sh, m_out].

The Sobek paper (Sec. 2 after Eq. 5; Sec. 4, Eq. 32) says only that the
Clebsch-Gordan coefficients of a path fix how angular components couple and
that c^pi carries the path normalization.  Reading fixed for this library:
c^pi is the SO(3) intertwiner V_l1 (x) V_l2 -> V_l3 in the real harmonic basis
of ``oracle.sh``: sum_ab c[a,b,m] (D1 x)_a (D2 y)_b = sum_m' D3[m,m'] f_m'(x,y).
It is unique up to scale; scale: every output column has unit norm
(sum_ab c[a,b,m]^2 = 1, i.e. ||c||_F^2 = 2 l3 + 1); sign: the first entry
(in C order over (a, b, m)) with |c| > 1e-9 is positive.  Path normalization
factor: 1.

Computed here as the null space of the stacked equivariance constraint for a
few random rotations, with Wigner-D matrices taken from the harmonics by least
squares.  This derivation shares nothing with a Racah-formula construction.

Pinned by tests/test_oracle_cg.py: sympy's complex Clebsch-Gordan moved to the
real basis, selection rules, completeness, dot/cross/identity special cases,
equivariance to 1e-12.
"""
from __future__ import annotations

import functools

import numpy as np

from .wigner import random_rotation, wigner_d


def triangle(l1: int, l2: int, l3: int) -> bool:
    return abs(l1 - l2) <= l3 <= l1 + l2


@functools.lru_cache(maxsize=None)
def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    if not triangle(l1, l2, l3):
        return np.zeros((n1, n2, n3))
    rng = np.random.default_rng(777 + 100 * l1 + 10 * l2 + l3)
    blocks = []
    for _ in range(3):
        R = random_rotation(rng)
        d1, d2, d3 = wigner_d(l1, R), wigner_d(l2, R), wigner_d(l3, R)
        # sum_ab c[a,b,m] d1[a,a'] d2[b,b'] - sum_m' d3[m,m'] c[a',b',m'] = 0 for all (a',b',m)
        t1 = np.kron(np.kron(d1.T, d2.T), np.eye(n3))
        t2 = np.kron(np.kron(np.eye(n1), np.eye(n2)), d3)
        blocks.append(t1 - t2)
    m = np.concatenate(blocks, axis=0)
    _, s, vt = np.linalg.svd(m)
    null = vt[-1]
    if s[-1] > 1e-8 or (len(s) > 1 and s[-2] < 1e-6):
        raise RuntimeError(f"unexpected null space for ({l1},{l2},{l3}): {s[-3:]}")
    c = null.reshape(n1, n2, n3)
    c = c * (np.sqrt(n3) / np.linalg.norm(c))
    flat = c.reshape(-1)
    first = flat[np.argmax(np.abs(flat) > 1e-9)]
    if first < 0:
        c = -c
    c[np.abs(c) < 1e-14] = 0.0
    return c
