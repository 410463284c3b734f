"""Pins for the oracle's coupling tensors (oracle/cg.py) and Wigner-D (oracle/wigner.py)."""
import itertools
import math

import numpy as np
import pytest
from sympy.physics.wigner import clebsch_gordan

from oracle.cg import real_cg, triangle
from oracle.wigner import random_rotation, wigner_d

TRIPLES = [(a, b, c) for a, b, c in itertools.product(range(4), range(4), range(4)) if triangle(a, b, c)]


def _u_complex_to_real(l):
    """Rows: real index m=-l..l; cols: complex index mu=-l..l (Condon-Shortley)."""
    n = 2 * l + 1
    u = np.zeros((n, n), dtype=complex)
    s = 1 / math.sqrt(2)
    for m in range(-l, l + 1):
        if m == 0:
            u[l, l] = 1
        elif m > 0:
            u[m + l, m + l] = (-1) ** m * s
            u[m + l, -m + l] = s
        else:
            k = -m
            u[m + l, -k + l] = 1j * s
            u[m + l, k + l] = -1j * (-1) ** k * s
    return u


def _sympy_real_cg(l1, l2, l3):
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    cc = np.zeros((n1, n2, n3))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                cc[m1 + l1, m2 + l2, m3 + l3] = float(clebsch_gordan(l1, l2, l3, m1, m2, m3))
    u1, u2, u3 = _u_complex_to_real(l1), _u_complex_to_real(l2), _u_complex_to_real(l3)
    c = np.einsum("mM,abM,Aa,Bb->ABm", u3, cc, u1.conj(), u2.conj())
    if np.abs(c.real).max() >= np.abs(c.imag).max():
        part, other = c.real, c.imag
    else:
        part, other = c.imag, c.real
    assert np.abs(other).max() < 1e-12
    part = part * (math.sqrt(n3) / np.linalg.norm(part))
    flat = part.reshape(-1)
    if flat[np.argmax(np.abs(flat) > 1e-9)] < 0:
        part = -part
    return part


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_matches_sympy_in_real_basis(l1, l2, l3):
    np.testing.assert_allclose(real_cg(l1, l2, l3), _sympy_real_cg(l1, l2, l3), atol=1e-11)


@pytest.mark.parametrize("l1,l2,l3", TRIPLES)
def test_equivariance_and_column_norm(l1, l2, l3, rng):
    c = real_cg(l1, l2, l3)
    R = random_rotation(rng)
    d1, d2, d3 = wigner_d(l1, R), wigner_d(l2, R), wigner_d(l3, R)
    lhs = np.einsum("abm,aA,bB->ABm", c, d1, d2)
    rhs = np.einsum("mM,ABM->ABm", d3, c)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    np.testing.assert_allclose(np.sum(c ** 2, axis=(0, 1)), np.ones(2 * l3 + 1), atol=1e-12)


def test_selection_rule_zero():
    assert np.all(real_cg(0, 1, 2) == 0) and np.all(real_cg(3, 0, 1) == 0)


@pytest.mark.parametrize("l1,l2", [(a, b) for a in range(4) for b in range(4)])
def test_completeness(l1, l2):
    cols = [real_cg(l1, l2, l3).reshape((2 * l1 + 1) * (2 * l2 + 1), -1)
            for l3 in range(abs(l1 - l2), l1 + l2 + 1) if l3 <= 3]
    q = np.concatenate(cols, axis=1)
    np.testing.assert_allclose(q.T @ q, np.eye(q.shape[1]), atol=1e-12)
    if l1 + l2 <= 3:      # all couplings present: square orthogonal matrix
        assert q.shape[0] == q.shape[1]
        np.testing.assert_allclose(q @ q.T, np.eye(q.shape[0]), atol=1e-12)


def test_special_cases():
    for l in range(4):
        c = real_cg(l, 0, l)[:, 0, :]
        np.testing.assert_allclose(c, np.eye(2 * l + 1), atol=1e-12)       # identity
    np.testing.assert_allclose(real_cg(1, 1, 0)[:, :, 0], np.eye(3) / math.sqrt(3), atol=1e-12)  # dot
    eps = np.zeros((3, 3, 3))
    for a, b, c_ in itertools.permutations(range(3)):
        eps[a, b, c_] = np.linalg.det(np.eye(3)[[a, b, c_]])
    np.testing.assert_allclose(real_cg(1, 1, 1), eps / math.sqrt(2), atol=1e-12)                  # cross
    c112 = real_cg(1, 1, 2)
    np.testing.assert_allclose(c112, c112.transpose(1, 0, 2), atol=1e-12)                         # symmetric
    np.testing.assert_allclose(np.einsum("aam->m", c112), 0, atol=1e-12)                          # traceless


def test_wigner_d_properties(rng):
    R1, R2 = random_rotation(rng), random_rotation(rng)
    for l in range(4):
        d1, d2, d12 = wigner_d(l, R1), wigner_d(l, R2), wigner_d(l, R1 @ R2)
        np.testing.assert_allclose(d1 @ d1.T, np.eye(2 * l + 1), atol=1e-12)
        np.testing.assert_allclose(d12, d1 @ d2, atol=1e-12)
    perm = np.eye(3)[[1, 2, 0]]          # (x, y, z) -> (y, z, x)
    np.testing.assert_allclose(wigner_d(1, R1), perm @ R1 @ perm.T, atol=1e-12)
