"""Pins for the oracle's real spherical harmonics (oracle/sh.py)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sp
import torch

from oracle import sh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sh_axes.json")


def _units(rng, n):
    u = rng.standard_normal((n, 3))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _y(l, u):
    return sh.sh(l, torch.from_numpy(np.asarray(u, dtype=np.float64))).numpy()


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_matches_scipy_complex_harmonics(l, rng):
    u = _units(rng, 200)
    theta = np.arccos(np.clip(u[:, 2], -1, 1))
    phi = np.arctan2(u[:, 1], u[:, 0])
    ours = _y(l, u)
    for m in range(-l, l + 1):
        c = math.sqrt(4 * math.pi) * (-1) ** abs(m) * sp.sph_harm_y(l, abs(m), theta, phi)
        if m == 0:
            ref = c.real
        elif m > 0:
            ref = math.sqrt(2) * c.real
        else:
            ref = math.sqrt(2) * c.imag
        np.testing.assert_allclose(ours[:, m + l], ref, atol=1e-12)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_addition_theorem_and_normalization(l, rng):
    a, b = _units(rng, 100), _units(rng, 100)
    lhs = np.sum(_y(l, a) * _y(l, b), axis=1)
    rhs = (2 * l + 1) * sp.eval_legendre(l, np.sum(a * b, axis=1))
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    np.testing.assert_allclose(np.sum(_y(l, a) ** 2, axis=1), 2 * l + 1, atol=1e-12)


@pytest.mark.parametrize("l", [0, 1, 2, 3])
def test_parity(l, rng):
    u = _units(rng, 50)
    np.testing.assert_allclose(_y(l, -u), (-1) ** l * _y(l, u), atol=1e-13)


@pytest.mark.parametrize("l", [1, 2, 3])
def test_solid_harmonic_is_harmonic(l, rng):
    pts = torch.from_numpy(rng.standard_normal((5, 3)))
    for p in pts:
        for m in range(2 * l + 1):
            def f(r):
                n = torch.linalg.vector_norm(r)
                return n ** l * sh.sh(l, (r / n)[None])[0, m]
            hess = torch.autograd.functional.hessian(f, p.clone())
            assert abs(torch.trace(hess).item()) < 1e-9


def test_axis_values_golden():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    axes = {"+x": [1.0, 0, 0], "+y": [0, 1.0, 0], "+z": [0, 0, 1.0]}
    for ax, vec in axes.items():
        for l in range(4):
            want = [eval(s, {"sqrt": math.sqrt}) for s in g[ax][str(l)]]
            np.testing.assert_allclose(_y(l, [vec])[0], want, atol=1e-14)
