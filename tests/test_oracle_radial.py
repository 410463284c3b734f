"""Pins for oracle/radial.py."""
import math

import numpy as np
import pytest
import torch
from scipy.integrate import quad

from oracle import radial


def test_gaussian_peaks_at_centres():
    B, lo, hi = 8, 0.0, 5.0
    mu = torch.linspace(lo, hi, B, dtype=torch.float64)
    phi = radial.gaussian(mu, B, lo, hi)
    np.testing.assert_allclose(torch.diagonal(phi).numpy(), 1.0, atol=1e-15)
    d = (hi - lo) / (B - 1)
    # neighbour value exp(-1/2) one spacing away
    np.testing.assert_allclose(phi[0, 1].item(), math.exp(-0.5), atol=1e-15)


@pytest.mark.parametrize("p", [5, 6, 7])
def test_envelope_boundary(p):
    u0 = torch.tensor(0.0, dtype=torch.float64)
    assert radial.poly_envelope(u0, p).item() == 1.0
    u = torch.tensor(1.0 - 1e-12, dtype=torch.float64, requires_grad=True)
    f = radial.poly_envelope(u, p)
    (g,) = torch.autograd.grad(f, u, create_graph=True)
    (h,) = torch.autograd.grad(g, u)
    assert abs(f.item()) < 1e-9 and abs(g.item()) < 1e-8 and abs(h.item()) < 1e-6
    assert radial.poly_envelope(torch.tensor(1.3, dtype=torch.float64), p).item() == 0.0


def test_bare_bessel_orthonormal():
    rc, B = 5.0, 6

    def bare(b, r):
        return math.sqrt(2 / rc) * math.sin(b * math.pi * r / rc) / r

    for a in range(1, B + 1):
        for b in range(1, B + 1):
            val, _ = quad(lambda r: r * r * bare(a, r) * bare(b, r), 1e-12, rc, limit=200)
            assert abs(val - (1.0 if a == b else 0.0)) < 1e-10


def test_bessel_matches_formula_with_envelope():
    rc, p = 5.0, 6
    r = torch.tensor([0.7, 2.5, 4.9, 5.2], dtype=torch.float64)
    phi = radial.bessel(r, 4, rc, p)
    assert torch.all(phi[-1] == 0)
    u = 2.5 / rc
    env = 1 - 28 * u ** 6 + 48 * u ** 7 - 21 * u ** 8      # p = 6 coefficients written out
    want = math.sqrt(2 / rc) * math.sin(3 * math.pi * 2.5 / rc) / 2.5 * env
    assert abs(phi[1, 2].item() - want) < 1e-14
