"""Radial bases phi_b(r) (the invariant edge embedding phi of the Sobek paper,
Sec. 2 after Eq. 8, width K; B here).

The paper fixes no radial family.  The two used by the workloads:

Gaussian: centres mu_b = r_lo + b*D, D = (r_hi - r_lo)/(B-1), b = 0..B-1,
  phi_b(r) = exp(-(r - mu_b)^2 / (2 D^2)); no envelope.
Bessel with polynomial envelope (the form of Klicpera et al., DimeNet, 2020):
  phi_b(r) = sqrt(2/r_c) sin(b pi r / r_c) / r * f_p(r / r_c), b = 1..B,
  f_p(u) = 1 - (p+1)(p+2)/2 u^p + p(p+2) u^(p+1) - p(p+1)/2 u^(p+2) for u < 1,
  and 0 for u >= 1.

Pinned by tests/test_oracle_radial.py: phi_b(mu_b) = 1, envelope boundary
values/derivatives, orthonormality of the bare Bessel functions with weight r^2.
"""
from __future__ import annotations

import math

import torch


def gaussian(r: torch.Tensor, n_basis: int, r_lo: float, r_hi: float) -> torch.Tensor:
    if n_basis < 2:
        raise ValueError("Gaussian basis needs at least two centres")
    d = (r_hi - r_lo) / (n_basis - 1)
    mu = r_lo + d * torch.arange(n_basis, dtype=r.dtype)
    return torch.exp(-((r[..., None] - mu) ** 2) / (2.0 * d * d))


def poly_envelope(u: torch.Tensor, p: int) -> torch.Tensor:
    f = (1.0 - 0.5 * (p + 1) * (p + 2) * u ** p + p * (p + 2) * u ** (p + 1)
         - 0.5 * p * (p + 1) * u ** (p + 2))
    return torch.where(u < 1.0, f, torch.zeros_like(f))


def bessel(r: torch.Tensor, n_basis: int, r_cut: float, p: int) -> torch.Tensor:
    b = torch.arange(1, n_basis + 1, dtype=r.dtype)
    bare = math.sqrt(2.0 / r_cut) * torch.sin(b * math.pi * r[..., None] / r_cut) / r[..., None]
    return bare * poly_envelope(r / r_cut, p)[..., None]


def radial(kind: str, r: torch.Tensor, n_basis: int, r_lo: float, r_hi: float, p: int) -> torch.Tensor:
    if kind == "gaussian":
        return gaussian(r, n_basis, r_lo, r_hi)
    if kind == "bessel":
        return bessel(r, n_basis, r_hi, p)
    raise ValueError(kind)
