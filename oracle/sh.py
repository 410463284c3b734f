"""Real spherical harmonics, degree l <= 3, of a unit vector r = (x, y, z).

The Sobek paper (Sec. 2, after Eq. 8) only says Y_ij holds spherical harmonics
of the edge direction with multiplicity one.  The basis fixed for this library:
real harmonics, component-normalized (sum_m Y_lm^2 = 2l+1), m = -l..l, z the
polar axis, m > 0 ~ cos(m phi) and m < 0 ~ sin(|m| phi) with positive leading
coefficients.  Degree-l harmonic has parity (-1)^l.

Written as polynomials of the unit vector (not homogeneous: only evaluated on
the sphere).  Works on torch float64 tensors so autograd can differentiate it.

Pinned by tests/test_oracle_sh.py: scipy.special.sph_harm_y, the addition
theorem, parity, harmonicity of r^l Y_l, component normalization and closed
values on the coordinate axes (tests/golden/sh_axes.json).
"""
from __future__ import annotations

import math
from typing import List

import torch

_S3 = math.sqrt(3.0)
_S5 = math.sqrt(5.0)
_S7 = math.sqrt(7.0)
_S15 = math.sqrt(15.0)
_S42 = math.sqrt(42.0)
_S70 = math.sqrt(70.0)
_S105 = math.sqrt(105.0)


def sh(l: int, u: torch.Tensor) -> torch.Tensor:
    """[..., 3] unit vectors -> [..., 2l+1]."""
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    if l == 0:
        return torch.ones_like(x)[..., None]
    if l == 1:
        return _S3 * torch.stack([y, z, x], dim=-1)
    if l == 2:
        return torch.stack([
            _S15 * x * y,
            _S15 * y * z,
            0.5 * _S5 * (3.0 * z * z - 1.0),
            _S15 * x * z,
            0.5 * _S15 * (x * x - y * y),
        ], dim=-1)
    if l == 3:
        return torch.stack([
            0.25 * _S70 * (3.0 * x * x * y - y ** 3),
            _S105 * x * y * z,
            0.25 * _S42 * y * (5.0 * z * z - 1.0),
            0.5 * _S7 * (5.0 * z ** 3 - 3.0 * z),
            0.25 * _S42 * x * (5.0 * z * z - 1.0),
            0.5 * _S105 * z * (x * x - y * y),
            0.25 * _S70 * (x ** 3 - 3.0 * x * y * y),
        ], dim=-1)
    raise ValueError("l > 3 is not supported")


def sh_all(lmax: int, u: torch.Tensor) -> List[torch.Tensor]:
    return [sh(l, u) for l in range(lmax + 1)]
