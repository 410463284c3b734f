"""Real-basis Wigner-D matrices, obtained from the harmonics themselves.

D^l(R) is the unique matrix with Y_l(R u) = D^l(R) Y_l(u) for all unit u; it is
found by least squares over random directions.  An improper element Q = -R acts
on an irrep block of parity s as s * D^l(R) (and on the harmonics themselves as
(-1)^l D^l(R)).  Used for the CG null space and for equivariance tests (the
transformation law of the Sobek paper, Eq. 1-2).

Pinned by tests/test_oracle_cg.py: orthogonality, the homomorphism property,
and D^1(R) = R in (y, z, x) order.
"""
from __future__ import annotations

import numpy as np
import torch

from . import sh as _sh


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def wigner_d(l: int, R: np.ndarray, n_dirs: int = 64, seed: int = 12345) -> np.ndarray:
    rng = np.random.default_rng(seed + l)
    u = rng.standard_normal((n_dirs, 3))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    a = _sh.sh(l, torch.from_numpy(u)).numpy()               # [K, n]
    b = _sh.sh(l, torch.from_numpy(u @ R.T)).numpy()         # Y(R u) rows
    dt, *_ = np.linalg.lstsq(a, b, rcond=None)               # b = a D^T
    return dt.T
