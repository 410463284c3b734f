"""Feature layouts at the boundary: mul_ir <-> ir_mul (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``__graft_entry__.smoke()``, never
by the product path.

A feature row is a direct sum of irrep blocks (Sobek paper, Sec. 2, Eq. 3-4); block k
has C channels of 2l+1 components.  The kernels use the ir_mul order, in which the
channels of one component m are adjacent (the block is a [2l+1][C] array); the common
default elsewhere is mul_ir, where the 2l+1 components of one channel are adjacent
(a [C][2l+1] array), and the wrapper converts between the two at the boundary (Sec. 4,
the implementation paragraph).  Converting is a transpose of every block; blocks follow
each other in irreps order in both layouts, with the same offsets.

Pinned by tests/test_oracle_layout.py (a hand-indexed example, identity on scalar and
single-channel blocks, round trips).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

Irrep = Tuple[int, int, int]


def _blocks(irreps: Sequence[Irrep]):
    off = 0
    for mul, l, _ in irreps:
        d = 2 * l + 1
        yield off, mul, d
        off += mul * d


def _check(x: np.ndarray, irreps: Sequence[Irrep]) -> np.ndarray:
    x = np.asarray(x)
    width = sum(mul * (2 * l + 1) for mul, l, _ in irreps)
    if x.ndim != 2 or x.shape[1] != width:
        raise ValueError(f"feature rows must be [N][{width}], got {x.shape}")
    return x


def mul_ir_to_ir_mul(x, irreps: Sequence[Irrep]) -> np.ndarray:
    """Rows in mul_ir order -> rows in ir_mul order."""
    x = _check(x, irreps)
    out = np.empty_like(x)
    n = x.shape[0]
    for off, mul, d in _blocks(irreps):
        blk = x[:, off:off + mul * d].reshape(n, mul, d)        # [N][C][2l+1]
        out[:, off:off + mul * d] = blk.transpose(0, 2, 1).reshape(n, mul * d)
    return out


def ir_mul_to_mul_ir(x, irreps: Sequence[Irrep]) -> np.ndarray:
    """Rows in ir_mul order -> rows in mul_ir order."""
    x = _check(x, irreps)
    out = np.empty_like(x)
    n = x.shape[0]
    for off, mul, d in _blocks(irreps):
        blk = x[:, off:off + mul * d].reshape(n, d, mul)        # [N][2l+1][C]
        out[:, off:off + mul * d] = blk.transpose(0, 2, 1).reshape(n, mul * d)
    return out
