"""Radius graph of a point set, by brute force over all pairs (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``, never by the product path.

The convolution runs on radius graphs: an edge joins two atoms closer than the
interaction cutoff r_c, so at fixed density |E| grows as |V| rho r_c^3 (Sobek paper,
Sec. 3, the paragraph on edge growth), and the wrapper prepares that graph from the
positions before calling the kernels (Sec. 4, the implementation paragraph).  The
pages fix neither the edge test nor an order, so these readings are this library's:

- both directions: for every unordered pair {i, j} within the cutoff there are the
  two edges j -> i and i -> j (a message from each side, Eq. 11);
- r_e = p_sender - p_receiver (Eq. 8) with the minimum image in an orthorhombic box
  of edge lengths L (all three > 0) or no image at all (box None);
- an edge exists iff 0 < |r_e|^2 < r_c^2: strictly inside the cutoff, and neither a
  self pair nor two coincident atoms (the edge direction would be undefined);
- the test is taken in float32, operation by operation, every product and sum
  rounded on its own (no fused multiply-add):
      d_a   = p_j,a - p_i,a
      d_a  -= L_a * rint(d_a * (1 / L_a))          (periodic; rint rounds half to even,
                                                   1 / L_a is the float32 quotient)
      |r|^2 = (d_x * d_x + d_y * d_y) + d_z * d_z,  r_c^2 = r_c * r_c
  because the test decides an integer result, both sides must take it in one precision;
- a periodic box needs every L_a >= 2 r_c, so at most one image of an atom lies
  within the cutoff;
- output order: edges sorted by receiver, then by sender (a canonical order that does
  not depend on how the pairs were found).

Pinned by tests/test_oracle_radius.py: coordination shells of a simple cubic lattice
(closed form), scipy's cKDTree on random points, strictness at the cutoff, symmetry,
translation invariance on a lattice, empty and single-atom sets.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def _f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32)


def neighbours_of(pos, receivers, cutoff: float, box: Optional[Sequence[float]] = None,
                  chunk: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """(src, dst) of every edge into the given receivers, sorted by (dst, src)."""
    p = _f32(pos).reshape(-1, 3)
    recv = np.asarray(receivers, dtype=np.int64).reshape(-1)
    c = np.float32(cutoff)
    c2 = np.float32(c * c)
    if box is not None:
        L = _f32(box).reshape(3)
        if not np.all(L > 0):
            raise ValueError("box edge lengths must all be positive")
        if np.any(L < np.float32(2) * c):
            raise ValueError("cutoff exceeds half the box: the minimum image is not unique")
        invL = np.float32(1) / L
    srcs, dsts = [], []
    for s in range(0, recv.size, chunk):
        ri = np.sort(recv[s:s + chunk])
        d = p[None, :, :] - p[ri][:, None, :]          # [R, N, 3]: sender minus receiver
        if box is not None:
            d = d - L * np.rint(d * invL)
        r2 = (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]
        assert r2.dtype == np.float32
        mask = (r2 > np.float32(0)) & (r2 < c2)
        mask[np.arange(ri.size), ri] = False
        rr, jj = np.nonzero(mask)                       # row-major: receiver, then sender
        srcs.append(jj.astype(np.int64))
        dsts.append(ri[rr])
    if not srcs:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    src = np.concatenate(srcs)
    dst = np.concatenate(dsts)
    order = np.lexsort((src, dst))
    return src[order].astype(np.int32), dst[order].astype(np.int32)


def radius_graph(pos, cutoff: float, box: Optional[Sequence[float]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Every edge of the radius graph, sorted by (receiver, sender)."""
    n = _f32(pos).reshape(-1, 3).shape[0]
    return neighbours_of(pos, np.arange(n), cutoff, box)
