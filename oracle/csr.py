"""Receiver and sender CSR views of a COO edge list (stable).

The Sobek paper (Sec. 4, the paragraph on layouts and graphs) keeps cached
stable CSR views, receiver-major and source-major, so that every reduction has
one owner and one fixed order.  Reading fixed here:

receiver view: edges sorted by receiver, ties by original COO index;
  rowptr[N+1], col = sender of each slot, eid = COO index of each slot.
sender view: receiver-view slots sorted by sender, ties by slot;
  s_rowptr[N+1], s_col = receiver of each sender slot, s_slot = receiver slot.
degree order: the nodes by decreasing row length of a CSR view, ties by increasing
  index, over all nodes or inside aligned windows (the dispatch order of the
  traversals; no arithmetic, a stable sort of the degrees).

Pinned by tests/test_oracle_csr.py against a brute-force construction.
"""
from __future__ import annotations

import numpy as np


def csr_build(n_nodes: int, src, dst):
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    perm = np.argsort(dst, kind="stable")
    col = src[perm]
    rowptr = np.zeros(n_nodes + 1, np.int64)
    rowptr[1:] = np.cumsum(np.bincount(dst, minlength=n_nodes))
    sperm = np.argsort(col, kind="stable")
    s_col = dst[perm][sperm]
    s_rowptr = np.zeros(n_nodes + 1, np.int64)
    s_rowptr[1:] = np.cumsum(np.bincount(src, minlength=n_nodes))
    i32 = lambda a: a.astype(np.int32)  # noqa: E731
    return dict(rowptr=i32(rowptr), col=i32(col), eid=i32(perm),
                s_rowptr=i32(s_rowptr), s_col=i32(s_col), s_slot=i32(sperm))


def degree_order(rowptr, window: int = 0):
    """Nodes by decreasing rowptr[v+1] - rowptr[v], ties by increasing v; with
    window > 0, the same inside each aligned window of `window` nodes."""
    deg = np.diff(np.asarray(rowptr, np.int64))
    if window <= 0:
        return np.argsort(-deg, kind="stable").astype(np.int32)
    out = []
    for w0 in range(0, deg.size, window):
        out.append(w0 + np.argsort(-deg[w0:w0 + window], kind="stable"))
    return np.concatenate(out).astype(np.int32) if out else np.zeros(0, np.int32)
