"""Pins for oracle/csr.py against a brute-force construction."""
import numpy as np

from oracle.csr import csr_build, degree_order


def _brute(n, src, dst):
    rows = [[] for _ in range(n)]
    for e in range(len(src)):
        rows[dst[e]].append(e)            # COO order within a receiver
    rowptr, col, eid = [0], [], []
    for i in range(n):
        for e in rows[i]:
            col.append(src[e]); eid.append(e)
        rowptr.append(len(col))
    srows = [[] for _ in range(n)]
    for slot in range(len(col)):
        srows[col[slot]].append(slot)     # receiver-slot order within a sender
    s_rowptr, s_col, s_slot = [0], [], []
    for j in range(n):
        for slot in srows[j]:
            s_col.append(dst[eid[slot]]); s_slot.append(slot)
        s_rowptr.append(len(s_col))
    return dict(rowptr=rowptr, col=col, eid=eid, s_rowptr=s_rowptr, s_col=s_col, s_slot=s_slot)


def test_random_graphs(rng):
    for n, e in [(1, 0), (5, 0), (7, 30), (50, 400), (13, 200)]:
        src = rng.integers(0, n, e) if e else np.zeros(0, np.int64)
        dst = rng.integers(0, n, e) if e else np.zeros(0, np.int64)
        got = csr_build(n, src, dst)
        want = _brute(n, src, dst)
        for k in want:
            assert list(got[k]) == list(want[k]), k
        assert np.all(np.diff(got["rowptr"]) >= 0) and got["rowptr"][-1] == e


def test_all_into_one_and_duplicates():
    src = np.array([3, 1, 3, 3, 0, 2])
    dst = np.array([2, 2, 2, 2, 2, 2])
    got = csr_build(4, src, dst)
    want = _brute(4, src, dst)
    for k in want:
        assert list(got[k]) == list(want[k])


def test_degree_order_brute_force(rng):
    """Selection of the remaining node with the largest degree, smallest index first."""
    for n, e in [(1, 0), (6, 0), (9, 40), (40, 300), (64, 2000)]:
        src = rng.integers(0, n, e) if e else np.zeros(0, np.int64)
        dst = rng.integers(0, n, e) if e else np.zeros(0, np.int64)
        g = csr_build(n, src, dst)
        deg = [int(g["s_rowptr"][v + 1] - g["s_rowptr"][v]) for v in range(n)]
        left, want = list(range(n)), []
        while left:
            best = left[0]
            for v in left[1:]:
                if deg[v] > deg[best]:
                    best = v
            want.append(best)
            left.remove(best)
        assert list(degree_order(g["s_rowptr"])) == want
        for w in (1, 4, 7, n, n + 3):
            # each aligned window alone: the same selection restricted to its nodes
            want_w = []
            for w0 in range(0, n, w):
                left = list(range(w0, min(n, w0 + w)))
                while left:
                    best = left[0]
                    for v in left[1:]:
                        if deg[v] > deg[best]:
                            best = v
                    want_w.append(best)
                    left.remove(best)
            assert list(degree_order(g["s_rowptr"], window=w)) == want_w
    assert list(degree_order(np.array([0, 2, 4, 4, 7]))) == [3, 0, 1, 2]
    assert list(degree_order(np.array([0, 2, 4, 4, 7]), window=2)) == [0, 1, 3, 2]
