"""Pins for oracle/radius.py against things other than itself.

- coordination shells of a simple cubic lattice (closed form: 6 at a, 12 at a sqrt 2,
  8 at a sqrt 3, 6 at 2a), periodic and open;
- scipy's cKDTree (a library routine) on random points: equal up to pairs within
  rounding of the cutoff sphere;
- strictness at the cutoff, self pairs and coincident atoms;
- symmetry (edge set equals its transpose) and translation invariance on a lattice;
- a receiver subset equals the matching rows of the full graph;
- empty and single-atom sets.
"""
import itertools

import numpy as np
import pytest
from scipy.spatial import cKDTree

from oracle import radius


def _lattice(n, a=1.0):
    g = np.array(list(itertools.product(range(n), repeat=3)), dtype=np.float32) * np.float32(a)
    return g


@pytest.mark.parametrize("cut,coord", [(1.1, 6), (1.5, 18), (1.8, 26), (2.05, 32)])
def test_simple_cubic_shells_periodic(cut, coord):
    n = 5
    pos = _lattice(n)
    src, dst = radius.radius_graph(pos, cut, box=(n, n, n))
    deg = np.bincount(dst, minlength=n ** 3)
    assert np.all(deg == coord)
    assert src.size == coord * n ** 3


def test_simple_cubic_open_nearest_neighbours():
    n = 4
    pos = _lattice(n, a=1.5)
    src, dst = radius.radius_graph(pos, 1.6)
    # nearest-neighbour bonds of an n^3 grid: 3 n^2 (n - 1) pairs, both directions
    assert src.size == 2 * 3 * n * n * (n - 1)
    d = pos[src] - pos[dst]
    assert np.allclose(np.linalg.norm(d, axis=1), 1.5)


def _kdtree_pairs(pos, cut, box):
    tree = cKDTree(pos, boxsize=box) if box is not None else cKDTree(pos)
    pr = tree.query_pairs(cut, output_type="ndarray").astype(np.int64)
    src = np.concatenate([pr[:, 0], pr[:, 1]])
    dst = np.concatenate([pr[:, 1], pr[:, 0]])
    o = np.lexsort((src, dst))
    return src[o], dst[o]


def _dist64(pos, src, dst, box):
    d = pos[src].astype(np.float64) - pos[dst].astype(np.float64)
    if box is not None:
        L = np.asarray(box, np.float64)
        d -= L * np.round(d / L)
    return np.linalg.norm(d, axis=1)


@pytest.mark.parametrize("periodic", [False, True])
def test_matches_kdtree(periodic):
    rng = np.random.default_rng(5)
    L = 12.0
    box = (L, L, L) if periodic else None
    pos = (rng.random((300, 3)) * L).astype(np.float32)
    src, dst = radius.radius_graph(pos, 3.0, box=box)
    ks, kd = _kdtree_pairs(pos.astype(np.float64), 3.0, box)
    a = set(zip(src.tolist(), dst.tolist()))
    b = set(zip(ks.tolist(), kd.tolist()))
    assert len(a) > 1000
    diff = np.array(sorted(a ^ b), dtype=np.int64).reshape(-1, 2)
    # the two may only differ on pairs whose float64 distance is within rounding of r_c
    if diff.size:
        r = _dist64(pos, diff[:, 0], diff[:, 1], box)
        assert np.all(np.abs(r - 3.0) < 1e-5), r
    assert len(diff) <= 4


def test_strict_cutoff_self_and_coincident():
    pos = np.array([[0, 0, 0], [2, 0, 0], [0, 1.5, 0], [0, 1.5, 0]], np.float32)
    src, dst = radius.radius_graph(pos, 2.0)
    pairs = set(zip(src.tolist(), dst.tolist()))
    assert (1, 0) not in pairs and (0, 1) not in pairs          # exactly at the cutoff
    assert (2, 0) in pairs and (0, 2) in pairs and (3, 0) in pairs
    assert (2, 3) not in pairs and (3, 2) not in pairs          # coincident atoms
    assert all(s != d for s, d in pairs)


def test_canonical_order_and_symmetry():
    rng = np.random.default_rng(8)
    pos = (rng.random((200, 3)) * 9).astype(np.float32)
    src, dst = radius.radius_graph(pos, 2.5, box=(9, 9, 9))
    key = dst.astype(np.int64) * 1000 + src
    assert np.all(np.diff(key) > 0)
    fwd = set(zip(src.tolist(), dst.tolist()))
    assert fwd == set(zip(dst.tolist(), src.tolist()))


def test_translation_invariance_on_lattice():
    n = 5
    pos = _lattice(n)
    a = radius.radius_graph(pos, 1.5, box=(n, n, n))
    shifted = pos + np.array([2, -3, 7], np.float32)                 # exact in float32
    b = radius.radius_graph(shifted, 1.5, box=(n, n, n))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_receiver_subset_matches_rows():
    rng = np.random.default_rng(9)
    pos = (rng.random((150, 3)) * 8).astype(np.float32)
    src, dst = radius.radius_graph(pos, 2.2, box=(8, 8, 8))
    recv = np.array([3, 77, 140])
    s2, d2 = radius.neighbours_of(pos, recv, 2.2, box=(8, 8, 8))
    m = np.isin(dst, recv)
    assert np.array_equal(s2, src[m]) and np.array_equal(d2, dst[m])


def test_empty_and_single():
    s, d = radius.radius_graph(np.zeros((0, 3), np.float32), 1.0)
    assert s.size == 0 and d.size == 0
    s, d = radius.radius_graph(np.zeros((1, 3), np.float32), 1.0, box=(4, 4, 4))
    assert s.size == 0


def test_box_too_small_rejected():
    with pytest.raises(ValueError):
        radius.radius_graph(np.zeros((2, 3), np.float32), 3.0, box=(5, 5, 5))
