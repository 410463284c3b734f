"""Host-side checks of bench.py helpers (no GPU): the Morton relabelling used by
--node-order keeps the graph and every per-node value, only the numbering changes; the
bench refuses more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import make_workload, small_variant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_morton_relabel_is_a_renumbering():
    cfg = small_variant("cfg2", 300)
    wl = make_workload(cfg, w_blocks=[(16, 1.0)], z_dim=8, scalar_out_mask=None)
    rw = bench.morton_relabel(wl)
    n = wl.n_nodes
    # the same edges between the same atoms: compare edge vectors as a multiset
    ev = np.sort(np.round(wl.pos[wl.src] - wl.pos[wl.dst], 5), axis=0)
    rv = np.sort(np.round(rw.pos[rw.src] - rw.pos[rw.dst], 5), axis=0)
    assert np.array_equal(ev, rv)
    # per-node rows move with their node: match nodes through their (unique) positions
    key = {tuple(p): i for i, p in enumerate(wl.pos.tolist())}
    old_of_new = np.array([key[tuple(p)] for p in rw.pos.tolist()])
    assert sorted(old_of_new.tolist()) == list(range(n))
    assert np.array_equal(rw.x, wl.x[old_of_new]) and np.array_equal(rw.z_bar, wl.z_bar[old_of_new])
    assert np.array_equal(np.bincount(rw.dst, minlength=n), np.bincount(wl.dst, minlength=n)[old_of_new])
    # neighbours are closer in index than in the generator's random order
    span = lambda w: np.median(np.abs(w.src.astype(np.int64) - w.dst))  # noqa: E731
    assert span(rw) < 0.5 * span(wl)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
