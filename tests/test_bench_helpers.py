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


def test_timeline_summary_of_a_synthetic_trace(tmp_path):
    """The concurrency summary of a hand-made kernel trace: two steps (warmup 1, timed 1);
    the timed step has a forward of two overlapping traversals and a GEMM tail, then a
    backward that starts at a weight re-layout, with a traversal, a concurrent GEMM and a
    tail.  Times in ns; every expected figure is worked out by hand below."""
    import csv
    tdir = tmp_path / "timeline_syn" / "run"
    tdir.mkdir(parents=True)
    F, B = "void etpc::fwd_detail::fwd_uvw_kernel<2>(A)", "void etpc::bwd_detail::bwd_uvw_kernel<2>(A)"
    G, W = "void etpc::gemm_f32_kernel<2>(A)", "etpc::wprep_kernel(A)"
    rows = [  # (name, start, end)
        (F, 0, 1000), (B, 1000, 2000),                       # warmup step
        (F, 10000, 13000), (F, 11000, 14000),                # timed step: forward traversals
        (G, 13500, 15000),                                   # forward GEMM tail: 14000 -> 15000
        (W, 15200, 15300),                                   # backward starts here
        (B, 15300, 18300), (G, 16000, 17000),                # traversal and a concurrent GEMM
        (G, 18300, 18800),                                   # backward tail: 18300 -> 18800
    ]
    with open(tdir / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)
    lines = bench.summarize_timeline(str(tmp_path), "syn", 1, 1, out_dir=str(tmp_path))
    row = [c.strip() for c in lines[-1].strip("|").split("|")]
    got = dict(zip(["step", "span", "busy", "trav", "fspan", "ftrav", "ftail", "bspan", "btrav", "btail",
                    "sf", "sb", "sg", "sa"], row))
    assert got["step"] == "1"
    assert float(got["span"]) == 8.8           # 10000 -> 18800 ns
    assert float(got["busy"]) == 8.6           # idle 15000-15200
    assert float(got["trav"]) == 7.0           # 10000-14000 and 15300-18300
    assert float(got["fspan"]) == 5.0 and float(got["ftrav"]) == 4.0 and float(got["ftail"]) == 1.0
    assert float(got["bspan"]) == 3.6 and float(got["btrav"]) == 3.0 and float(got["btail"]) == 0.5
    assert float(got["sf"]) == 6.0 and float(got["sb"]) == 3.0 and float(got["sg"]) == 3.0 and float(got["sa"]) == 0.1
    assert (tmp_path / "timeline_syn.md").exists()
