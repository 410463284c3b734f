#!/usr/bin/env python3
"""Throughput of the streaming tensor-product convolution on one MI355X.

One step = forward + backward (gradients w.r.t. x, W and positions) of the
uvw convolution on the MACE-like workload: N = 4096 atoms at 0.1 / A^3 in a
periodic box, radius graph with a 5 A cutoff (about 2.14e5 edges),
x = 64x0e+64x1o+64x2e, outputs 64x(0e,1o,2e,3o) over all valid paths, SH up to
l = 3, 8 Bessel bases with a polynomial envelope.  Inputs are seeded synthetic
data, resident in HBM before timing starts.

Prints one JSON line (see the "metric" key); diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2] [--no-cpu-baseline]

Counter summaries for the `traffic` field (rocprofv3 runs of this same script; the
--copy-calibration-mib run adds a plain device copy of known size whose counter reading
gives the scale factor):

    rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace_cfg2 -o run -- \
        python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration-mib 256
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch_cfg2 -o run -- python3 bench.py <same>
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write_cfg2 -o run -- python3 bench.py <same>
    python bench.py --summarize-profile DIR --steps 3 --warmup 1 --workload cfg2 --lanes 1 --copy-calibration-mib 256

(--lanes 1 serializes the launches, as the event-timed pass does, so the trace's per-kernel
durations are the kernels' own.)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 matrix and (packed) vector peak
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flop_model(plan, n_nodes, n_edges, radial_b, force_step=False):
    """Algorithmic FLOPs per step by kernel kind (2 per multiply-add).

    Per path pi: i = 2l_in+1, o = 2l_out+1, kappa = i*o.
      fwd traversal   E * sum C_in (kappa + B o)
      channel GEMM    N * sum B C_in C_out o
      bwd traversal   E * sum C_out (2 kappa + 3 B i)       (x_bar, W_bar and pos_bar)
      node GEMMs      3 N * sum B C_in C_out i              (Xt, x_bar, W_bar)
    uvu: fwd E * sum C (B + kappa + min(i, o)), bwd E * sum C (3B + 3i + 2 kappa).
    Force step (forward, pos_bar-only backward, double backward along pos_dot for d/dx, d/dW):
      bwd traversal   E * sum C_out (2 kappa + 2 B i) twice, node GEMMs 3 N * sum B C_in C_out i.
    """
    ins = plan.irreps_in
    outs = plan.out_irreps()
    B = radial_b
    f = dict(fwd_traverse=0.0, channel_gemm=0.0, bwd_traverse=0.0, node_gemm=0.0)
    for q in plan.paths():
        ci, li, _ = ins[q["in_block"]]
        co, lo, _ = outs[q["out_block"]]
        i, o = 2 * li + 1, 2 * lo + 1
        k = i * o
        if plan.mode == "uvw" and force_step:
            f["fwd_traverse"] += n_edges * ci * (k + B * o)
            f["channel_gemm"] += n_nodes * B * ci * co * o
            f["bwd_traverse"] += 2 * n_edges * co * (2 * k + 2 * B * i)
            f["node_gemm"] += 3 * n_nodes * B * ci * co * i
        elif plan.mode == "uvw":
            f["fwd_traverse"] += n_edges * ci * (k + B * o)
            f["channel_gemm"] += n_nodes * B * ci * co * o
            f["bwd_traverse"] += n_edges * co * (2 * k + 3 * B * i)
            f["node_gemm"] += 3 * n_nodes * B * ci * co * i
        else:
            f["fwd_traverse"] += n_edges * ci * (B + k + min(i, o))
            f["bwd_traverse"] += n_edges * ci * (3 * B + 3 * i + 2 * k)
    return {key: 2.0 * v for key, v in f.items()}


def algorithmic_bytes(plan, n_nodes, n_edges, radial_b, force_step=False):
    """Compulsory HBM bytes per step by kernel kind: every operand a launch reads or writes,
    touched once (fp32 data, int32 indices); re-reads through the caches are not counted.

    Per uvw path pi (i = 2l_in+1, o = 2l_out+1):
      fwd traversal   read x block (N i C_in), CSR (rowptr, col: 4 N + 4 E), pos (12 N);
                      write S columns (N B C_in o)
      channel GEMM    read S (N B sum_g C_in o), W; write z
      bwd traversal   read z_bar block (N o C_out), Xt and write P (N B C_out i each), sender
                      CSR (s_rowptr, s_col, s_slot: 4 N + 8 E), pos (12 N); edge adjoint
                      read-modify-write (24 E; 12 E for the first path of a lane)
      node GEMMs      Xt = x W, x_bar = P W^T, W_bar = x^T P: each operand once
    uvu (per path): forward reads x block, W block, CSR, pos and read-modify-writes its z
    block; backward reads z_bar and x blocks, read-modify-writes x_bar, edge adjoint as uvw.
    The force step counts the backward's kinds twice (backward and double backward)."""
    ins = plan.irreps_in
    outs = plan.out_irreps()
    B = radial_b
    f = dict(fwd_traverse=0.0, channel_gemm=0.0, bwd_traverse=0.0, node_gemm=0.0)
    graph_r = 4.0 * n_nodes + 4.0 * n_edges
    graph_s = 4.0 * n_nodes + 8.0 * n_edges
    lanes_seen = 0
    for q in plan.paths():
        ci, li, _ = ins[q["in_block"]]
        co, lo, _ = outs[q["out_block"]]
        i, o = 2 * li + 1, 2 * lo + 1
        rbar = 12.0 * n_edges if lanes_seen < 2 else 24.0 * n_edges
        lanes_seen += 1
        if plan.mode == "uvw":
            f["fwd_traverse"] += 4.0 * (n_nodes * i * ci + n_nodes * B * ci * o) + graph_r + 12.0 * n_nodes
            f["channel_gemm"] += 4.0 * (n_nodes * B * ci * o + B * ci * co)
            f["bwd_traverse"] += 4.0 * (n_nodes * o * co + 2 * n_nodes * B * co * i) + graph_s + 12.0 * n_nodes + rbar
            f["node_gemm"] += 4.0 * 3 * (n_nodes * i * ci + B * ci * co + n_nodes * B * co * i)
        else:
            f["fwd_traverse"] += 4.0 * (n_nodes * i * ci + B * ci + 2 * n_nodes * o * ci) + graph_r + 12.0 * n_nodes
            f["bwd_traverse"] += 4.0 * (n_nodes * o * ci + 3 * n_nodes * i * ci + B * ci) + graph_s + \
                12.0 * n_nodes + rbar
    if plan.mode == "uvw":
        zrow = sum(4.0 * n_nodes * m * (2 * l + 1) for m, l, _ in outs)
        f["channel_gemm"] += zrow
    if force_step:
        f["bwd_traverse"] *= 2
        f["node_gemm"] *= 2
    return f


def kernel_source_hash(kind):
    shared = ["common.hpp", "kernels.hpp", "wave.hpp", "triples.hpp", "cg_tables.inc"]
    files = {
        "fwd_traverse": ["fwd_impl.hpp", "geom.hpp"] + shared,
        "bwd_traverse": ["bwd_impl.hpp", "geom.hpp"] + shared,
        "channel_gemm": ["gemm.hip", "common.hpp", "kernels.hpp"],
        "node_gemm": ["gemm.hip", "common.hpp", "kernels.hpp"],
    }.get(kind, [])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "equivariant_gnn_tensor_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "equivariant_gnn_tensor_amd", "build.py"), "rb") as fh:   # compiler flags
        h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind, workload):
    """(HBM bytes per launch, per step) for one kernel kind from the committed rocprofv3
    counter summaries, or (None, None) when absent or taken on a different kernel build."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_src_sha") != kernel_source_hash(kind):
        return None, None
    return d.get("hbm_bytes_per_launch"), d.get("hbm_bytes_per_step")


def cpu_baseline(cfg, wl, seconds):
    """The float64 oracle (materialized schedule) on a bounded random sample of edges."""
    import numpy as np
    import torch
    from oracle import conv
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    spec = conv.spec_from_config(cfg)
    rng = np.random.default_rng(4242)
    order = rng.permutation(wl.n_edges)
    chunk = 256
    conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=order[:16])          # warm caches
    conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=order[:16])
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds and done < wl.n_edges:
        e = order[done:done + chunk]
        conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=e)
        conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=e)
        done += len(e)
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="edges/s", cores=torch.get_num_threads(), kind="oracle",
                sample=f"float64 materialized forward+backward of {done} randomly chosen edges "
                       f"({done / wl.n_edges:.1%} of the graph) in {dt:.1f} s",
                cpu=_cpu_model(), blas=_blas_name())


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_name():
    import re
    import torch
    m = re.search(r"BLAS_INFO=([^,\s]+)", torch.__config__.show())
    return m.group(1) if m else "unknown"


KERNEL_FAMILIES = (
    ("fwd_traverse", ("fwd_uvw_kernel", "fwd_uvu_kernel", "fwd_uvu_acc_kernel")),
    ("bwd_traverse", ("bwd_uvw_kernel", "bwd_uvu_kernel", "bwd_uvu_first_kernel")),
    ("gemm", ("gemm_f32_kernel", "gemm_low_kernel")),
    ("csr", ("radix_", "scan_", "lower_bound", "validate_", "iota_", "gather_", "copy_kernel", "degree_key_kernel",
             "window_key_kernel")),
    ("aux", ("fill_kernel", "wprep_kernel", "reduce_wbar_kernel", "segment_sum_kernel", "pos_bar_kernel",
             "splitk_reduce_kernel")),
)


def kernel_family(name):
    if "etpc::" not in name:
        return "other"
    for fam, keys in KERNEL_FAMILIES:
        if any(k in name for k in keys):
            return fam
    return "other"


def summarize_profile(d, workload, steps, warmup, copy_mib):
    """Turn the three rocprofv3 runs (kernel trace, FETCH_SIZE, WRITE_SIZE) into
    profiles/trace_<workload>.md and profiles/pmc_<kind>_<workload>.json."""
    import csv
    import glob
    import collections
    execs = warmup + 2 * steps            # timed pass + event-profiled pass
    stats = glob.glob(os.path.join(d, f"trace_{workload}", "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {d}/trace_{workload}")
    fam_t = collections.defaultdict(lambda: [0.0, 0])
    rows = []
    for r in csv.DictReader(open(stats[0])):
        f = kernel_family(r["Name"])
        fam_t[f][0] += float(r["TotalDurationNs"])
        fam_t[f][1] += int(r["Calls"])
        rows.append((float(r["TotalDurationNs"]), int(r["Calls"]), float(r["AverageNs"]), f, r["Name"]))
    rows.sort(reverse=True)

    def counters(kind):
        files = glob.glob(os.path.join(d, f"{kind}_{workload}", "**", "*counter_collection.csv"), recursive=True)
        per = collections.defaultdict(list)     # family -> [KiB per dispatch]
        copy = []
        for fn in files:
            for r in csv.DictReader(open(fn)):
                name = r.get("Kernel_Name", "")
                v = float(r["Counter_Value"])
                if "copy" in name.lower() and kernel_family(name) == "other":
                    copy.append(v)
                else:
                    per[kernel_family(name)].append(v)
        return per, copy

    fetch, fcopy = counters("fetch")
    write, wcopy = counters("write")
    known_kib = copy_mib * 1024.0
    # the calibration copy is the largest copy dispatch; its reading should be copy_mib
    f_scale = known_kib / max(fcopy) if fcopy else None
    w_scale = known_kib / max(wcopy) if wcopy else None
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    cmd_args = f"--steps {steps} --warmup {warmup} --no-cpu-baseline --workload {workload} --lanes 1 " \
               f"--copy-calibration-mib {copy_mib}"
    lines = [f"# rocprofv3 kernel trace, workload {workload}", "",
             "Commands (repo root, one MI355X):", "",
             "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace_{workload} -o run -- "
             f"python3 bench.py {cmd_args}",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch_{workload} -o run -- "
             f"python3 bench.py {cmd_args}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write_{workload} -o run -- "
             f"python3 bench.py {cmd_args}",
             f"python bench.py --summarize-profile DIR --steps {steps} --warmup {warmup} --workload {workload} "
             f"--lanes 1 --copy-calibration-mib {copy_mib}",
             "```", "",
             f"Each run executes {execs} steps (warmup {warmup} + timed {steps} + event-profiled {steps}).", "",
             "| family | launches/step | ms/step (trace) | avg us/launch | HBM MB/step (calibrated) |",
             "|---|---|---|---|---|"]
    out = {}
    for fam in ("fwd_traverse", "bwd_traverse", "gemm", "aux", "csr"):
        if fam not in fam_t:
            continue
        tot_ns, calls = fam_t[fam]
        fk = sum(fetch.get(fam, [])) * (f_scale or 0.0)
        wk = sum(write.get(fam, [])) * (w_scale or 0.0)
        nd = max(len(fetch.get(fam, [])), 1)
        mb_step = (fk + wk) * 1024.0 / execs / 1e6 if f_scale and w_scale else None
        lines.append(f"| {fam} | {calls / execs:.1f} | {tot_ns / execs / 1e6:.4f} | {tot_ns / max(calls, 1) / 1e3:.1f} | "
                     f"{mb_step if mb_step is None else round(mb_step, 1)} |")
        out[fam] = dict(launches_per_step=calls / execs, ms_per_step=tot_ns / execs / 1e6,
                        hbm_bytes_per_step=None if mb_step is None else mb_step * 1e6,
                        hbm_bytes_per_launch=None if mb_step is None else (fk + wk) * 1024.0 / nd,
                        fetch_kib_raw_per_dispatch=sum(fetch.get(fam, [])) / nd,
                        write_kib_raw_per_dispatch=sum(write.get(fam, [])) / nd)
    lines += ["", f"Copy calibration: a {copy_mib} MiB device-to-device copy read FETCH_SIZE "
                  f"{max(fcopy) if fcopy else 'n/a'} KiB and WRITE_SIZE {max(wcopy) if wcopy else 'n/a'} KiB; "
                  f"scale factors {f_scale} (fetch), {w_scale} (write).", "",
              "Top kernels by total time (all executions):", "",
              "| total ms | calls | avg us | family | kernel |", "|---|---|---|---|---|"]
    for tot, calls, avg, fam, name in rows[:16]:
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"| {tot / 1e6:.3f} | {calls} | {avg / 1e3:.1f} | {fam} | `{short}` |")
    with open(os.path.join(ROOT, "profiles", f"trace_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    kind_of = {"fwd_traverse": "fwd_traverse", "bwd_traverse": "bwd_traverse", "gemm": "gemm"}
    for fam, kind in kind_of.items():
        if fam in out and out[fam]["hbm_bytes_per_step"] is not None:
            rec = dict(out[fam], kind=kind, workload=workload, kernel_src_sha=kernel_source_hash(kind),
                       fetch_scale=f_scale, write_scale=w_scale, copy_calibration_mib=copy_mib,
                       command=f"python bench.py --summarize-profile DIR --steps {steps} --warmup {warmup} "
                               f"--workload {workload} --lanes 1 --copy-calibration-mib {copy_mib}")
            with open(os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.json"), "w") as fh:
                json.dump(rec, fh, indent=1)
    summarize_counters(d, workload, steps, warmup, {f: v[0] for f, v in fam_t.items()}, execs, cmd_args)
    print(json.dumps(out, indent=1))


def summarize_timeline(d, workload, steps, warmup, out_dir=None):
    """Concurrency of one step as run (default lanes and post stream) from a rocprofv3 kernel
    trace, DIR/timeline_<workload>, into profiles/timeline_<workload>.md: for each timed step
    the wall span, the time any kernel runs, the time a traversal runs, and per pass (forward:
    up to the backward's first weight re-layout; backward: the rest) the span, the traversal
    time and the tail after the last traversal."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, f"timeline_{workload}", "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}/timeline_{workload}")
    ev = []
    for r in csv.DictReader(open(files[0])):
        fam = kernel_family(r["Kernel_Name"])
        ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), fam, "wprep" in r["Kernel_Name"]))
    ev.sort()
    # a step starts at a forward traversal that follows backward work
    starts, prev = [], None
    for i, (_, _, fam, _) in enumerate(ev):
        if fam == "fwd_traverse" and prev in (None, "bwd_traverse"):
            starts.append(i)
        if fam in ("fwd_traverse", "bwd_traverse"):
            prev = fam
    segs = [ev[a:b] for a, b in zip(starts, starts[1:] + [len(ev)])]

    def union(iv):
        tot, cs, ce = 0, None, None
        for s0, e0 in sorted(iv):
            if cs is None or s0 > ce:
                tot += 0 if cs is None else ce - cs
                cs, ce = s0, e0
            else:
                ce = max(ce, e0)
        return tot + (0 if cs is None else ce - cs)

    trav = ("fwd_traverse", "bwd_traverse")
    cmd_args = f"--steps {steps} --warmup {warmup} --no-cpu-baseline --workload {workload}"
    lines = [f"# Concurrency of a step as run (two lanes and the post stream), workload {workload}", "",
             "Commands (repo root, one MI355X):", "", "```",
             f"rocprofv3 --kernel-trace --output-format csv -d DIR/timeline_{workload} -o run -- "
             f"python3 bench.py {cmd_args}",
             f"python bench.py --summarize-timeline DIR --steps {steps} --warmup {warmup} --workload {workload}",
             "```", "",
             f"Steps {warmup}..{warmup + steps - 1} of the run (after {warmup} warmup steps) are the timed, concurrent "
             "ones; times in us from the kernel trace (the profiler itself adds launch overhead). "
             "`busy`: some kernel runs; `traversal`: some traversal runs; `tail`: from the pass's last traversal "
             "end to its last kernel end (node-side GEMMs and reductions left after the traversals). "
             "Sums are kernel durations added up (concurrent kernels each count in full).", "",
             "| step | span | busy | traversal | fwd span | fwd traversal | fwd tail | bwd span | bwd traversal | "
             "bwd tail | sum fwd_traverse | sum bwd_traverse | sum gemm | sum aux |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in range(warmup, min(warmup + steps, len(segs))):
        seg = segs[k]
        t0, t1 = seg[0][0], max(e for _, e, _, _ in seg)
        b0 = next((s0 for s0, _, _, w in seg if w), t1)
        fw = [x for x in seg if x[0] < b0]
        bw = [x for x in seg if x[0] >= b0]

        def part(xs):
            if not xs:
                return 0, 0, 0
            a0, a1 = xs[0][0], max(e for _, e, _, _ in xs)
            tr = [(s0, e0) for s0, e0, f, _ in xs if f in trav]
            last = max((e0 for _, e0 in tr), default=a0)
            return (a1 - a0) / 1e3, union(tr) / 1e3, (a1 - last) / 1e3

        fs, ft, ftl = part(fw)
        bs, bt, btl = part(bw)
        sums = {f: sum(e0 - s0 for s0, e0, g, _ in seg if g == f) / 1e3 for f in ("fwd_traverse", "bwd_traverse",
                                                                               "gemm", "aux")}
        lines.append(f"| {k} | {(t1 - t0) / 1e3:.1f} | {union([(s0, e0) for s0, e0, _, _ in seg]) / 1e3:.1f} | "
                     f"{union([(s0, e0) for s0, e0, f, _ in seg if f in trav]) / 1e3:.1f} | {fs:.1f} | {ft:.1f} | "
                     f"{ftl:.1f} | {bs:.1f} | {bt:.1f} | {btl:.1f} | {sums['fwd_traverse']:.1f} | "
                     f"{sums['bwd_traverse']:.1f} | {sums['gemm']:.1f} | {sums['aux']:.1f} |")
    with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"timeline_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return lines


SQ_RUNS = {
    # one rocprofv3 --pmc pass each (at most 8 SQ counters per pass)
    "sq1": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAVES "
           "SQ_INSTS_LDS SQ_ACTIVE_INST_VALU",
    "sq2": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS "
           "SQ_LDS_BANK_CONFLICT SQ_WAVES SQ_INSTS_VALU",
}


def summarize_counters(d, workload, steps, warmup, fam_ns, execs, cmd_args):
    """Issue rates, matrix-core use, occupancy and LDS bank conflicts per kernel family from
    the two SQ counter passes (DIR/sq1_<workload>, DIR/sq2_<workload>) and the kernel trace,
    into profiles/counters_<workload>.md.  Skipped when the passes are absent."""
    import csv
    import glob
    import collections
    runs = {}
    for tag in SQ_RUNS:
        files = glob.glob(os.path.join(d, f"{tag}_{workload}", "**", "*counter_collection.csv"), recursive=True)
        if not files:
            return
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        for fn in files:
            for r in csv.DictReader(open(fn)):
                agg[kernel_family(r.get("Kernel_Name", ""))][r["Counter_Name"]] += float(r["Counter_Value"])
        runs[tag] = agg
    simd_cycles = lambda ns: ns * 1e-9 * 2.4e9 * 1024          # noqa: E731  (256 CUs x 4 SIMDs)
    lines = [f"# Issue rates, matrix cores, occupancy and LDS bank conflicts, workload {workload}", "",
             "Commands (repo root, one MI355X; each run executes "
             f"{execs} steps: warmup {warmup}, timed {steps}, event-profiled {steps}):", "", "```"]
    for tag, ctrs in SQ_RUNS.items():
        lines.append(f"rocprofv3 --pmc {ctrs} --output-format csv -d DIR/{tag}_{workload} -o run -- "
                     f"python3 bench.py {cmd_args}")
    lines += [f"python bench.py --summarize-profile DIR --steps {steps} --warmup {warmup} --workload {workload} "
              f"--lanes 1 --copy-calibration-mib 256", "```", "",
              "Counters are summed over all dispatches of a family; durations come from the kernel trace "
              "(trace_" + workload + ".md) of the same command.",
              "- VALU issue = SQ_INSTS_VALU x 4 cycles / (duration x 2.4 GHz x 1024 SIMDs): a wave64 fp32 VALU "
              "operation holds a 16-lane SIMD for four cycles (SQ_INSTS_VALU includes the MFMA instructions).",
              "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (duration x 2.4 GHz x 1024).",
              "- waves / SIMD = 4 x SQ_WAVE_CYCLES (quad-cycles) / (duration x 2.4 GHz x 1024).",
              "- active / wait / wait-issue: SQ_ACTIVE_INST_ANY, SQ_WAIT_ANY, SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES.",
              "- LDS bank conflict rate = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (conflict cycles per LDS-active "
              "cycle).", "",
              "| family | ms (all steps) | VALU issue | MFMA busy | waves / SIMD | active / wait / wait-issue | "
              "LDS instr / wave | LDS bank conflict rate |", "|---|---|---|---|---|---|---|---|"]
    for fam in ("fwd_traverse", "bwd_traverse", "gemm", "aux", "csr"):
        if fam not in fam_ns or fam not in runs["sq1"]:
            continue
        ns = fam_ns[fam]
        a, b = runs["sq1"][fam], runs["sq2"].get(fam, {})
        cyc = simd_cycles(ns)
        wc = b.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        lines.append(
            f"| {fam} | {ns / 1e6:.3f} | {a['SQ_INSTS_VALU'] * 4 / cyc:.3f} | "
            f"{a['SQ_VALU_MFMA_BUSY_CYCLES'] / cyc:.3f} | {4 * a['SQ_WAVE_CYCLES'] / cyc:.2f} | "
            f"{b.get('SQ_ACTIVE_INST_ANY', 0) / wc:.2f} / {b.get('SQ_WAIT_ANY', 0) / wc:.2f} / "
            f"{b.get('SQ_WAIT_INST_ANY', 0) / wc:.2f} | {a['SQ_INSTS_LDS'] / max(a['SQ_WAVES'], 1):.0f} | "
            f"{b.get('SQ_LDS_BANK_CONFLICT', 0) / max(b.get('SQ_ACTIVE_INST_LDS', 0), 1):.3f} |")
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def morton_relabel(wl):
    """Renumber the workload's nodes in Morton (Z-curve) order of their positions: the same
    graph and values, with neighbours close in index.  Returns a new Workload."""
    import dataclasses

    import numpy as np
    pos = wl.pos.astype(np.float64)
    lo, hi = pos.min(axis=0), pos.max(axis=0)
    q = np.clip(((pos - lo) / np.maximum(hi - lo, 1e-12) * 1023).astype(np.int64), 0, 1023)
    code = np.zeros(len(pos), np.int64)
    for bit in range(10):
        for a in range(3):
            code |= ((q[:, a] >> bit) & 1) << (3 * bit + a)
    order = np.argsort(code, kind="stable")          # new index -> old index
    new_of_old = np.empty_like(order)
    new_of_old[order] = np.arange(len(order))
    perm = lambda a: None if a is None else np.ascontiguousarray(a[order])  # noqa: E731
    return dataclasses.replace(wl, pos=perm(wl.pos), x=perm(wl.x), z_bar=perm(wl.z_bar), force_c=perm(wl.force_c),
                               src=new_of_old[wl.src].astype(np.int32), dst=new_of_old[wl.dst].astype(np.int32))


def measure(args, name):
    """Time one workload: (result dict without cpu_baseline, config, workload)."""
    import numpy as np
    import torch
    import equivariant_gnn_tensor_amd as etpc
    from workloads import CONFIGS, make_workload
    from workloads.generate import scalar_mask

    dev = torch.device("cuda:0")
    cfg = CONFIGS[name]

    def make_plan(lanes):
        return etpc.Plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.radial, cfg.n_basis, cfg.r_lo,
                         cfg.r_hi, cfg.poly_p, box=cfg.box, out_per_path=cfg.out_per_path,
                         gemm_precision=args.gemm_precision, lanes=lanes)
    plan = make_plan(args.lanes)
    # the same plan with every launch in order on one stream, for the per-kernel timing pass
    plan_serial = make_plan(1)
    info = plan.info()
    mask = scalar_mask(cfg.irreps_out) if cfg.cotangent == "energy" else None
    wl = make_workload(cfg, w_blocks=plan.w_blocks(), z_dim=info["z_dim"], scalar_out_mask=mask)
    if args.node_order == "morton":
        wl = morton_relabel(wl)
    N, E = wl.n_nodes, wl.n_edges
    log(f"workload {cfg.name}: N={N} E={E} paths={info['n_paths']} x_dim={info['x_dim']} z_dim={info['z_dim']}")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    x, pos, w, zb = T(wl.x), T(wl.pos), T(wl.w), T(wl.z_bar)
    src, dst = T(wl.src), T(wl.dst)
    torch.cuda.synchronize()

    # CSR build (with the dispatch orders), timed on its own (not part of a step).  The
    # spatial base order needs one shared frame: batches of cells that overlap in space
    # (workload 6) keep the index base, whose cell-major numbering is already local.
    spatial = args.dispatch_base == "spatial" and cfg.n_graphs == 1
    sp_kw = dict(pos=pos, box=(cfg.box,) * 3 if cfg.box else None) if spatial else {}
    graph = etpc.etpc_csr_build(N, src, dst, order=args.sender_order == "degree", **sp_kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        graph = etpc.etpc_csr_build(N, src, dst, order=args.sender_order == "degree", **sp_kw)
    torch.cuda.synchronize()
    csr_ms = (time.perf_counter() - t0) / 3 * 1e3

    force_step = "dbl" in cfg.passes
    budget = int(args.workspace_mib * 2 ** 20) if args.workspace_mib > 0 else 0
    # the passes of a step run one after another on one stream: one workspace, sized to the
    # largest pass, serves them all
    passes = (etpc.PASS_FWD, etpc.PASS_BWD) + ((etpc.PASS_DBL,) if force_step else ())
    ws_all = torch.empty(max(etpc.etpc_workspace_size(plan, p_, N, E, budget) for p_ in passes),
                         dtype=torch.uint8, device=dev)
    ws_f = ws_b = ws_d = ws_all
    z = torch.empty(N, info["z_dim"], device=dev)
    outs = (torch.empty(N, info["x_dim"], device=dev), torch.empty(info["w_numel"], device=dev),
            torch.empty(N, 3, device=dev))
    if force_step:
        pos_dot = T(-wl.force_c)
        outs = (None, None, torch.empty(N, 3, device=dev))
        douts = (None, torch.empty(N, info["x_dim"], device=dev), torch.empty(info["w_numel"], device=dev))
    resident = torch.cuda.memory_allocated()

    def step(plan=plan):
        etpc.etpc_forward(plan, graph, x, pos, w, z=z, ws=ws_f)
        etpc.etpc_backward(plan, graph, x, pos, w, zb, outs=outs, ws=ws_b)
        if force_step:
            etpc.etpc_double_backward(plan, graph, x, pos, w, zb, pos_dot=pos_dot, outs=douts, ws=ws_d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one step captured as a HIP graph (every launch of the library, no host work, no
        # memset nodes: buffers are cleared by fill kernels) and replayed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        hg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(hg):
            step()
        hg.replay()
        torch.cuda.synchronize()
        run = hg.replay
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated()
    ms = dt / args.steps * 1e3
    value = E / (ms / 1e3)

    # per-kind kernel time: event pairs recorded by the library on its launch streams, with
    # the lanes serialized so that each launch's duration is its own (concurrent launches
    # share the chip and would each look slower)
    timed_lanes = plan.spec.lanes or 2
    etpc.etpc_profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step(plan_serial)
    torch.cuda.synchronize()
    prof_ms = (time.perf_counter() - t1) / args.steps * 1e3
    kinds = {}
    for k in etpc.KINDS:
        tot, n = etpc.etpc_profile_read(k)
        kinds[k] = dict(ms_per_step=tot / args.steps, launches_per_step=n / args.steps)
    etpc.etpc_profile_enable(False)
    flops = flop_model(plan, N, E, cfg.n_basis, force_step)
    log(f"step {ms:.3f} ms (profiled pass {prof_ms:.3f} ms); csr build {csr_ms:.3f} ms")
    for k, v in kinds.items():
        tf = flops.get(k, 0.0) / (v["ms_per_step"] * 1e-3) / 1e12 if v["ms_per_step"] > 0 and k in flops else 0.0
        log(f"  {k:13s} {v['ms_per_step']:8.3f} ms/step  {v['launches_per_step']:5.1f} launches  {tf:7.2f} TFLOP/s")
    compute = {k: kinds[k]["ms_per_step"] for k in flops}
    dom = max(compute, key=compute.get)
    dom_ms = kinds[dom]["ms_per_step"]
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    bound = "mfma" if dom.endswith("gemm") else "alu"
    traffic, traffic_step = traffic_from_profiles(dom, name)
    alg_bytes = algorithmic_bytes(plan, N, E, cfg.n_basis, force_step).get(dom)
    hbm_achieved = None if traffic_step is None else traffic_step / (dom_ms * 1e-3) / 1e9
    total_tf = sum(flops.values()) / (ms * 1e-3) / 1e12
    log(f"whole step: {total_tf:.2f} TFLOP/s algorithmic ({total_tf / PEAK_FP32_TFLOPS:.1%} of fp32 peak)")

    result = {
        "metric": "edges/s fwd+bwd (uvw, 64x0e+1o+2e)" if cfg.index == 2 else
                  (f"edges/s fwd+bwd+dbl ({cfg.name})" if force_step else f"edges/s fwd+bwd ({cfg.name})"),
        "value": value,
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.gemm_precision == "fp32" else f"f32, {args.gemm_precision} channel GEMMs",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: N={N} atoms at 0.1/A^3 (periodic), radius graph 5 A, E={E}, "
                        f"x {cfg.irreps_in} -> {cfg.irreps_out}, lmax_sh={cfg.lmax_sh}, B={cfg.n_basis} {cfg.radial}"
                        if cfg.graph == "radius" else
                        f"{cfg.name}: N={N}, in-degree {cfg.degree}, E={E}, x {cfg.irreps_in} -> {cfg.irreps_out}",
            "n_nodes": N,
            "n_edges": E,
            "mode": cfg.mode,
            "pass": ("forward + backward (pos_bar) + double backward along pos_dot (d/dx, d/dW)" if force_step
                     else "forward + backward (x_bar, W_bar, pos_bar)"),
            "launch": "hip graph replay" if args.graph else "eager",
            "node_order": args.node_order,
            "sender_order": args.sender_order,
            "dispatch_base": "spatial" if spatial and args.sender_order == "degree" else "index",
            "lanes": timed_lanes,
        },
        "roofline": {
            "kernel": dom,
            "bound": bound,
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": traffic,
            "traffic_per_step": traffic_step,
            "hbm_gbs": hbm_achieved,
            "hbm_frac": None if hbm_achieved is None else hbm_achieved / PEAK_HBM_GBS,
            "algorithmic_bytes_per_step": alg_bytes,
            "algorithmic_gbs": None if alg_bytes is None else alg_bytes / (dom_ms * 1e-3) / 1e9,
            "launches_per_step": kinds[dom]["launches_per_step"],
            "kernel_ms_per_step": dom_ms,
        },
        "step_tflops_algorithmic": total_tf,
        "step_frac_fp32_peak": total_tf / PEAK_FP32_TFLOPS,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kinds.items()},
        "csr_build_ms": csr_ms,
        "peak_mib": peak / 2 ** 20,
        "workspace_mib": ws_all.numel() / 2 ** 20,
        "workspace_budget_mib": budget / 2 ** 20 if budget else None,
        "resident_mib": resident / 2 ** 20,
    }
    return result, cfg, wl


def graph_count_sweep(args):
    """Throughput of the block-diagonal batches of 128-atom cells (graph-count scaling):
    prints one JSON line with every point and the endpoint's share of the peak."""
    import gc
    import torch
    from workloads.configs import GRAPH_COUNTS
    points = []
    for b in GRAPH_COUNTS:
        r, cfg, wl = measure(args, f"cfg6_b{b}")
        points.append(dict(graphs=b, n_nodes=cfg.n_nodes, n_edges=wl.n_edges, ms_per_step=r["ms_per_step"],
                           edges_per_s=r["value"], peak_mib=r["peak_mib"]))
        log(f"graphs {b:4d}: E={wl.n_edges:9d}  {r['ms_per_step']:8.3f} ms  {r['value']:.4g} edges/s")
        del r, cfg, wl
        gc.collect()
        torch.cuda.empty_cache()
    peak = max(p["edges_per_s"] for p in points)
    end = points[-1]
    print(json.dumps({
        "metric": "edges/s fwd+bwd, graph-count sweep (uvw, 64x0e+1o+2e, 128-atom periodic cells)",
        "value": end["edges_per_s"], "unit": "edges/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": end["ms_per_step"], "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"graph_count: {len(points)} batch sizes of 128-atom cells, 0.1/A^3, radius 5 A"},
        "retention_at_endpoint": end["edges_per_s"] / peak, "sweep": points}), flush=True)


def prep_bench(args):
    """Graph preparation: radius-graph builds at the workloads' density and mul_ir -> ir_mul
    conversions, each timed over --steps calls after --warmup; one JSON line."""
    import ctypes as C

    import numpy as np
    import torch
    import equivariant_gnn_tensor_amd as etpc
    from workloads import CONFIGS

    dev = torch.device("cuda:0")
    rows = []
    for n in (4096, 65536, 262144):
        L = (n / 0.1) ** (1.0 / 3.0)
        pos = torch.from_numpy(np.random.default_rng(n).uniform(0.0, L, size=(n, 3)).astype(np.float32)).to(dev)
        cap = 64 * n
        src = torch.empty(cap, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        ws = torch.empty(etpc.etpc_radius_graph_workspace_size(n, cap), dtype=torch.uint8, device=dev)
        ne = C.c_int64()
        box = (C.c_float * 3)(L, L, L)

        def build():
            st = etpc.lib.etpc_radius_graph(n, pos.data_ptr(), 5.0, box, cap, src.data_ptr(), dst.data_ptr(),
                                            C.byref(ne), ws.data_ptr(), ws.numel(), None)
            if st != 0:
                raise RuntimeError(etpc.lib.etpc_last_error().decode())
        for _ in range(args.warmup):
            build()
        torch.cuda.synchronize()
        etpc.etpc_profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            build()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        kms, launches = etpc.etpc_profile_read("prep")
        etpc.etpc_profile_enable(False)
        rows.append(dict(n_nodes=n, box=round(L, 3), n_edges=int(ne.value), ms=ms, edges_per_s=ne.value / ms * 1e3,
                         kernel_ms=kms / args.steps))
        log(f"radius graph N={n}: E={ne.value} {ms:.3f} ms/build (kernels {kms / args.steps:.3f} ms) "
            f"{ne.value / ms * 1e3:.3g} edges/s")
        del pos, src, dst, ws
    conv = []
    cfg = CONFIGS["cfg2"]
    plan = etpc.Plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.radial, cfg.n_basis, cfg.r_lo,
                     cfg.r_hi, cfg.poly_p, box=cfg.box, out_per_path=cfg.out_per_path)
    zdim = plan.info()["z_dim"]
    for n in (4096, 262144):
        x = torch.randn(n, zdim, device=dev)
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            etpc.etpc_layout_convert(plan, "out", "to_ir_mul", x, out=y)
        torch.cuda.synchronize()
        etpc.etpc_profile_enable(True)
        for _ in range(args.steps):
            etpc.etpc_layout_convert(plan, "out", "to_ir_mul", x, out=y)
        kms, _ = etpc.etpc_profile_read("prep")
        etpc.etpc_profile_enable(False)
        per = kms / args.steps
        gbs = 2 * x.numel() * 4 / (per * 1e-3) / 1e9
        conv.append(dict(rows=n, width=zdim, kernel_ms=per, gb_per_s=gbs, frac_hbm=gbs / 8000.0))
        log(f"layout mul_ir->ir_mul {n}x{zdim}: {per * 1e3:.1f} us, {gbs:.0f} GB/s ({gbs / 8000:.3f} of 8 TB/s)")
        del x, y
    main_row = rows[1]
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle (brute force over all pairs) on a bounded sample of receivers of the 65,536-atom case
        from oracle import radius as oradius
        n = main_row["n_nodes"]
        L = (n / 0.1) ** (1.0 / 3.0)
        pos = np.random.default_rng(n).uniform(0.0, L, size=(n, 3)).astype(np.float32)
        t0 = time.perf_counter()
        done = edges = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            recv = np.arange(done, min(done + 256, n))
            s_, _ = oradius.neighbours_of(pos, recv, 5.0, (L, L, L))
            edges += s_.size
            done += recv.size
        dt = time.perf_counter() - t0
        cpu = {"value": edges / dt, "unit": "edges/s", "cores": 1,   # numpy elementwise work: one thread
               "kind": "oracle", "sample": f"brute-force rows of {done} of {n} receivers ({edges} edges) in {dt:.1f} s"}
        log(f"oracle radius graph: {edges / dt:.3g} edges/s on {done} receivers")
    print(json.dumps({
        "metric": "radius graph build, edges/s", "value": main_row["edges_per_s"], "unit": "edges/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_row["ms"], "higher_is_better": True,
        "scaling": "strong", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "radius graph of uniform points at 0.1/A^3, cutoff 5 A, periodic cube",
                   "n_nodes": main_row["n_nodes"]},
        "radius_graph": rows, "layout_convert": conv, "cpu_baseline": cpu}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workspace-mib", type=float, default=0.0,
                    help="cap each pass's workspace (0 = the full size; smaller runs in node chunks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (counter calibration)")
    ap.add_argument("--lanes", type=int, default=0,
                    help="concurrent launch lanes per pass for the timed steps (0 = library default)")
    ap.add_argument("--node-order", choices=("given", "morton"), default="given",
                    help="node numbering: as generated (random in space) or Morton order of the positions")
    ap.add_argument("--dispatch-base", choices=("spatial", "index"), default="spatial",
                    help="base sequence of the degree-windowed dispatch orders: the Morton order of the "
                         "positions (single graphs) or the node index")
    ap.add_argument("--sender-order", choices=("degree", "index"), default="degree",
                    help="traversal dispatch: nodes by decreasing degree (the graph's s_order and r_order) "
                         "or in index order")
    ap.add_argument("--gemm-precision", choices=("fp32", "bf16", "fp16"), default="fp32",
                    help="channel GEMM operands: fp32 (reference), or bf16 / fp16 with fp32 accumulation")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured as a HIP graph (launch-bound small workloads)")
    ap.add_argument("--graph-count-sweep", action="store_true",
                    help="time the graph-count batches (1..511 cells) and report throughput retention")
    ap.add_argument("--prep", action="store_true",
                    help="time the graph-preparation steps (radius graph, layout conversion)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="summarize rocprofv3 output under DIR into profiles/ and exit (no GPU needed)")
    ap.add_argument("--summarize-timeline", metavar="DIR", default=None,
                    help="summarize a rocprofv3 kernel trace of a concurrent run under DIR into profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_timeline:
        summarize_timeline(args.summarize_timeline, args.workload, args.steps, args.warmup)
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.steps, args.warmup, args.copy_calibration_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU (no multi-GPU path); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.graph_count_sweep:
        graph_count_sweep(args)
        return
    if args.prep:
        prep_bench(args)
        return
    result, cfg, wl = measure(args, args.workload)
    if args.copy_calibration_mib > 0:
        nel = args.copy_calibration_mib * 2 ** 20 // 4
        a_src = torch.ones(nel, device=dev)
        a_dst = torch.empty_like(a_src)
        for _ in range(3):
            a_dst.copy_(a_src)
        torch.cuda.synchronize()
        del a_src, a_dst
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
