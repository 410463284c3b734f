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


def kernel_source_hash(kind):
    files = {
        "fwd_traverse": ["fwd_impl.hpp", "geom.hpp"],
        "bwd_traverse": ["bwd_impl.hpp", "geom.hpp"],
        "channel_gemm": ["gemm.hip"],
        "node_gemm": ["gemm.hip"],
    }.get(kind, [])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "equivariant_gnn_tensor_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind, workload):
    """HBM bytes per step for one kernel kind from committed rocprofv3 counter summaries,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_src_sha") != kernel_source_hash(kind):
        return None
    return d.get("hbm_bytes_per_step")


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
                       f"({done / wl.n_edges:.1%} of the graph) in {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU (no multi-GPU path); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import equivariant_gnn_tensor_amd as etpc
    from workloads import CONFIGS, make_workload
    from workloads.generate import scalar_mask

    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.workload]
    plan = etpc.Plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.radial, cfg.n_basis, cfg.r_lo,
                     cfg.r_hi, cfg.poly_p, box=cfg.box, out_per_path=cfg.out_per_path)
    info = plan.info()
    mask = scalar_mask(cfg.irreps_out) if cfg.cotangent == "energy" else None
    wl = make_workload(cfg, w_blocks=plan.w_blocks(), z_dim=info["z_dim"], scalar_out_mask=mask)
    N, E = wl.n_nodes, wl.n_edges
    log(f"workload {cfg.name}: N={N} E={E} paths={info['n_paths']} x_dim={info['x_dim']} z_dim={info['z_dim']}")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    x, pos, w, zb = T(wl.x), T(wl.pos), T(wl.w), T(wl.z_bar)
    src, dst = T(wl.src), T(wl.dst)
    torch.cuda.synchronize()

    # CSR build, timed on its own (not part of a step)
    graph = etpc.etpc_csr_build(N, src, dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        graph = etpc.etpc_csr_build(N, src, dst)
    torch.cuda.synchronize()
    csr_ms = (time.perf_counter() - t0) / 3 * 1e3

    force_step = "dbl" in cfg.passes
    ws_f = torch.empty(etpc.etpc_workspace_size(plan, etpc.PASS_FWD, N, E), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(etpc.etpc_workspace_size(plan, etpc.PASS_BWD, N, E), dtype=torch.uint8, device=dev)
    ws_d = (torch.empty(etpc.etpc_workspace_size(plan, etpc.PASS_DBL, N, E), dtype=torch.uint8, device=dev)
            if force_step else torch.empty(0, dtype=torch.uint8, device=dev))
    z = torch.empty(N, info["z_dim"], device=dev)
    outs = (torch.empty(N, info["x_dim"], device=dev), torch.empty(info["w_numel"], device=dev),
            torch.empty(N, 3, device=dev))
    if force_step:
        pos_dot = T(-wl.force_c)
        outs = (None, None, torch.empty(N, 3, device=dev))
        douts = (None, torch.empty(N, info["x_dim"], device=dev), torch.empty(info["w_numel"], device=dev))
    resident = torch.cuda.memory_allocated()

    def step():
        etpc.etpc_forward(plan, graph, x, pos, w, z=z, ws=ws_f)
        etpc.etpc_backward(plan, graph, x, pos, w, zb, outs=outs, ws=ws_b)
        if force_step:
            etpc.etpc_double_backward(plan, graph, x, pos, w, zb, pos_dot=pos_dot, outs=douts, ws=ws_d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated()
    ms = dt / args.steps * 1e3
    value = E / (ms / 1e3)

    # per-kind kernel time: event pairs recorded by the library on its launch stream
    etpc.etpc_profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
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
    traffic = traffic_from_profiles(dom, args.workload)
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
        "dtype": "f32",
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
        },
        "roofline": {
            "kernel": dom,
            "bound": bound,
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": traffic,
            "launches_per_step": kinds[dom]["launches_per_step"],
            "kernel_ms_per_step": dom_ms,
        },
        "step_tflops_algorithmic": total_tf,
        "step_frac_fp32_peak": total_tf / PEAK_FP32_TFLOPS,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in kinds.items()},
        "csr_build_ms": csr_ms,
        "peak_mib": peak / 2 ** 20,
        "workspace_mib": (ws_f.numel() + ws_b.numel() + ws_d.numel()) / 2 ** 20,
        "resident_mib": resident / 2 ** 20,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
