"""Shared setup for GPU parity tests: one workload on both sides."""
import dataclasses
import sys

import numpy as np
import torch

from oracle import conv
from tests.planner_helpers import plan_from_config
from workloads import make_workload
from workloads.generate import scalar_mask


def note(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Case:
    cfg: object
    spec: object           # oracle spec
    plan: object           # library plan
    wl: object             # numpy workload
    graph: object          # device CSR
    x: torch.Tensor
    pos: torch.Tensor
    w: torch.Tensor
    z_bar: torch.Tensor


def make_case(cfg, dev="cuda:0", gemm_precision="fp32"):
    import equivariant_gnn_tensor_amd as etpc
    spec = conv.spec_from_config(cfg)
    mask = scalar_mask(cfg.irreps_out) if cfg.cotangent == "energy" else None
    wl = make_workload(cfg, w_blocks=spec.plan.w_blocks(), z_dim=spec.plan.z_dim, scalar_out_mask=mask)
    plan = plan_from_config(cfg, gemm_precision)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    graph = etpc.etpc_csr_build(cfg.n_nodes, t(wl.src), t(wl.dst))
    return Case(cfg, spec, plan, wl, graph, t(wl.x), t(wl.pos), t(wl.w), t(wl.z_bar))


def rel_err(got, ref):
    got = got.detach().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))
