"""GPU parity against the float64 oracle, element by element, in the launch
configurations the benchmark runs.

Small parity cases (N <= 512, tests/test_gpu_parity.py) take the edge-split traversal
instantiations, because a launch over so few nodes splits each node's edges over
several waves.  The benchmark's graphs are large enough for the unsplit, one-wave-per-node
instantiations.  The cases here reach those paths with the oracle still affordable:
- workload 2 and 5 recipes at N = 600 (1200 waves per launch, above the split limit of
  1024, so every traversal runs unsplit): forward, backward with every element of
  W_bar, and workload 5's force double backward;
- the same graphs with a fraction of the full workspace, and with workspaces sized by a
  scratch budget (the bounded schedule: one buffer set, node chunks per output group or
  input block, one or two edge-adjoint copies);
- a channelwise (uvu) graph of 10240 nodes, so each of the 4608 persistent backward
  workgroups strides over two or three senders and sums W_bar partials over them, and the
  4608 partial copies are reduced in three levels;
- workload 2 at its full size (N = 4096, E = 214,980): z, x_bar, W_bar and pos_bar
  compared with the whole-graph oracle element by element.
Tolerance (max|d| / max|ref| per output tensor): 1e-4 forward and backward, 1e-3 double
backward.  The streaming order differs from the materialized one only by rounding
(Sobek paper, Sec. 3: the reassociation is exact in exact arithmetic).
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

from oracle import conv
from tests.gpu_helpers import make_case, note, rel_err
from workloads import CONFIGS, small_variant

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_DBL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import equivariant_gnn_tensor_amd  # noqa: F401  (fails loudly if the library is missing)
    torch.set_num_threads(max(1, len(os.sched_getaffinity(0))))


def _etpc():
    import equivariant_gnn_tensor_amd as etpc
    return etpc


def _oracle_fwd_bwd(c):
    wl = c.wl
    rz = conv.forward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    rb = conv.backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar)
    return rz, rb


@pytest.fixture(scope="module")
def cfg2_600():
    cfg = small_variant("cfg2", 600)
    c = make_case(cfg)
    note(f"{cfg.name}: N={cfg.n_nodes} E={c.wl.n_edges}, oracle forward + backward")
    rz, rb = _oracle_fwd_bwd(c)
    return c, rz, rb


def _check_fwd_bwd(etpc, c, rz, rb, ws_f=None, ws_b=None, tag=""):
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, ws=ws_f)
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, ws=ws_b)
    torch.cuda.synchronize()
    errs = (rel_err(z, rz), rel_err(xb, rb[0]), rel_err(wb, rb[1]), rel_err(pb, rb[2]))
    note(f"{c.cfg.name}{tag}: rel err z {errs[0]:.2e} x_bar {errs[1]:.2e} W_bar {errs[2]:.2e} pos_bar {errs[3]:.2e}")
    assert max(errs) <= TOL, errs


def test_cfg2_unsplit_traversals(cfg2_600):
    c, rz, rb = cfg2_600
    _check_fwd_bwd(_etpc(), c, rz, rb)


def test_cfg2_chunked_workspace(cfg2_600):
    """A fifth (forward) and a third (backward) of the full workspace: receiver and
    sender chunks, the backward pipeline alternating its two buffer sets over chunks."""
    etpc = _etpc()
    c, rz, rb = cfg2_600
    N, E = c.cfg.n_nodes, c.wl.n_edges
    ff = etpc.etpc_workspace_size(c.plan, etpc.PASS_FWD, N, E)
    fb = etpc.etpc_workspace_size(c.plan, etpc.PASS_BWD, N, E)
    ws_f = torch.empty(ff // 5, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(fb // 3, dtype=torch.uint8, device="cuda")
    _check_fwd_bwd(etpc, c, rz, rb, ws_f, ws_b, tag=" (chunked)")


@pytest.mark.parametrize("name,n,d,budget_mib", [("cfg2", 600, None, 24), ("cfg4_d64", 300, 64, 3)])
def test_budgeted_workspace(name, n, d, budget_mib, cfg2_600):
    """Workspaces sized by a scratch budget well below the full size run the bounded
    schedule (one buffer set, per-group / per-block node chunks): workload 2 at 24 MiB
    keeps an edge-adjoint copy per lane; the edge-sweep recipe at 3 MiB keeps one copy and
    one lane.  Forward and backward against the oracle."""
    etpc = _etpc()
    if name == "cfg2":
        c, rz, rb = cfg2_600
    else:
        c = make_case(small_variant(name, n, d))
        note(f"{c.cfg.name}: N={c.cfg.n_nodes} E={c.wl.n_edges}, oracle forward + backward")
        rz, rb = _oracle_fwd_bwd(c)
    N, E = c.cfg.n_nodes, c.wl.n_edges
    budget = budget_mib << 20
    sizes = [etpc.etpc_workspace_size(c.plan, p_, N, E, budget) for p_ in (etpc.PASS_FWD, etpc.PASS_BWD)]
    full = [etpc.etpc_workspace_size(c.plan, p_, N, E) for p_ in (etpc.PASS_FWD, etpc.PASS_BWD)]
    note(f"{c.cfg.name}: budget {budget_mib} MiB -> fwd {sizes[0] / 2**20:.1f} MiB (full {full[0] / 2**20:.1f}), "
         f"bwd {sizes[1] / 2**20:.1f} MiB (full {full[1] / 2**20:.1f})")
    assert all(sz <= budget for sz in sizes) and full[1] > 2 * budget
    ws_f, ws_b = (torch.empty(sz, dtype=torch.uint8, device="cuda") for sz in sizes)
    _check_fwd_bwd(etpc, c, rz, rb, ws_f, ws_b, tag=f" (budget {budget_mib} MiB)")


@pytest.mark.timeout(600)
def test_cfg5_unsplit_double_backward():
    """Workload 5's force step at N = 600: forward, backward, and the double backward of
    L = <c, F> (F = -pos_bar) along pos_dot = -c, whole and with a 16 MiB scratch budget."""
    etpc = _etpc()
    cfg = small_variant("cfg5", 600)
    c = make_case(cfg)
    wl = c.wl
    note(f"{cfg.name}: N={cfg.n_nodes} E={wl.n_edges}, oracle forward + backward")
    rz, rb = _oracle_fwd_bwd(c)
    _check_fwd_bwd(etpc, c, rz, rb)
    note(f"{cfg.name}: oracle double backward")
    pd_np = -wl.force_c.astype(np.float64)
    ref = conv.double_backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, pos_dot=pd_np)
    pos_dot = torch.from_numpy(-wl.force_c).cuda()
    small = etpc.etpc_workspace_size(c.plan, etpc.PASS_DBL, cfg.n_nodes, wl.n_edges, 16 << 20)
    for tag, ws in (("", None), (" (16 MiB budget)", torch.empty(small, dtype=torch.uint8, device="cuda"))):
        got = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pos_dot, ws=ws)
        torch.cuda.synchronize()
        errs = tuple(rel_err(g, r) for g, r in zip(got, ref))
        note(f"{cfg.name}{tag} double backward rel err z_bar {errs[0]:.2e} x {errs[1]:.2e} W {errs[2]:.2e} "
             f"pos {errs[3]:.2e}")
        assert max(errs) <= TOL_DBL, errs


@pytest.mark.timeout(900)
def test_uvu_persistent_grid_strides():
    """Channelwise workload recipe at N = 10240 (16 channels per block): the backward's
    persistent grid of 4608 workgroups takes two or three senders per workgroup, so every
    W_bar partial sums over several senders before the fixed-order reduction."""
    etpc = _etpc()
    cfg = dataclasses.replace(small_variant("cfg3", 10240), irreps_in="16x0e+16x1o+16x2e+16x3o",
                              name="uvu_strided_n10240")
    c = make_case(cfg)
    note(f"{cfg.name}: N={cfg.n_nodes} E={c.wl.n_edges}, oracle forward + backward")
    rz, rb = _oracle_fwd_bwd(c)
    _check_fwd_bwd(etpc, c, rz, rb)


@pytest.mark.timeout(900)
def test_cfg2_full_size_elementwise():
    """Workload 2 at its full size, as the benchmark runs it: every element of z, x_bar,
    W_bar and pos_bar against the whole-graph oracle (evaluated over edge subsets whose
    sum is the whole, with a progress line per subset)."""
    etpc = _etpc()
    cfg = CONFIGS["cfg2"]
    c = make_case(cfg)
    wl = c.wl
    note(f"{cfg.name}: N={cfg.n_nodes} E={wl.n_edges}, GPU forward + backward")
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in (z, xb, wb, pb)]
    parts = np.array_split(np.arange(wl.n_edges), 12)
    rz = np.zeros_like(got[0])
    rb = [np.zeros_like(g) for g in got[1:]]
    for k, e in enumerate(parts):
        rz += conv.forward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=e)
        for acc, part in zip(rb, conv.backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=e)):
            acc += part
        note(f"  oracle edge subset {k + 1}/{len(parts)} done")
    errs = (rel_err(got[0], rz), rel_err(got[1], rb[0]), rel_err(got[2], rb[1]), rel_err(got[3], rb[2]))
    note(f"{cfg.name} full size: rel err z {errs[0]:.2e} x_bar {errs[1]:.2e} W_bar {errs[2]:.2e} "
         f"pos_bar {errs[3]:.2e}")
    assert max(errs) <= TOL, errs
