"""Host-side checks of the C ABI library: symbols, planner, validation (no GPU needed)."""
import re
import os

import numpy as np
import pytest

import equivariant_gnn_tensor_amd as etpc
from equivariant_gnn_tensor_amd import _binding
from oracle import irreps as oir
from oracle.cg import real_cg
from tests.planner_helpers import plan_from_config
from workloads import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "etpc.h")


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:etpc_status|void|const char\*|int32_t)\s+(etpc_[a-z_]+)\s*\(", text, re.M))
    assert declared == set(etpc.SYMBOLS)
    for name in declared:
        assert hasattr(etpc.lib, name), name


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg4_d64", "cfg5"])
def test_planner_matches_oracle_plan(name):
    cfg = CONFIGS[name]
    plan = plan_from_config(cfg)
    oplan = oir.make_plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.n_basis,
                          out_per_path=cfg.out_per_path)
    info = plan.info()
    assert (info["x_dim"], info["z_dim"], info["w_numel"], info["n_paths"]) == \
        (oplan.x_dim, oplan.z_dim, oplan.w_numel, len(oplan.paths))
    assert plan.out_irreps() == [tuple(t) for t in oplan.irreps_out]
    xoff, zoff = oir.offsets(oplan.irreps_in), oir.offsets(oplan.irreps_out)
    for p, (q, o) in enumerate(zip(plan.paths(), oplan.paths)):
        assert (q["in_block"], q["l_sh"], q["out_block"], q["w_off"], q["w_numel"]) == \
            (o.in_block, o.l_sh, o.out_block, o.w_off, o.w_numel)
        assert (q["l_in"], q["l_out"], q["x_off"], q["z_off"]) == \
            (o.l_in, o.l_out, xoff[o.in_block], zoff[o.out_block])
        assert q["fan_in"] == oplan.fan_in(o)
        np.testing.assert_allclose(plan.cg(p), real_cg(o.l_in, o.l_sh, o.l_out), atol=1e-12)


def test_racah_cg_all_triples():
    """Planner (Racah + real-basis change) vs oracle (null space) for every l <= 3 triple."""
    for li in range(4):
        for lo in range(4):
            plan = etpc.Plan(f"1x{li}e", "+".join(f"1x{lo}{'e' if (li + ls) % 2 == 0 else 'o'}" for ls in range(4)),
                             3, "uvw", "gaussian", 2, 0.0, 1.0)
            for p, q in enumerate(plan.paths()):
                np.testing.assert_allclose(plan.cg(p), real_cg(li, q["l_sh"], lo), atol=1e-12)


@pytest.mark.parametrize("kwargs,status", [
    (dict(irreps_in="4x4e"), "UNSUPPORTED"),
    (dict(lmax_sh=4), "UNSUPPORTED"),
    (dict(n_basis=17), "UNSUPPORTED"),
    (dict(n_basis=1), "INVALID_ARG"),
    (dict(r_hi=-1.0), "INVALID_ARG"),
    (dict(instructions=[(0, 1, 0)]), "INVALID_PATH"),      # 0e x Y1 -> 0e violates Eq. 5
    (dict(instructions=[(0, 0, 0), (0, 0, 0)]), "INVALID_ARG"),
    (dict(instructions=[(5, 0, 0)]), "INVALID_ARG"),
    (dict(mode="uvu", irreps_out="8x0e"), "INVALID_PATH"),  # uvu needs C_out == C_in
    (dict(box=(1.0, 0.0, 1.0)), "INVALID_ARG"),
])
def test_invalid_specs(kwargs, status):
    base = dict(irreps_in="4x0e+4x1o", irreps_out="4x0e+4x1o", lmax_sh=2, mode="uvw", radial="gaussian",
                n_basis=4, r_lo=0.0, r_hi=5.0)
    base.update(kwargs)
    with pytest.raises(etpc.EtpcError) as ei:
        etpc.Plan(**base)
    assert ei.value.name == status


def test_gemm_precision_codes():
    """fp32, bf16 and fp16 channel GEMMs are accepted; any other code is an argument error."""
    base = dict(irreps_in="4x0e+4x1o", irreps_out="4x0e+4x1o", lmax_sh=2)
    for prec in ("fp32", "bf16", "fp16"):
        etpc.Plan(**base, gemm_precision=prec)
    spec = etpc.Plan(**base).spec
    spec.gemm_precision = 3
    with pytest.raises(etpc.EtpcError) as ei:
        _binding.etpc_plan_create(spec)
    assert ei.value.name == "INVALID_ARG"


def test_workspace_is_node_sized():
    """Workspace grows with N; with E only by the 12 B/edge position adjoint, one copy per
    concurrent launch lane (backward, and double backward with its d/dpos output)."""
    plan = plan_from_config(CONFIGS["cfg4_d16"])
    n = 32768
    f = [etpc.etpc_workspace_size(plan, etpc.PASS_FWD, n, e) for e in (500000, 2000000, 16000000)]
    assert f[0] == f[1] == f[2]
    lanes = min(2, plan.info()["n_paths"])   # one edge-adjoint copy per concurrent lane (two)
    b = [etpc.etpc_workspace_size(plan, etpc.PASS_BWD, n, int(e)) for e in (5e5, 2e6)]
    assert abs((b[1] - b[0]) - 12 * lanes * 1.5e6) < 4096
    d = [etpc.etpc_workspace_size(plan, etpc.PASS_DBL, n, int(e)) for e in (5e5, 2e6)]
    assert abs((d[1] - d[0]) - 12 * lanes * 1.5e6) < 4096


def test_csr_workspace_size_and_argument_errors():
    assert etpc.etpc_csr_workspace_size(10, 100) > 0
    with pytest.raises(etpc.EtpcError):
        etpc.etpc_csr_workspace_size(-1, 10)


def test_workspace_budget():
    """budget = 0 gives the full (one chunk) size; a budget caps the node-state scratch at the
    largest chunk that fits; below one node's state (plus the per-edge adjoint) the call is
    refused with the minimum reported."""
    plan = plan_from_config(CONFIGS["cfg2"])
    n, e = 4096, 214980
    for pass_ in (etpc.PASS_FWD, etpc.PASS_BWD, etpc.PASS_DBL):
        full = etpc.etpc_workspace_size(plan, pass_, n, e)
        assert etpc.etpc_workspace_size(plan, pass_, n, e, budget=full) == full
        assert etpc.etpc_workspace_size(plan, pass_, n, e, budget=4 * full) == full
        for mib in (512, 256, 128):
            b = etpc.etpc_workspace_size(plan, pass_, n, e, budget=mib << 20)
            assert b <= min(full, mib << 20)
            # monotone: a larger budget never gives a smaller workspace
            assert etpc.etpc_workspace_size(plan, pass_, n, e, budget=2 * (mib << 20)) >= b
        with pytest.raises(etpc.EtpcError) as ei:
            etpc.etpc_workspace_size(plan, pass_, n, e, budget=1024)
        assert ei.value.name == "WORKSPACE" and "minimum" in str(ei.value)
    # an empty graph needs no chunking
    assert etpc.etpc_workspace_size(plan, etpc.PASS_FWD, 0, 0, budget=1) >= 0


def test_lanes_belong_to_the_plan():
    """Concurrent launch lanes are a plan field (no process-wide setting): 0 = default (2),
    1 serializes, anything else is refused; a one-lane plan keeps one edge-adjoint copy."""
    base = dict(irreps_in="4x0e+4x1o", irreps_out="4x0e+4x1o", lmax_sh=2)
    for lanes in (0, 1, 2):
        etpc.Plan(**base, lanes=lanes)
    for bad in (-1, 3, 99):
        with pytest.raises(etpc.EtpcError) as ei:
            etpc.Plan(**base, lanes=bad)
        assert ei.value.name == "INVALID_ARG"
    cfg = CONFIGS["cfg4_d16"]
    two = plan_from_config(cfg)
    one = etpc.Plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.radial, cfg.n_basis, cfg.r_lo,
                    cfg.r_hi, cfg.poly_p, box=cfg.box, lanes=1)
    n = 32768
    b2 = [etpc.etpc_workspace_size(two, etpc.PASS_BWD, n, int(e)) for e in (5e5, 2e6)]
    b1 = [etpc.etpc_workspace_size(one, etpc.PASS_BWD, n, int(e)) for e in (5e5, 2e6)]
    assert abs((b2[1] - b2[0]) - 24 * 1.5e6) < 4096 and abs((b1[1] - b1[0]) - 12 * 1.5e6) < 4096
    assert not hasattr(etpc.lib, "etpc_set_lanes")


def test_plan_path_argument_errors():
    plan = plan_from_config(CONFIGS["cfg1"])
    n = plan.info()["n_paths"]
    lib = etpc.lib
    assert lib.etpc_plan_path(plan.handle, n, None, None, None, None, None, None, None, None, None, None) == 1
    assert lib.etpc_plan_path(plan.handle, -1, None, None, None, None, None, None, None, None, None, None) == 1
    assert lib.etpc_plan_path(None, 0, None, None, None, None, None, None, None, None, None, None) == 1
    assert lib.etpc_plan_path(plan.handle, 0, None, None, None, None, None, None, None, None, None, None) == 0


def test_missing_library_fails_loudly(tmp_path):
    """With the HIP library absent the package refuses to import (there is no CPU path)."""
    import os
    import subprocess
    import sys
    env = dict(os.environ, ETPC_LIBRARY=str(tmp_path / "absent" / "libetpc.so"))
    r = subprocess.run([sys.executable, "-c", "import equivariant_gnn_tensor_amd"], cwd=os.path.dirname(
        os.path.dirname(os.path.abspath(__file__))), env=env, capture_output=True, text=True)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr


def _radius_status(n, pos, cutoff, box, cap=0):
    import ctypes as C
    ne = C.c_int64(-1)
    box_c = None if box is None else (C.c_float * 3)(*box)
    st = etpc.lib.etpc_radius_graph(n, pos, cutoff, box_c, cap, None, None, C.byref(ne), None, 0, None)
    return st, ne.value


def test_radius_graph_argument_errors():
    """Validated on the host before anything is enqueued."""
    import ctypes as C
    fake = 4096   # never dereferenced: every case below fails validation first
    assert _radius_status(4, fake, 0.0, None)[0] == 1          # cutoff must be positive
    assert _radius_status(4, fake, float("nan"), None)[0] == 1
    assert _radius_status(4, fake, 3.0, (5.0, 8.0, 8.0))[0] == 1   # box below 2 r_c
    assert _radius_status(4, fake, 1.0, (5.0, 0.0, 8.0))[0] == 1
    assert _radius_status(-1, fake, 1.0, None)[0] == 1
    assert _radius_status(1 << 30, fake, 1.0, None)[0] == 5
    assert _radius_status(4, None, 1.0, None)[0] == 1          # null positions
    assert _radius_status(0, None, 1.0, None) == (0, 0)       # empty point set: no edges
    st = etpc.lib.etpc_radius_graph(4, fake, 1.0, None, 0, None, None, None, None, 0, None)
    assert st == 1                                             # null n_edges
    assert "n_edges" in etpc.lib.etpc_last_error().decode()
    assert _radius_status(4, fake, 1.0, None, cap=8)[0] == 1   # null outputs with capacity


def test_radius_graph_workspace_grows_with_capacity():
    a = etpc.etpc_radius_graph_workspace_size(1000, 0)
    b = etpc.etpc_radius_graph_workspace_size(1000, 100000)
    assert a > 36 * 1000 and 16 * 100000 <= b - a <= 17 * 100000


def test_layout_convert_argument_errors():
    plan = plan_from_config(CONFIGS["cfg2"])
    lib = etpc.lib
    assert lib.etpc_layout_convert(None, 0, 0, 4, 4096, 8192, None) == 1
    assert lib.etpc_layout_convert(plan.handle, 2, 0, 4, 4096, 8192, None) == 1
    assert lib.etpc_layout_convert(plan.handle, 0, 5, 4, 4096, 8192, None) == 1
    assert lib.etpc_layout_convert(plan.handle, 0, 0, 4, 4096, 4096 + 16, None) == 1   # overlap
    assert "overlap" in lib.etpc_last_error().decode()
    assert lib.etpc_layout_convert(plan.handle, 1, 1, 0, None, None, None) == 0       # no rows


def test_degree_order_argument_errors():
    assert etpc.etpc_degree_order_workspace_size(4096) > 0
    with pytest.raises(etpc.EtpcError):
        etpc.etpc_degree_order_workspace_size(-1)
    lib = _binding.lib
    assert lib.etpc_degree_order(0, None, 0, None, None, 0, None) == 0      # empty: nothing to do
    assert lib.etpc_degree_order(-1, None, 0, None, None, 0, None) != 0
    assert lib.etpc_degree_order(8, None, 0, None, None, 0, None) != 0      # null arrays
    assert lib.etpc_degree_order(8, 16, -1, 16, 16, 1 << 20, None) != 0    # negative window
    assert "window" in etpc.lib.etpc_last_error().decode().lower()
    # a workspace too small is refused before anything is launched
    st = lib.etpc_degree_order(8, 16, 0, 16, 16, 8, None)
    assert st != 0 and "workspace" in etpc.lib.etpc_last_error().decode().lower()


def test_spatial_and_based_order_argument_errors():
    """The spatial order and the degree order along a base sequence check their arguments
    on the host before any launch (placeholder pointers are never dereferenced)."""
    import ctypes as C
    lib = _binding.lib
    assert etpc.etpc_spatial_order_workspace_size(4096) > 0
    with pytest.raises(etpc.EtpcError):
        etpc.etpc_spatial_order_workspace_size(-1)
    assert lib.etpc_spatial_order(0, None, None, None, None, 0, None) == 0     # empty: nothing to do
    assert lib.etpc_spatial_order(-1, None, None, None, None, 0, None) != 0
    assert lib.etpc_spatial_order(8, None, None, None, None, 0, None) != 0     # null arrays
    bad_box = (C.c_float * 3)(10.0, 0.0, 10.0)
    assert lib.etpc_spatial_order(8, 16, bad_box, 16, 16, 1 << 20, None) != 0
    assert "box" in lib.etpc_last_error().decode()
    good_box = (C.c_float * 3)(10.0, 10.0, 10.0)
    assert lib.etpc_spatial_order(8, 16, good_box, 16, 16, 8, None) != 0      # workspace too small
    assert "workspace" in lib.etpc_last_error().decode().lower()
    assert lib.etpc_degree_order_within(0, None, 0, None, None, None, 0, None) == 0
    assert lib.etpc_degree_order_within(8, 16, 0, None, 16, 16, 1 << 20, None) != 0   # null base
    assert lib.etpc_degree_order_within(8, 16, -1, 16, 16, 16, 1 << 20, None) != 0    # negative window
    assert lib.etpc_degree_order_within(8, 16, 0, 16, 16, 16, 8, None) != 0           # workspace too small
    assert "workspace" in lib.etpc_last_error().decode().lower()


def test_noalloc_forward_refuses_oversized_state():
    """The allocation-free forward refuses, on the host and before any HIP call, a plan whose
    single-receiver state exceeds its fixed 128 MiB scratch.  The size is confirmed through
    the workspace query first, so the call below can only take the refusal path (its
    pointers are placeholders that nothing dereferences)."""
    import ctypes as C
    huge = etpc.Plan("600000x0e+600000x1o", "4x0e+4x1o", 1, "uvw", "gaussian", 16, 0.0, 5.0)
    # the smallest forward workspace of any schedule: a one-byte budget is refused with it
    one_receiver = C.c_size_t()
    st = etpc.lib.etpc_workspace_size(huge.handle, etpc.PASS_FWD, 1, 0, 1, C.byref(one_receiver))
    assert st == 4 and one_receiver.value > (128 << 20)
    g = _binding.etpc_graph()
    g.n_nodes, g.n_edges = 1, 0
    g.rowptr = g.s_rowptr = 4096
    st = etpc.lib.etpc_forward_noalloc(huge.handle, C.byref(g), 4096, 4096, 4096, 4096, None)
    assert st == 4 and "fixed scratch" in etpc.lib.etpc_last_error().decode()
