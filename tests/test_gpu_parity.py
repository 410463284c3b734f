"""GPU parity: HIP path (through the C ABI) vs the float64 oracle.

Tolerance: max|d| / max|ref| <= 1e-4 for forward and backward, 1e-3 for double
backward, per output tensor (fp32 arithmetic on the GPU, float64 oracle).
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import conv
from oracle.csr import csr_build
from tests.gpu_helpers import make_case, note, rel_err
from tests.planner_helpers import plan_from_config
from workloads import CONFIGS, small_variant

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_DBL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import equivariant_gnn_tensor_amd  # noqa: F401  (fails loudly if the library is missing)


def _etpc():
    import equivariant_gnn_tensor_amd as etpc
    return etpc


# ---------------------------------------------------------------- CSR
def _csr_cases(rng):
    yield "empty", 5, np.zeros(0, np.int32), np.zeros(0, np.int32)
    yield "single-node-no-edges", 1, np.zeros(0, np.int32), np.zeros(0, np.int32)
    yield "all-into-one", 7, rng.integers(0, 7, 3000).astype(np.int32), np.full(3000, 3, np.int32)
    yield "duplicates", 4, np.array([1, 1, 1, 0, 2, 2], np.int32), np.array([0, 0, 0, 1, 0, 0], np.int32)
    for n, e in [(100, 5000), (70000, 300000), (300, 20000)]:
        yield f"random-{n}-{e}", n, rng.integers(0, n, e).astype(np.int32), rng.integers(0, n, e).astype(np.int32)


def test_csr_bit_exact():
    etpc = _etpc()
    rng = np.random.default_rng(5)
    for name, n, src, dst in _csr_cases(rng):
        note(f"csr {name} n={n} e={len(src)}")
        g = etpc.etpc_csr_build(n, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
        want = csr_build(n, src, dst)
        got = dict(rowptr=g.rowptr, col=g.col, eid=g.eid, s_rowptr=g.s_rowptr, s_col=g.s_col, s_slot=g.s_slot)
        for k, v in want.items():
            assert np.array_equal(got[k].cpu().numpy(), v), (name, k)


def test_graph_validate_accepts_built_and_rejects_broken():
    etpc = _etpc()
    rng = np.random.default_rng(6)
    n, e = 50, 400
    src = rng.integers(0, n, e).astype(np.int32)
    dst = (src + rng.integers(1, n, e).astype(np.int32)) % n
    g = etpc.etpc_csr_build(n, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    etpc.etpc_graph_validate(g)
    bad_col = g.col.clone()
    bad_col[3] = n + 5                       # out of range, caught on the host side of the check
    gb = etpc.Graph(n, g.rowptr, bad_col, g.s_rowptr, g.s_col, g.s_slot)
    with pytest.raises(etpc.EtpcError):
        etpc.etpc_graph_validate(gb)
    bad_slot = g.s_slot.clone()
    bad_slot[[0, 1]] = bad_slot[[1, 0]]      # breaks the stable order within a sender row or the mapping
    gs = etpc.Graph(n, g.rowptr, g.col, g.s_rowptr, g.s_col, bad_slot)
    with pytest.raises(etpc.EtpcError):
        etpc.etpc_graph_validate(gs)


# ---------------------------------------------------------------- forward / backward parity
FWD_CASES = [
    ("cfg1", None, None),
    ("cfg2", 256, None),
    ("cfg3", 256, None),
    ("cfg4_d16", 600, None),
    ("cfg4_d64", 300, None),
    ("cfg5", 256, None),
    ("cfg6_b4", None, None),     # block-diagonal batch of four 128-atom cells
]


def _cfg(name, n, d):
    return CONFIGS[name] if n is None else small_variant(name, n, d)


@pytest.mark.parametrize("name,n,d", FWD_CASES)
def test_forward_parity(name, n, d):
    etpc = _etpc()
    cfg = _cfg(name, n, d)
    note(f"forward {cfg.name} N={cfg.n_nodes}")
    c = make_case(cfg)
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    torch.cuda.synchronize()
    ref = conv.forward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst)
    err = rel_err(z, ref)
    note(f"forward {cfg.name} rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("name,n,d", [c for c in FWD_CASES if c[0] != "cfg1"])
def test_backward_parity(name, n, d):
    etpc = _etpc()
    cfg = _cfg(name, n, d)
    note(f"backward {cfg.name} N={cfg.n_nodes}")
    c = make_case(cfg)
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    rx, rw, rp = conv.backward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst, c.wl.z_bar)
    errs = (rel_err(xb, rx), rel_err(wb, rw), rel_err(pb, rp))
    note(f"backward {cfg.name} rel err x {errs[0]:.2e} w {errs[1]:.2e} pos {errs[2]:.2e}")
    assert max(errs) <= TOL
    # subsets of outputs give the same values (kernel variants may differ in the last bits)
    xb2, _, pb2 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, want=("x", "pos"))
    _, _, pb3 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, want=("pos",))
    _, wb4, _ = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, want=("w",))
    for got, ref in ((xb2, xb), (pb2, pb), (pb3, pb), (wb4, wb)):
        assert rel_err(got, ref.double().cpu().numpy()) <= 1e-6


@pytest.mark.parametrize("name,n", [("cfg5", 256), ("cfg3", 128)])
def test_double_backward_force_loss(name, n):
    """L = <c, F> with F = -pos_bar: outputs d/dz_bar, d/dx, d/dW along pos_dot = -c."""
    etpc = _etpc()
    cfg = small_variant(name, n)
    note(f"double backward {cfg.name} N={cfg.n_nodes}")
    c = make_case(cfg)
    fc = c.wl.force_c if c.wl.force_c is not None else np.random.default_rng(9).standard_normal(
        (cfg.n_nodes, 3)).astype(np.float32)
    pos_dot = torch.from_numpy(-fc).cuda()
    gz, gx, gw, gp = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pos_dot)
    torch.cuda.synchronize()
    rz, rx, rw, rp = conv.double_backward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst, c.wl.z_bar,
                                          pos_dot=-fc.astype(np.float64))
    errs = (rel_err(gz, rz), rel_err(gx, rx), rel_err(gw, rw), rel_err(gp, rp))
    note(f"double backward {cfg.name} rel err z_bar {errs[0]:.2e} x {errs[1]:.2e} w {errs[2]:.2e} pos {errs[3]:.2e}")
    assert max(errs) <= TOL_DBL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n", [("cfg5", 128), ("cfg3", 128)])
def test_double_backward_all_cotangents(name, n):
    """Each cotangent alone, and all three at once.  The double backward is linear in
    (x_dot, w_dot, pos_dot), so the reference for all three is the fp64 sum of the three
    single-cotangent oracle results (three oracle calls instead of four: the oracle's
    double backward of workload 3 takes over a minute on the host)."""
    etpc = _etpc()
    cfg = small_variant(name, n)
    note(f"double backward (all cotangents) {cfg.name}")
    c = make_case(cfg)
    rng = np.random.default_rng(11)
    xd = rng.standard_normal(c.wl.x.shape).astype(np.float32)
    wd = rng.standard_normal(c.wl.w.shape).astype(np.float32)
    pd = rng.standard_normal(c.wl.pos.shape).astype(np.float32)
    zb = rng.standard_normal((cfg.n_nodes, c.spec.plan.z_dim)).astype(np.float32)
    T = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    gall = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, T(zb), x_dot=T(xd), w_dot=T(wd),
                                     pos_dot=T(pd))
    torch.cuda.synchronize()
    rsum = None
    for kw, ref_kw in ((dict(x_dot=T(xd)), dict(x_dot=xd)), (dict(w_dot=T(wd)), dict(w_dot=wd)),
                       (dict(pos_dot=T(pd)), dict(pos_dot=pd))):
        got = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, T(zb), **kw)
        ref = conv.double_backward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst, zb, **ref_kw)
        ref = [np.asarray(r, dtype=np.float64) for r in ref]
        rsum = ref if rsum is None else [a + b for a, b in zip(rsum, ref)]
        for g, r in zip(got, ref):
            if np.abs(r).max() == 0:
                assert torch.count_nonzero(g) == 0
            else:
                assert rel_err(g, r) <= TOL_DBL
        note(f"  {list(ref_kw)[0]} alone: ok")
    errs = tuple(rel_err(g, r) for g, r in zip(gall, rsum))
    note(f"double backward all {cfg.name} rel err {errs}")
    assert max(errs) <= TOL_DBL


@pytest.mark.parametrize("name,n", [("cfg2", 256), ("cfg2", None), ("cfg3", 128)])
def test_dispatch_order_is_bit_identical(name, n):
    """Dispatching nodes in decreasing degree (the graph's s_order and r_order, along the
    node index or along the spatial order of the positions) changes only which workgroup
    takes which node: forward, backward and double backward are bit-identical to the
    index-order dispatch (the small graph takes the edge-split
    launches, the full one the plain ones; workload 3 is the channelwise forward)."""
    etpc = _etpc()
    cfg = CONFIGS[name] if n is None else small_variant(name, n)
    c = make_case(cfg)
    assert c.graph.s_order is not None and c.graph.r_order is not None
    g0 = c.graph.without_order()
    note(f"dispatch order {cfg.name}")
    za = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    zb = etpc.etpc_forward(c.plan, g0, c.x, c.pos, c.w)
    a = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    b = etpc.etpc_backward(c.plan, g0, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    assert torch.equal(za, zb)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # the same along the spatial order of the positions
    box = (cfg.box,) * 3 if cfg.box else None
    gsp = etpc.etpc_csr_build(cfg.n_nodes, torch.from_numpy(c.wl.src).cuda(), torch.from_numpy(c.wl.dst).cuda(),
                              pos=c.pos, box=box)
    etpc.etpc_graph_validate(gsp)
    zs = etpc.etpc_forward(c.plan, gsp, c.x, c.pos, c.w)
    s_ = etpc.etpc_backward(c.plan, gsp, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    assert torch.equal(zs, zb)
    for u, v in zip(s_, b):
        assert torch.equal(u, v)
    if n is not None and name == "cfg2":
        rng = np.random.default_rng(5)
        kw = dict(x_dot=torch.from_numpy(rng.standard_normal(c.wl.x.shape).astype(np.float32)).cuda(),
                  pos_dot=torch.from_numpy(rng.standard_normal(c.wl.pos.shape).astype(np.float32)).cuda())
        a = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, **kw)
        b = etpc.etpc_double_backward(c.plan, g0, c.x, c.pos, c.w, c.z_bar, **kw)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v)


def test_determinism_and_chunked_workspace():
    etpc = _etpc()
    cfg = small_variant("cfg2", 256)
    c = make_case(cfg)
    note("determinism / chunking")
    z1 = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    z2 = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    b1 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    b2 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    assert torch.equal(z1, z2) and all(torch.equal(a, b) for a, b in zip(b1, b2))
    # a workspace a fifth of the full size runs the bounded schedule (receiver / sender
    # chunks, fewer split-K partial slots): the same values up to summation order, and
    # deterministic for that workspace
    full = etpc.etpc_workspace_size(c.plan, etpc.PASS_FWD, cfg.n_nodes, c.graph.n_edges)
    ws = torch.empty(full // 5, dtype=torch.uint8, device="cuda")
    z3 = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, ws=ws)
    z4 = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, ws=ws)
    assert torch.equal(z3, z4) and rel_err(z3, z1.double().cpu().numpy()) < 1e-5
    fullb = etpc.etpc_workspace_size(c.plan, etpc.PASS_BWD, cfg.n_nodes, c.graph.n_edges)
    wsb = torch.empty(fullb // 3, dtype=torch.uint8, device="cuda")
    b3 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, ws=wsb)
    b4 = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, ws=wsb)
    assert all(torch.equal(u, v) for u, v in zip(b3, b4))
    for u, v in zip(b3, b1):
        assert rel_err(u, v.double().cpu().numpy()) < 1e-5
    with pytest.raises(etpc.EtpcError) as ei:
        etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.name == "WORKSPACE"


def test_isolated_nodes_and_empty_graph():
    etpc = _etpc()
    cfg = dataclasses.replace(CONFIGS["cfg1"], n_nodes=64)
    c = make_case(cfg)
    note("empty graph")
    empty = etpc.etpc_csr_build(cfg.n_nodes, torch.zeros(0, dtype=torch.int32, device="cuda"),
                                torch.zeros(0, dtype=torch.int32, device="cuda"))
    z = etpc.etpc_forward(c.plan, empty, c.x, c.pos, c.w)
    zb = torch.randn(cfg.n_nodes, c.plan.info()["z_dim"], device="cuda")
    xb, wb, pb = etpc.etpc_backward(c.plan, empty, c.x, c.pos, c.w, zb)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z) == 0 and torch.count_nonzero(xb) == 0
    assert torch.count_nonzero(wb) == 0 and torch.count_nonzero(pb) == 0


# ---------------------------------------------------------------- ragged channel counts
# Multiplicities below 4 (slots narrower than a matrix-core lane group), odd widths, and
# widths above one wave with a ragged last tile; 12 radial bases (partial basis quads).
RAGGED = [
    ("uvw_small", "cfg5", dict(irreps_in="3x0e+1x1o+2x2e+1x3o", irreps_out="2x0e+1x1o+5x2e+1x3o")),
    ("uvw_wide", "cfg5", dict(irreps_in="70x0e+65x1o", irreps_out="33x0e+66x1o+1x2e", lmax_sh=2, n_basis=12)),
    ("uvu_small", "cfg3", dict(irreps_in="1x0e+3x1o+2x2e+5x3o")),
    ("uvu_wide", "cfg3", dict(irreps_in="70x0e+129x1o", lmax_sh=2, n_basis=12)),
]


@pytest.mark.parametrize("tag,base,kw", RAGGED, ids=[r[0] for r in RAGGED])
def test_ragged_channels(tag, base, kw):
    etpc = _etpc()
    cfg = dataclasses.replace(small_variant(base, 128), name=f"ragged_{tag}", **kw)
    if cfg.mode == "uvu":
        cfg = dataclasses.replace(cfg, irreps_out="0e+1o+2e+3o" if cfg.lmax_sh == 3 else "0e+1o+2e")
    note(f"ragged {tag}: {cfg.irreps_in} -> {cfg.irreps_out}")
    c = make_case(cfg)
    wl = c.wl
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    rz = conv.forward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    rx, rw, rp = conv.backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar)
    errs = [rel_err(z, rz), rel_err(xb, rx), rel_err(wb, rw), rel_err(pb, rp)]
    note(f"  fwd/bwd rel err {['%.2e' % e for e in errs]}")
    assert max(errs) <= TOL
    rng = np.random.default_rng(5)
    pd = rng.standard_normal(wl.pos.shape).astype(np.float32)
    xd = rng.standard_normal(wl.x.shape).astype(np.float32)
    T = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    gz, gx, gw, gp = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, x_dot=T(xd),
                                               pos_dot=T(pd))
    torch.cuda.synchronize()
    r = conv.double_backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, x_dot=xd, pos_dot=pd)
    derrs = [rel_err(gz, r[0]), rel_err(gx, r[1]), rel_err(gw, r[2]), rel_err(gp, r[3])]
    note(f"  double backward rel err {['%.2e' % e for e in derrs]}")
    assert max(derrs) <= TOL_DBL


# ---------------------------------------------------------------- HIP graph capture
@pytest.mark.parametrize("name,n", [("cfg1", None), ("cfg5", 128)])
def test_graph_capture_replays_match_eager(name, n):
    """A captured forward + backward (+ double backward) step replays bit-identically to the
    eager step, several times, with eager work and synchronizations between replays."""
    etpc = _etpc()
    cfg = CONFIGS[name] if n is None else small_variant(name, n)
    note(f"graph capture {cfg.name}")
    c = make_case(cfg)
    info = c.plan.info()
    N = cfg.n_nodes
    dev = c.x.device
    ws = {p: torch.empty(etpc.etpc_workspace_size(c.plan, p, N, c.wl.n_edges), dtype=torch.uint8, device=dev)
          for p in (etpc.PASS_FWD, etpc.PASS_BWD, etpc.PASS_DBL)}
    z = torch.empty(N, info["z_dim"], device=dev)
    outs = (torch.empty(N, info["x_dim"], device=dev), torch.empty(info["w_numel"], device=dev),
            torch.empty(N, 3, device=dev))
    pd = torch.from_numpy(np.random.default_rng(3).standard_normal((N, 3)).astype(np.float32)).to(dev)
    douts = tuple(torch.empty_like(t) for t in (z, outs[0], outs[1], outs[2]))

    def step():
        etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, z=z, ws=ws[etpc.PASS_FWD])
        etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, outs=outs, ws=ws[etpc.PASS_BWD])
        etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pd, outs=douts,
                                  ws=ws[etpc.PASS_DBL])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (z, *outs, *douts)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (z, *outs, *douts):
            t.fill_(float("nan"))          # eager work between replays; stale values would show
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((z, *outs, *douts), ref):
            assert torch.equal(got, want), f"replay {rep} differs from the eager step"
    note(f"graph capture {cfg.name}: 3 replays bit-identical")


def test_concurrent_schedules_are_deterministic_and_agree():
    """Lanes and the post stream change only where work runs, not what it computes:
    repeated calls are bit-identical, forward / x_bar / W_bar equal the serialized
    schedule bit for bit, pos_bar (per-lane edge-adjoint copies summed in a fixed order)
    to 1e-6; calls issued on a non-default stream give the same results."""
    etpc = _etpc()
    cfg = small_variant("cfg5", 256)
    c = make_case(cfg)
    note(f"schedules {cfg.name}")
    pos_dot = torch.from_numpy(-c.wl.force_c).cuda()
    serial_plan = plan_from_config(cfg, lanes=1)

    def run(stream=None, plan=c.plan):
        z = etpc.etpc_forward(plan, c.graph, c.x, c.pos, c.w, stream=stream)
        b = etpc.etpc_backward(plan, c.graph, c.x, c.pos, c.w, c.z_bar, stream=stream)
        d = etpc.etpc_double_backward(plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pos_dot, stream=stream)
        return [z, *b, *d]

    first = run()
    for _ in range(3):
        again = run()
        assert all(torch.equal(a, b) for a, b in zip(first, again))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        on_side = run(stream=side)
    side.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(first, on_side))
    serial = run(plan=serial_plan)
    torch.cuda.synchronize()
    z, xb, wb, pb = first[:4]
    assert torch.equal(z, serial[0]) and torch.equal(xb, serial[1]) and torch.equal(wb, serial[2])
    assert rel_err(pb, serial[3].double().cpu().numpy()) < 1e-6
    for a, b in zip(first[4:], serial[4:]):
        if a is not None:
            assert rel_err(a, b.double().cpu().numpy()) < 1e-5
    # a third of the full workspace: the double backward runs the block pipeline over
    # several sender chunks
    full = etpc.etpc_workspace_size(c.plan, etpc.PASS_DBL, cfg.n_nodes, c.graph.n_edges)
    ws = torch.empty(full // 3, dtype=torch.uint8, device="cuda")
    chunked = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pos_dot, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip(chunked, first[4:]):
        if a is not None:
            assert rel_err(a, b.double().cpu().numpy()) < 1e-5


def test_binding_rejects_wrong_shapes_before_launch():
    """The binding compares every dense operand with the plan and the graph before calling
    the library, so a wrong-sized tensor is an argument error, not an out-of-bounds access."""
    etpc = _etpc()
    cfg = CONFIGS["cfg1"]
    c = make_case(cfg)
    N = cfg.n_nodes
    info = c.plan.info()
    bad = [
        dict(x=c.x[:-1]), dict(pos=c.pos[:, :2]), dict(w=c.w[:-3]),
    ]
    for kw in bad:
        args = dict(x=c.x, pos=c.pos, w=c.w)
        args.update(kw)
        with pytest.raises(ValueError):
            etpc.etpc_forward(c.plan, c.graph, args["x"], args["pos"], args["w"])
    with pytest.raises(ValueError):
        etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, z=torch.empty(N, info["z_dim"] - 1, device="cuda"))
    zb = torch.randn(N, info["z_dim"], device="cuda")
    with pytest.raises(ValueError):
        etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, zb[:, 1:])
    with pytest.raises(ValueError):
        etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, zb,
                           outs=(torch.empty(N, info["x_dim"], device="cuda"), torch.empty(5, device="cuda"), None))
    with pytest.raises(ValueError):
        etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, zb, pos_dot=torch.zeros(N + 1, 3, device="cuda"))
    with pytest.raises(ValueError):
        etpc.etpc_layout_convert(c.plan, "in", "to_mul_ir", c.x, out=torch.empty(N, info["x_dim"] + 1, device="cuda"))
    with pytest.raises(ValueError):
        etpc.etpc_csr_build(N, torch.zeros(4, dtype=torch.int32, device="cuda"),
                            torch.zeros(3, dtype=torch.int32, device="cuda"))
    # the correct shapes still run, also on a non-default stream with library-allocated
    # outputs and workspace (allocated on that stream)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w, stream=side)
    side.synchronize()
    z0 = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    torch.cuda.synchronize()
    assert torch.equal(z, z0)
