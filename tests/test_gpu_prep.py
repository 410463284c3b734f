"""GPU parity of the graph-preparation steps against the oracle (bit-exact: integer output
and pure data movement).

Radius graph: the edge list (receiver-major, senders ascending) must equal the brute-force
oracle's exactly.  Cases: the workloads' own densities (0.1 atoms / A^3, cutoff 5 A,
periodic cubes of 4096 and 16384 atoms), open boundaries, ragged sizes, boxes with fewer
than three cells per axis, atoms outside the box, coincident atoms and a pair exactly at
the cutoff, far-apart clusters (the cell grid is widened to its cap), one and two atoms,
rows longer than one wavefront (the global-sort path), and the capacity error.  At 65,536 atoms the oracle checks sampled receivers' rows, and
the whole list is checked for order, symmetry and validity.

Degree order: the dispatch orders (decreasing degree, ties by index; over all nodes or
in aligned windows) equal the oracle's stable sorts bit for bit; etpc_graph_validate
accepts the graph's orders and rejects wrong ones.  Spatial order: the Morton sort of the
positions and the degree orders along it equal a direct numpy sort (a dispatch heuristic,
not part of the method, so the reference lives here rather than in the oracle).

Layout: mul_ir <-> ir_mul of the workloads' input and output irreps, ragged row counts,
round trips.
"""
import numpy as np
import pytest
import torch

from oracle import csr as ocsr
from oracle import layout as olayout
from oracle import radius as oradius
from tests.gpu_helpers import note
from tests.planner_helpers import plan_from_config
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _etpc():
    import equivariant_gnn_tensor_amd as etpc
    return etpc


def _uniform(n, L, seed):
    return np.random.default_rng(seed).uniform(0.0, L, size=(n, 3)).astype(np.float32)


def _run(pos, cutoff, box):
    etpc = _etpc()
    src, dst = etpc.etpc_radius_graph(torch.from_numpy(np.ascontiguousarray(pos)).cuda(), cutoff, box=box)
    torch.cuda.synchronize()
    return src.cpu().numpy(), dst.cpu().numpy()


def _assert_same(pos, cutoff, box, what):
    note(f"radius graph {what}: N={pos.shape[0]} cutoff={cutoff} box={box}")
    gs, gd = _run(pos, cutoff, box)
    rs, rd = oradius.radius_graph(pos, cutoff, box)
    note(f"  edges gpu {gs.size} oracle {rs.size}")
    assert gs.size == rs.size
    assert np.array_equal(gd, rd) and np.array_equal(gs, rs)
    return gs.size


def _box_side(n, density=0.1):
    return float((n / density) ** (1.0 / 3.0))


@pytest.mark.parametrize("n", [4096, 16384])
def test_radius_graph_workload_density(n):
    L = _box_side(n)
    pos = _uniform(n, L, 100 + n)
    e = _assert_same(pos, 5.0, (L, L, L), f"periodic density 0.1, {n} atoms")
    assert e > 40 * n   # about 52 neighbours per atom at this density


def test_radius_graph_open_and_ragged():
    pos = _uniform(1237, 30.0, 3)
    _assert_same(pos, 4.0, None, "open, ragged")
    pos = np.random.default_rng(4).normal(0.0, 3.0, size=(777, 3)).astype(np.float32)
    _assert_same(pos, 2.5, None, "open, Gaussian cloud")


def test_radius_graph_few_cells_and_wrapping():
    # L = 2.4 r_c: two cells per axis, every cell visited once
    pos = _uniform(300, 12.0, 5)
    _assert_same(pos, 5.0, (12.0, 12.0, 12.0), "two cells per axis")
    # L = 2 r_c exactly: one cell per axis
    _assert_same(_uniform(120, 10.0, 6), 5.0, (10.0, 10.0, 10.0), "one cell per axis")
    # atoms outside the box and non-cubic boxes
    pos = (_uniform(500, 1.0, 7) * np.array([60.0, 20.0, 33.0], np.float32)
           - np.array([25.0, 8.0, 40.0], np.float32)).astype(np.float32)
    _assert_same(pos, 4.0, (20.0, 10.0, 11.0), "outside the box, orthorhombic")


def test_radius_graph_degenerate_pairs():
    pos = _uniform(200, 15.0, 8)
    pos[10] = pos[11]                          # coincident atoms: no edge between them
    pos[20] = pos[21] + np.array([3.0, 0.0, 0.0], np.float32)
    pos = np.concatenate([pos, np.array([[0, 0, 0], [3, 0, 0], [0, 0, 0]], np.float32)])
    _assert_same(pos, 3.0, None, "coincident and at-cutoff pairs")
    lat = np.array(np.meshgrid(*[np.arange(6)] * 3, indexing="ij"), np.float32).reshape(3, -1).T
    n = _assert_same(lat, 1.5, (6.0, 6.0, 6.0), "simple cubic lattice, 18 neighbours")
    assert n == 18 * 216


def test_radius_graph_far_clusters_and_tiny_sets():
    a = _uniform(150, 8.0, 9)
    b = _uniform(150, 8.0, 10) + np.float32(1e4)
    _assert_same(np.concatenate([a, b]).astype(np.float32), 3.0, None, "far-apart clusters")
    _assert_same(np.zeros((1, 3), np.float32), 2.0, None, "one atom")
    _assert_same(np.array([[0, 0, 0], [1, 1, 1]], np.float32), 2.0, (5.0, 5.0, 5.0), "two atoms")
    _assert_same(_uniform(64, 4.0, 11), 10.0, None, "all atoms in one cell")


def test_radius_graph_rows_longer_than_a_wavefront():
    """Rows of more than 64 edges take the global-sort path, shorter ones the per-row sort."""
    dense = _uniform(300, 6.0, 15)                     # ~299 neighbours each
    n = _assert_same(dense, 5.0, None, "dense cluster, rows > 64")
    assert n > 64 * 300
    mixed = np.concatenate([_uniform(150, 4.0, 16), _uniform(400, 60.0, 17) + np.float32(20)]).astype(np.float32)
    _assert_same(mixed, 3.0, None, "dense core and sparse halo")


def test_radius_graph_capacity_error_reports_size():
    etpc = _etpc()
    pos = torch.from_numpy(_uniform(500, 12.0, 12)).cuda()
    rs, _ = oradius.radius_graph(pos.cpu().numpy(), 3.0, None)
    with pytest.raises(etpc.EtpcError) as ei:
        etpc.etpc_radius_graph(pos, 3.0, max_edges=10)
    assert ei.value.name == "CAPACITY" and str(rs.size) in str(ei.value)
    src, dst = etpc.etpc_radius_graph(pos, 3.0, max_edges=rs.size)
    assert src.numel() == rs.size


def test_radius_graph_large_sampled():
    etpc = _etpc()
    n = 65536
    L = _box_side(n)
    pos = _uniform(n, L, 13)
    note(f"radius graph large: N={n} box={L:.2f}")
    src, dst = etpc.etpc_radius_graph(torch.from_numpy(pos).cuda(), 5.0, box=(L, L, L))
    torch.cuda.synchronize()
    s64, d64 = src.long(), dst.long()
    e = s64.numel()
    note(f"  edges {e}")
    key = d64 * n + s64
    assert bool((key[1:] > key[:-1]).all())                              # canonical order, no duplicates
    assert bool((s64 != d64).all()) and int(s64.min()) >= 0 and int(s64.max()) < n
    tkey, _ = torch.sort(s64 * n + d64)                                   # the transpose, sorted
    assert torch.equal(tkey, key)                                         # symmetric
    rowptr = torch.searchsorted(d64, torch.arange(n + 1, device=d64.device))
    rng = np.random.default_rng(14)
    recv = np.sort(rng.choice(n, 24, replace=False))
    rs, rd = oradius.neighbours_of(pos, recv, 5.0, (L, L, L))
    rp = rowptr.cpu().numpy()
    gs = np.concatenate([src[rp[i]:rp[i + 1]].cpu().numpy() for i in recv])
    assert np.array_equal(gs, rs)


@pytest.mark.parametrize("name", ["cfg2", "cfg3", "cfg1"])
@pytest.mark.parametrize("n_rows", [1, 37, 1000])
def test_layout_convert_matches_oracle(name, n_rows):
    etpc = _etpc()
    cfg = CONFIGS[name]
    plan = plan_from_config(cfg)
    rng = np.random.default_rng(n_rows)
    for features, irreps in (("in", etpc.parse_irreps(cfg.irreps_in)), ("out", plan.out_irreps())):
        width = sum(m * (2 * l + 1) for m, l, _ in irreps)
        x = rng.standard_normal((n_rows, width)).astype(np.float32)
        xt = torch.from_numpy(x).cuda()
        a = etpc.etpc_layout_convert(plan, features, "to_ir_mul", xt)
        b = etpc.etpc_layout_convert(plan, features, "to_mul_ir", xt)
        back = etpc.etpc_layout_convert(plan, features, "to_mul_ir", a)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), olayout.mul_ir_to_ir_mul(x, irreps))
        assert np.array_equal(b.cpu().numpy(), olayout.ir_mul_to_mul_ir(x, irreps))
        assert torch.equal(back, xt)


@pytest.mark.parametrize("irreps", ["3x0e+1x1o+5x2e", "2048x2e+3x0e+7x3o", "16x1o+1x0e+1x0o+2x3o"])
def test_layout_convert_odd_widths_and_offsets(irreps):
    """Widths that are not a multiple of 4 or exceed the LDS strip, and misaligned rows."""
    etpc = _etpc()
    plan = etpc.Plan(irreps, irreps, 1, "uvw", "gaussian", 4, 0.0, 5.0, 6)
    ir = etpc.parse_irreps(irreps)
    width = sum(m * (2 * l + 1) for m, l, _ in ir)
    rng = np.random.default_rng(width)
    for n_rows in (1, 29):
        x = rng.standard_normal((n_rows, width)).astype(np.float32)
        for shift in (0, 1):
            buf_in = torch.zeros(n_rows * width + 1, device="cuda")
            buf_out = torch.zeros(n_rows * width + 1, device="cuda")
            xin = buf_in[shift:shift + n_rows * width].view(n_rows, width)
            xin.copy_(torch.from_numpy(x))
            xout = buf_out[shift:shift + n_rows * width].view(n_rows, width)
            etpc.etpc_layout_convert(plan, "in", "to_ir_mul", xin, out=xout)
            torch.cuda.synchronize()
            assert np.array_equal(xout.cpu().numpy(), olayout.mul_ir_to_ir_mul(x, ir))
            etpc.etpc_layout_convert(plan, "out", "to_mul_ir", xin, out=xout)
            torch.cuda.synchronize()
            assert np.array_equal(xout.cpu().numpy(), olayout.ir_mul_to_mul_ir(x, ir))


@pytest.mark.parametrize("n,e", [(1, 0), (7, 0), (500, 4000), (4096, 200000), (70000, 300000)])
def test_degree_order_matches_oracle(n, e):
    etpc = _etpc()
    rng = np.random.default_rng(n + e)
    src = rng.integers(0, n, e).astype(np.int32)
    dst = rng.integers(0, n, e).astype(np.int32)
    keep = src != dst
    src, dst = src[keep], dst[keep]
    note(f"degree order N={n} E={src.size}")
    g = etpc.etpc_csr_build(n, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    r_all = etpc.etpc_degree_order(g.rowptr)
    s_win = {w: etpc.etpc_degree_order(g.s_rowptr, window=w) for w in (1, 3, 512, 70000, 10 ** 6)}
    torch.cuda.synchronize()
    ref = ocsr.csr_build(n, src, dst)
    assert np.array_equal(g.s_order.cpu().numpy(), ocsr.degree_order(ref["s_rowptr"], window=etpc.SEND_ORDER_WINDOW))
    assert np.array_equal(g.r_order.cpu().numpy(), ocsr.degree_order(ref["rowptr"], window=etpc.RECV_ORDER_WINDOW))
    assert np.array_equal(r_all.cpu().numpy(), ocsr.degree_order(ref["rowptr"]))
    for w, o in s_win.items():
        assert np.array_equal(o.cpu().numpy(), ocsr.degree_order(ref["s_rowptr"], window=w)), w
    etpc.etpc_graph_validate(g)
    # any permutation whose degrees do not increase inside a window is a valid dispatch
    # order (the global degree order too); the validator rejects the others
    etpc.etpc_graph_validate(etpc.Graph(n, g.rowptr, g.col, g.s_rowptr, g.s_col, g.s_slot,
                                        s_order=s_win[10 ** 6], r_order=r_all))
    if n > 1:
        deg = np.diff(ref["s_rowptr"])
        bad = g.s_order.clone()
        bad[[0, -1]] = bad[[-1, 0]]
        if deg[int(bad[0])] < deg[int(bad[1])]:          # the swap raised a degree inside window 0
            with pytest.raises(etpc.EtpcError) as ei:
                etpc.etpc_graph_validate(etpc.Graph(n, g.rowptr, g.col, g.s_rowptr, g.s_col, g.s_slot, s_order=bad))
            assert ei.value.name == "GRAPH"
        bad = g.s_order.clone()
        bad[1] = n
        with pytest.raises(etpc.EtpcError):
            etpc.etpc_graph_validate(etpc.Graph(n, g.rowptr, g.col, g.s_rowptr, g.s_col, g.s_slot, s_order=bad))
        bad = g.r_order.clone()
        bad[-1] = bad[-2]                                  # a node twice, another never
        with pytest.raises(etpc.EtpcError):
            etpc.etpc_graph_validate(etpc.Graph(n, g.rowptr, g.col, g.s_rowptr, g.s_col, g.s_slot, r_order=bad))


def _morton_reference(pos, box):
    """Morton keys as the spatial order defines them, in float32 with every operation rounded
    on its own; returns the stable argsort (ties by index)."""
    p = pos.astype(np.float32)
    if box is None:
        lo = p.min(axis=0)
        ext = np.maximum(p.max(axis=0) - lo, np.float32(1e-30)).astype(np.float32)
        t = (p - lo) / ext
    else:
        L = np.asarray(box, dtype=np.float32)
        t = (p - L * np.floor(p / L)) / L
    c = np.minimum(np.maximum(t * np.float32(1024.0), np.float32(0.0)), np.float32(1023.0)).astype(np.uint32)

    def spread(v):
        v = v & np.uint32(0x3FF)
        v = (v | (v << np.uint32(16))) & np.uint32(0x030000FF)
        v = (v | (v << np.uint32(8))) & np.uint32(0x0300F00F)
        v = (v | (v << np.uint32(4))) & np.uint32(0x030C30C3)
        v = (v | (v << np.uint32(2))) & np.uint32(0x09249249)
        return v

    code = spread(c[:, 0]) | (spread(c[:, 1]) << np.uint32(1)) | (spread(c[:, 2]) << np.uint32(2))
    return np.argsort(code, kind="stable").astype(np.int32)


def _degree_order_along(rowptr, window, base):
    """Windows of positions along `base`, heaviest first inside each, ties in base order."""
    deg = np.diff(rowptr)[base]
    win = np.arange(base.size) // window if window > 0 else np.zeros(base.size, dtype=np.int64)
    return base[np.lexsort((np.arange(base.size), -deg, win))].astype(np.int32)


@pytest.mark.parametrize("n,periodic", [(1, True), (4096, True), (16384, True), (5000, False)])
def test_spatial_order_and_orders_along_it(n, periodic):
    """etpc_spatial_order equals the Morton sort of the positions (periodic wrap or bounding
    box, including atoms outside the box), and etpc_degree_order_within takes windows and
    ties along it; a CSR build given positions carries these orders and validates."""
    etpc = _etpc()
    rng = np.random.default_rng(n + 11)
    L = (n / 0.1) ** (1.0 / 3.0)
    pos = rng.uniform(-0.2 * L, 1.2 * L, (n, 3)).astype(np.float32)
    box = (L, L, L) if periodic else None
    note(f"spatial order N={n} periodic={periodic}")
    pt = torch.from_numpy(pos).cuda()
    got = etpc.etpc_spatial_order(pt, box).cpu().numpy()
    ref = _morton_reference(pos, box)
    assert np.array_equal(got, ref)
    e = 40 * n
    src = rng.integers(0, n, e).astype(np.int32)
    dst = rng.integers(0, n, e).astype(np.int32)
    keep = src != dst
    src, dst = src[keep], dst[keep]
    g = etpc.etpc_csr_build(n, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), pos=pt, box=box)
    cref = ocsr.csr_build(n, src, dst)
    assert np.array_equal(g.s_order.cpu().numpy(), _degree_order_along(cref["s_rowptr"], etpc.SEND_ORDER_WINDOW, ref))
    assert np.array_equal(g.r_order.cpu().numpy(), _degree_order_along(cref["rowptr"], etpc.RECV_ORDER_WINDOW, ref))
    whole = etpc.etpc_degree_order(g.rowptr, window=0, base=torch.from_numpy(ref).cuda())
    assert np.array_equal(whole.cpu().numpy(), _degree_order_along(cref["rowptr"], 0, ref))
    etpc.etpc_graph_validate(g)
