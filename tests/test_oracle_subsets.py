"""Pins for the oracle's edge-subset helpers (oracle/conv.py: edges_into, edges_touching
and the ``edges=`` argument of forward / backward / double_backward).

The full-size GPU tests compare sampled rows against the oracle evaluated on the edges
that reach those rows, and the long oracle runs are split into edge subsets.  Both rely
on two facts checked here against brute force and against the whole-graph oracle:
- the helpers return exactly the edges a brute-force scan selects;
- every output is a sum over edges, so a row is complete once all edges that touch it
  are included, and the results over a partition of the edges sum to the whole.
"""
import numpy as np

from oracle import conv
from tests.oracle_helpers import tiny_config, tiny_workload


def _case(periodic=False, mode="uvw"):
    if mode == "uvw":
        cfg = tiny_config(n_nodes=14, degree=4, irreps_in="3x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e+1x3o",
                          lmax_sh=3, radial="bessel" if periodic else "gaussian",
                          box=7.0 if periodic else None, pos_extent=7.0 if periodic else 4.0, r_hi=3.4 if periodic else 5.0)
    else:
        cfg = tiny_config(n_nodes=14, degree=4, mode="uvu", irreps_in="3x0e+3x1o+3x2e", irreps_out="0e+1o+2e",
                          out_per_path=True, lmax_sh=2, n_basis=4, w_std="uvu")
    return tiny_workload(cfg)


def test_helpers_match_brute_force():
    _, wl = _case()
    nodes = [2, 5, 11]
    into = [e for e in range(len(wl.src)) if int(wl.dst[e]) in nodes]
    touch = [e for e in range(len(wl.src)) if int(wl.dst[e]) in nodes or int(wl.src[e]) in nodes]
    assert conv.edges_into(wl.dst, nodes).tolist() == into
    assert conv.edges_touching(wl.src, wl.dst, nodes).tolist() == touch
    assert conv.edges_into(wl.dst, []).size == 0
    assert conv.edges_touching(wl.src, wl.dst, np.arange(wl.x.shape[0])).tolist() == list(range(len(wl.src)))


def test_subset_rows_equal_full_graph_rows():
    for periodic, mode in ((False, "uvw"), (True, "uvw"), (False, "uvu")):
        spec, wl = _case(periodic, mode)
        nodes = np.array([1, 6, 9])
        zf = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
        zs = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=conv.edges_into(wl.dst, nodes))
        np.testing.assert_allclose(zs[nodes], zf[nodes], rtol=0, atol=1e-13 * np.abs(zf).max())
        # rows the subset does not reach stay zero; a proper subset leaves some
        other = np.setdiff1d(np.arange(wl.x.shape[0]), np.unique(wl.dst[conv.edges_into(wl.dst, nodes)]))
        assert np.all(zs[other] == 0.0) and np.abs(zf[other]).max() > 0
        et = conv.edges_touching(wl.src, wl.dst, nodes)
        xf, _, pf = conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar)
        xs, _, ps = conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=et)
        np.testing.assert_allclose(xs[nodes], xf[nodes], rtol=0, atol=1e-13 * np.abs(xf).max())
        np.testing.assert_allclose(ps[nodes], pf[nodes], rtol=0, atol=1e-13 * np.abs(pf).max())
        rng = np.random.default_rng(4)
        pdot = rng.standard_normal(wl.pos.shape)
        df = conv.double_backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, pos_dot=pdot)
        ds = conv.double_backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, pos_dot=pdot, edges=et)
        for full, sub in zip(df, ds):
            if full.ndim == 2:   # node rows: d/dz_bar, d/dx, d/dpos
                np.testing.assert_allclose(sub[nodes], full[nodes], rtol=0, atol=1e-12 * max(np.abs(full).max(), 1e-300))


def test_partition_sums_to_whole():
    spec, wl = _case(periodic=True)
    E = len(wl.src)
    parts = np.array_split(np.random.default_rng(8).permutation(E), 3)
    zf = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    full = conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar)
    zsum = sum(conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=np.sort(p)) for p in parts)
    np.testing.assert_allclose(zsum, zf, rtol=0, atol=1e-13 * np.abs(zf).max())
    sums = [np.zeros_like(a) for a in full]
    for p in parts:
        for acc, part in zip(sums, conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=p)):
            acc += part
    for acc, want in zip(sums, full):
        np.testing.assert_allclose(acc, want, rtol=0, atol=1e-13 * np.abs(want).max())
    # an empty subset contributes nothing
    for a in conv.backward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=np.zeros(0, np.int64)):
        assert np.all(a == 0.0)
