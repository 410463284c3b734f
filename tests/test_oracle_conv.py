"""Pins for the oracle forward (oracle/conv.py)."""
import math

import numpy as np
import pytest
import torch

from oracle import conv, irreps as ir, radial, sh
from oracle.cg import real_cg
from oracle.wigner import random_rotation, wigner_d
from tests.oracle_helpers import o3_transform_features, tiny_config, tiny_workload


def _brute_forward(spec, x, pos, w, src, dst):
    """Pure-Python loops over edges, paths and every index (ir_mul layout)."""
    plan = spec.plan
    n = x.shape[0]
    z = [[0.0] * plan.z_dim for _ in range(n)]
    xoff, zoff = ir.offsets(plan.irreps_in), ir.offsets(plan.irreps_out)
    B = plan.n_basis
    for e in range(len(src)):
        j, i = int(src[e]), int(dst[e])
        rv = [float(pos[j][d]) - float(pos[i][d]) for d in range(3)]
        if spec.box is not None:
            rv = [rv[d] - spec.box[d] * round(rv[d] / spec.box[d]) for d in range(3)]
        r = math.sqrt(sum(v * v for v in rv))
        u = torch.tensor([[v / r for v in rv]], dtype=torch.float64)
        phi = radial.radial(spec.radial, torch.tensor([r], dtype=torch.float64), B, spec.r_lo, spec.r_hi,
                            spec.poly_p)[0].tolist()
        Y = [sh.sh(l, u)[0].tolist() for l in range(plan.lmax_sh + 1)]
        for p in plan.paths:
            c = real_cg(p.l_in, p.l_sh, p.l_out)
            ni, ns, no = 2 * p.l_in + 1, 2 * p.l_sh + 1, 2 * p.l_out + 1
            for wo in range(p.c_out):
                for mo in range(no):
                    acc = 0.0
                    for ui in range(p.c_in):
                        if plan.mode == "uvw":
                            wt = sum(phi[q] * float(w[p.w_off + (q * p.c_in + ui) * p.c_out + wo]) for q in range(B))
                        else:
                            if ui != wo:
                                continue
                            wt = sum(phi[q] * float(w[p.w_off + q * p.c_in + ui]) for q in range(B))
                        for a in range(ni):
                            for b in range(ns):
                                acc += wt * c[a, b, mo] * float(x[j][xoff[p.in_block] + a * p.c_in + ui]) * Y[p.l_sh][b]
                    z[i][zoff[p.out_block] + mo * p.c_out + wo] += acc
    return np.array(z)


@pytest.mark.parametrize("mode,periodic", [("uvw", False), ("uvw", True), ("uvu", False)])
def test_brute_force_tiny(mode, periodic):
    if mode == "uvw":
        cfg = tiny_config(n_nodes=6, degree=2, irreps_in="2x0e+2x1o+1x2e", irreps_out="2x0e+1x1o+2x2e+1x3o",
                          lmax_sh=3, n_basis=3, radial="bessel" if periodic else "gaussian",
                          box=8.0 if periodic else None, pos_extent=8.0 if periodic else 4.0)
    else:
        cfg = tiny_config(n_nodes=6, degree=2, mode="uvu", irreps_in="2x0e+2x1o+2x2e", irreps_out="0e+1o+2e",
                          out_per_path=True, lmax_sh=2, n_basis=3, w_std="uvu")
    spec, wl = tiny_workload(cfg)
    got = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, budget=64)
    want = _brute_forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    np.testing.assert_allclose(got, want, atol=1e-12 * max(1.0, np.abs(want).max()))
    assert np.abs(want).max() > 1e-3


def _o3_case(rng, det):
    cfg = tiny_config(n_nodes=12, degree=5, irreps_in="3x0e+2x1o+2x2e+1x3o", irreps_out="2x0e+2x1o+2x2e+2x3o",
                      lmax_sh=3)
    spec, wl = tiny_workload(cfg)
    R = random_rotation(rng)
    Q = R if det > 0 else -R
    D = lambda l: wigner_d(l, R)  # noqa: E731
    return spec, wl, Q, D


@pytest.mark.parametrize("det", [1, -1])
def test_o3_equivariance(det, rng):
    spec, wl, Q, D = _o3_case(rng, det)
    z = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    xq = o3_transform_features(wl.x.astype(np.float64), spec.plan.irreps_in, D, det)
    zq = conv.forward(spec, xq, wl.pos.astype(np.float64) @ Q.T, wl.w, wl.src, wl.dst)
    want = o3_transform_features(z, spec.plan.irreps_out, D, det)
    np.testing.assert_allclose(zq, want, atol=1e-11 * np.abs(z).max())


def test_translation_permutation_linearity(rng):
    cfg = tiny_config(n_nodes=10, degree=4)
    spec, wl = tiny_workload(cfg)
    z = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    zt = conv.forward(spec, wl.x, wl.pos.astype(np.float64) + np.array([1.3, -0.4, 7.0]), wl.w, wl.src, wl.dst)
    np.testing.assert_allclose(zt, z, atol=1e-12 * np.abs(z).max())
    perm = rng.permutation(len(wl.src))
    zp = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src[perm], wl.dst[perm])
    np.testing.assert_allclose(zp, z, atol=1e-12 * np.abs(z).max())
    x2 = rng.standard_normal(wl.x.shape)
    z2 = conv.forward(spec, x2, wl.pos, wl.w, wl.src, wl.dst)
    zc = conv.forward(spec, 2.0 * wl.x - 3.0 * x2, wl.pos, wl.w, wl.src, wl.dst)
    np.testing.assert_allclose(zc, 2.0 * z - 3.0 * z2, atol=1e-11 * np.abs(zc).max())
    w2 = rng.standard_normal(wl.w.shape)
    zw2 = conv.forward(spec, wl.x, wl.pos, w2, wl.src, wl.dst)
    zwc = conv.forward(spec, wl.x, wl.pos, 0.5 * wl.w + w2, wl.src, wl.dst)
    np.testing.assert_allclose(zwc, 0.5 * z + zw2, atol=1e-11 * np.abs(zwc).max())


def test_periodic_minimum_image():
    cfg = tiny_config(n_nodes=10, degree=4, box=6.0, pos_extent=6.0, radial="bessel", r_hi=2.9)
    spec, wl = tiny_workload(cfg)
    z = conv.forward(spec, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    assert np.abs(z).max() > 1e-3
    p2 = wl.pos.astype(np.float64).copy()
    p2[3] += np.array([6.0, -12.0, 6.0])
    z2 = conv.forward(spec, wl.x, p2, wl.w, wl.src, wl.dst)
    np.testing.assert_allclose(z2, z, atol=1e-11 * np.abs(z).max())


def test_uvu_equals_uvw_with_diagonal_weights(rng):
    c = 3
    cu = tiny_config(n_nodes=8, degree=3, mode="uvu", irreps_in=f"{c}x0e+{c}x1o+{c}x2e", irreps_out="0e+1o+2e",
                     out_per_path=True, lmax_sh=2, n_basis=4, w_std="uvu")
    spec_u, wl = tiny_workload(cu)
    zu = conv.forward(spec_u, wl.x, wl.pos, wl.w, wl.src, wl.dst)
    plan_w = ir.make_plan(f"{c}x0e+{c}x1o+{c}x2e", f"{c}x0e+{c}x1o+{c}x2e", 2, "uvw", 4)
    spec_w = conv.Spec(plan_w, spec_u.radial, spec_u.r_lo, spec_u.r_hi, spec_u.poly_p, spec_u.box)
    ww = np.zeros(plan_w.w_numel)
    zsum = np.zeros((wl.x.shape[0], plan_w.z_dim))
    zoff_u, zoff_w = ir.offsets(spec_u.plan.irreps_out), ir.offsets(plan_w.irreps_out)
    for pu in spec_u.plan.paths:
        (pw,) = [q for q in plan_w.paths if (q.in_block, q.l_sh, q.l_out) == (pu.in_block, pu.l_sh, pu.l_out)]
        wu = wl.w[pu.w_off:pu.w_off + pu.w_numel].reshape(4, c).astype(np.float64)
        blk = np.zeros((4, c, c))
        for u in range(c):
            blk[:, u, u] = wu[:, u]
        ww[pw.w_off:pw.w_off + pw.w_numel] = blk.reshape(-1)
        width = c * (2 * pu.l_out + 1)
        zsum[:, zoff_w[pw.out_block]:zoff_w[pw.out_block] + width] += zu[:, zoff_u[pu.out_block]:zoff_u[pu.out_block] + width]
    zw = conv.forward(spec_w, wl.x, wl.pos, ww, wl.src, wl.dst)
    np.testing.assert_allclose(zw, zsum, atol=1e-12 * np.abs(zw).max())


def test_streaming_reassociation_equals_materialized():
    """Eq. 33-35 (receiver state S, then S A) equals the materialized schedule."""
    cfg = tiny_config(n_nodes=16, degree=6, irreps_in="4x0e+4x1o+4x2e", irreps_out="3x0e+3x1o+3x2e+3x3o", lmax_sh=3)
    spec, wl = tiny_workload(cfg)
    plan = spec.plan
    x, pos, w = wl.x.astype(np.float64), wl.pos.astype(np.float64), wl.w.astype(np.float64)
    rv = pos[wl.src] - pos[wl.dst]
    r = np.linalg.norm(rv, axis=1)
    u = torch.from_numpy(rv / r[:, None])
    phi = radial.radial(spec.radial, torch.from_numpy(r), plan.n_basis, spec.r_lo, spec.r_hi, spec.poly_p).numpy()
    xoff, zoff = ir.offsets(plan.irreps_in), ir.offsets(plan.irreps_out)
    z = np.zeros((x.shape[0], plan.z_dim))
    for p in plan.paths:
        ni, no = 2 * p.l_in + 1, 2 * p.l_out + 1
        y = sh.sh(p.l_sh, u).numpy()
        xj = x[wl.src, xoff[p.in_block]:xoff[p.in_block] + ni * p.c_in].reshape(-1, ni, p.c_in)
        C = np.einsum("abm,eau,eb->eum", real_cg(p.l_in, p.l_sh, p.l_out), xj, y)       # Eq. 32
        S = np.zeros((x.shape[0], plan.n_basis, p.c_in, no))
        np.add.at(S, wl.dst, np.einsum("eq,eum->equm", phi, C))                       # Eq. 33
        A = w[p.w_off:p.w_off + p.w_numel].reshape(plan.n_basis, p.c_in, p.c_out)
        m = np.einsum("iqum,quw->imw", S, A)                                            # Eq. 34-35
        z[:, zoff[p.out_block]:zoff[p.out_block] + no * p.c_out] += m.reshape(x.shape[0], -1)
    want = conv.forward(spec, x, pos, w, wl.src, wl.dst)
    np.testing.assert_allclose(z, want, atol=1e-12 * np.abs(want).max())
