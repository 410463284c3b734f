"""Pins for the oracle backward and double backward (oracle/conv.py)."""
import numpy as np
import pytest

from oracle import conv
from oracle.wigner import random_rotation, wigner_d
from tests.oracle_helpers import o3_transform_features, tiny_config, tiny_workload
from workloads import make_workload
from workloads.generate import scalar_mask


def _loss(spec, wl, x, pos, w, zb):
    return float(np.sum(conv.forward(spec, x, pos, w, wl.src, wl.dst) * zb))


def _fd(f, base, v, h):
    return (f(base + h * v) - f(base - h * v)) / (2 * h)


@pytest.mark.parametrize("mode,periodic", [("uvw", False), ("uvw", True), ("uvu", False)])
def test_backward_finite_differences(mode, periodic, rng):
    if mode == "uvw":
        cfg = tiny_config(n_nodes=10, degree=4, irreps_in="3x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e+1x3o",
                          lmax_sh=3, radial="bessel" if periodic else "gaussian",
                          box=7.0 if periodic else None, pos_extent=7.0 if periodic else 4.0, r_hi=3.4 if periodic else 5.0)
    else:
        cfg = tiny_config(n_nodes=10, degree=4, mode="uvu", irreps_in="2x0e+2x1o+2x2e", irreps_out="0e+1o+2e",
                          out_per_path=True, lmax_sh=2, w_std="uvu")
    spec, wl = tiny_workload(cfg)
    x, pos, w, zb = (a.astype(np.float64) for a in (wl.x, wl.pos, wl.w, wl.z_bar))
    gx, gw, gp = conv.backward(spec, x, pos, w, wl.src, wl.dst, zb)
    for g, base, which in ((gx, x, "x"), (gw, w, "w"), (gp, pos, "p")):
        v = rng.standard_normal(base.shape)
        if which == "x":
            f = lambda t: _loss(spec, wl, t, pos, w, zb)  # noqa: E731
        elif which == "w":
            f = lambda t: _loss(spec, wl, x, pos, t, zb)  # noqa: E731
        else:
            f = lambda t: _loss(spec, wl, x, t, w, zb)  # noqa: E731
        fd = _fd(f, base, v, 1e-5)
        an = float(np.sum(g * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)
    np.testing.assert_allclose(gp.sum(axis=0), 0.0, atol=1e-10 * np.abs(gp).max())   # translation invariance


@pytest.mark.parametrize("det", [1, -1])
def test_backward_equivariance(det, rng):
    cfg = tiny_config(n_nodes=10, degree=4, irreps_in="3x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e+1x3o", lmax_sh=3)
    spec, wl = tiny_workload(cfg)
    x, pos, w, zb = (a.astype(np.float64) for a in (wl.x, wl.pos, wl.w, wl.z_bar))
    R = random_rotation(rng)
    Q = R if det > 0 else -R
    D = lambda l: wigner_d(l, R)  # noqa: E731
    gx, gw, gp = conv.backward(spec, x, pos, w, wl.src, wl.dst, zb)
    hx, hw, hp = conv.backward(spec, o3_transform_features(x, spec.plan.irreps_in, D, det), pos @ Q.T, w,
                               wl.src, wl.dst, o3_transform_features(zb, spec.plan.irreps_out, D, det))
    np.testing.assert_allclose(hx, o3_transform_features(gx, spec.plan.irreps_in, D, det), atol=1e-11 * np.abs(gx).max())
    np.testing.assert_allclose(hw, gw, atol=1e-11 * np.abs(gw).max())
    np.testing.assert_allclose(hp, gp @ Q.T, atol=1e-11 * np.abs(gp).max())


def test_torque_free_for_scalar_inputs():
    cfg = tiny_config(n_nodes=12, degree=5, irreps_in="4x0e", irreps_out="3x0e+3x1o+3x2e", lmax_sh=2,
                      cotangent="energy")
    spec = conv.spec_from_config(cfg)
    wl = make_workload(cfg, w_blocks=spec.plan.w_blocks(), scalar_out_mask=scalar_mask(cfg.irreps_out))
    pos = wl.pos.astype(np.float64)
    _, _, gp = conv.backward(spec, wl.x, pos, wl.w, wl.src, wl.dst, wl.z_bar)
    force = -gp
    torque = np.cross(pos, force).sum(axis=0)
    np.testing.assert_allclose(torque, 0.0, atol=1e-11 * np.abs(force).max() * np.abs(pos).max())


def _force_case(periodic):
    cfg = tiny_config(n_nodes=12, degree=5, irreps_in="3x0e+2x1o+2x2e", irreps_out="3x0e+2x1o+2x2e", lmax_sh=2,
                      cotangent="energy", radial="bessel", r_hi=3.4 if periodic else 5.0,
                      box=7.0 if periodic else None, pos_extent=7.0 if periodic else 4.0)
    spec = conv.spec_from_config(cfg)
    wl = make_workload(cfg, w_blocks=spec.plan.w_blocks(), scalar_out_mask=scalar_mask(cfg.irreps_out))
    return spec, wl


@pytest.mark.parametrize("periodic", [False, True])
def test_force_loss_double_backward(periodic, rng):
    """L = <c, F> with F = -d(sum of 0e outputs)/dpos; d/dW and d/dx by central differences."""
    spec, wl = _force_case(periodic)
    x, pos, w, zb, c = (a.astype(np.float64) for a in (wl.x, wl.pos, wl.w, wl.z_bar, wl.force_c))

    def L(xx, ww):
        _, _, gp = conv.backward(spec, xx, pos, ww, wl.src, wl.dst, zb)
        return float(np.sum(c * -gp))

    _, dx, dw, _ = conv.double_backward(spec, x, pos, w, wl.src, wl.dst, zb, pos_dot=-c)
    vw, vx = rng.standard_normal(w.shape), rng.standard_normal(x.shape)
    fdw = _fd(lambda t: L(x, t), w, vw, 1e-5)
    fdx = _fd(lambda t: L(t, w), x, vx, 1e-5)
    assert abs(fdw - np.sum(dw * vw)) < 1e-7 * max(1, abs(fdw))
    assert abs(fdx - np.sum(dx * vx)) < 1e-7 * max(1, abs(fdx))
    # exact structure: only paths into 0e receive a weight gradient, and it does not depend on w
    for p in spec.plan.paths:
        blk = dw[p.w_off:p.w_off + p.w_numel].reshape(spec.n_basis, p.c_in, p.c_out)
        if p.l_out != 0:
            assert np.all(blk == 0)
        else:
            np.testing.assert_allclose(blk, np.repeat(blk[:, :, :1], p.c_out, axis=2), atol=1e-12 * np.abs(blk).max())
            assert np.abs(blk).max() > 0
    _, _, gp = conv.backward(spec, x, pos, w, wl.src, wl.dst, zb)
    np.testing.assert_allclose(gp.sum(axis=0), 0.0, atol=1e-10 * np.abs(gp).max())


def test_general_double_backward_finite_differences(rng):
    """All four outputs of the VJP of backward, against central differences of
    L = <x_dot, x_bar> + <w_dot, w_bar> + <pos_dot, pos_bar>."""
    cfg = tiny_config(n_nodes=9, degree=4, irreps_in="2x0e+2x1o+1x2e", irreps_out="2x0e+2x1o+1x2e", lmax_sh=2)
    spec, wl = tiny_workload(cfg)
    x, pos, w, zb = (a.astype(np.float64) for a in (wl.x, wl.pos, wl.w, wl.z_bar))
    xd, wd, pd = rng.standard_normal(x.shape), rng.standard_normal(w.shape), rng.standard_normal(pos.shape)

    def L(zz, xx, ww, pp):
        gx, gw, gp = conv.backward(spec, xx, pp, ww, wl.src, wl.dst, zz)
        return float(np.sum(xd * gx) + np.sum(wd * gw) + np.sum(pd * gp))

    gz, gx, gw, gp = conv.double_backward(spec, x, pos, w, wl.src, wl.dst, zb, x_dot=xd, w_dot=wd, pos_dot=pd)
    args = [zb, x, w, pos]
    for idx, g in enumerate((gz, gx, gw, gp)):
        v = rng.standard_normal(args[idx].shape)

        def f(t, idx=idx):
            a = list(args)
            a[idx] = t
            return L(*a)

        fd = _fd(f, args[idx], v, 1e-5)
        assert abs(fd - np.sum(g * v)) < 1e-7 * max(1, abs(fd)), idx
