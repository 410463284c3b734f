"""GPU parity at the full workload sizes, in the launch configuration the bench uses.

The oracle cannot evaluate whole graphs of 1e5-1e7 edges in seconds, so:
- rows of z, x_bar, pos_bar, z_bar_grad, d/dx and d/dpos are checked for sampled nodes, the
  oracle summing exactly the edges that reach those rows;
- W-gradients are checked through linearity, which holds at any size: z is linear in
  W, so <W_bar, V> = <z_bar, z(W = V)>, and <dL/dW, V> = <pos_dot, pos_bar(W = V)>;
  likewise <x_bar, U> = <z_bar, z(x = U)> (V, U seeded normal draws).
Tolerance: max|d| / max|ref| <= 1e-4 (forward, backward), 1e-3 (double backward); the
linearity identities to 1e-4 (1e-3) of the root sum of squares of the terms of both
inner products, the scale their rounding error grows with (a sum of 1e7 random-sign
terms can cancel to almost nothing, so the result itself is no scale).
"""
import numpy as np
import pytest
import torch

from oracle import conv
from tests.gpu_helpers import make_case, note, rel_err
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

SAMPLES = 6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _etpc():
    import equivariant_gnn_tensor_amd as etpc
    return etpc


def _rows(t, idx):
    return t.detach().double().cpu().numpy()[idx]


def _dot(a, b):
    return float((a.double() * b.double()).sum().item())


def _l2_terms(a, b):
    """sqrt(sum_i (a_i b_i)^2): the scale of the rounding error of <a, b> when each a_i
    carries an independent relative error (fp32 results)."""
    return float(((a.double() * b.double()) ** 2).sum().sqrt().item())


def _close(lhs, rhs, scale, tol):
    """|lhs - rhs| <= tol * scale.  The scale is the root sum of squares of the terms of
    both inner products: independent per-element rounding errors add up like that, while
    the result itself, a sum of ~1e7 random-sign terms, can cancel to almost nothing and
    is no scale.  A wrong value in even a small fraction of the elements moves the sum by
    far more than tol * scale."""
    return abs(lhs - rhs) <= tol * scale


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg4_d16", "cfg4_d512", "cfg5"])
def test_full_size_sampled(name):
    etpc = _etpc()
    cfg = CONFIGS[name]
    note(f"full size {cfg.name}: building workload")
    c = make_case(cfg)
    wl = c.wl
    note(f"full size {cfg.name}: N={wl.n_nodes} E={wl.n_edges} forward")
    rng = np.random.default_rng(77)
    nodes = np.sort(rng.choice(wl.n_nodes, SAMPLES, replace=False))
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    torch.cuda.synchronize()
    e_in = conv.edges_into(wl.dst, nodes)
    rz = conv.forward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, edges=e_in)[nodes]
    err = rel_err(_rows(z, nodes), rz)
    note(f"  z rows rel err {err:.2e}")
    assert err <= 1e-4
    if "bwd" not in cfg.passes:
        return
    note(f"full size {cfg.name}: backward")
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    torch.cuda.synchronize()
    e_touch = conv.edges_touching(wl.src, wl.dst, nodes)
    rx, _, rp = conv.backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar, edges=e_touch)
    ex, ep = rel_err(_rows(xb, nodes), rx[nodes]), rel_err(_rows(pb, nodes), rp[nodes])
    note(f"  x_bar rows {ex:.2e}  pos_bar rows {ep:.2e}")
    assert ex <= 1e-4 and ep <= 1e-4
    # linearity identities for W_bar and x_bar
    gen = torch.Generator(device="cuda").manual_seed(1234)
    V = torch.randn(c.w.shape, generator=gen, device="cuda")
    zV = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, V)
    U = torch.randn(c.x.shape, generator=gen, device="cuda")
    zU = etpc.etpc_forward(c.plan, c.graph, U, c.pos, c.w)
    torch.cuda.synchronize()
    lw, rw = _dot(wb, V), _dot(c.z_bar, zV)
    lx, rx2 = _dot(xb, U), _dot(c.z_bar, zU)
    sw = _l2_terms(wb, V) + _l2_terms(c.z_bar, zV)
    sx = _l2_terms(xb, U) + _l2_terms(c.z_bar, zU)
    note(f"  <W_bar,V> {lw:.6e} vs {rw:.6e} (scale {sw:.3e});  <x_bar,U> {lx:.6e} vs {rx2:.6e} (scale {sx:.3e})")
    assert _close(lw, rw, sw, 1e-4) and _close(lx, rx2, sx, 1e-4)
    if "dbl" not in cfg.passes:
        return
    note(f"full size {cfg.name}: double backward")
    pos_dot = torch.from_numpy(-wl.force_c).cuda()
    gz, gx, gw, gp = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, pos_dot=pos_dot)
    torch.cuda.synchronize()
    rgz, rgx, _, rgp = conv.double_backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar,
                                            pos_dot=-wl.force_c.astype(np.float64), edges=e_touch)
    ez = rel_err(_rows(gz, nodes), rgz[nodes])
    ep = rel_err(_rows(gp, nodes), rgp[nodes])
    note(f"  d/dpos rows {ep:.2e}")
    assert ep <= 1e-3
    e_src = np.nonzero(np.isin(wl.src, nodes))[0]
    _, rgx2, _, _ = conv.double_backward(c.spec, wl.x, wl.pos, wl.w, wl.src, wl.dst, wl.z_bar,
                                         pos_dot=-wl.force_c.astype(np.float64), edges=e_src)
    egx = rel_err(_rows(gx, nodes), rgx2[nodes])
    note(f"  z_bar_grad rows {ez:.2e}  x_grad rows {egx:.2e}")
    assert ez <= 1e-3 and egx <= 1e-3
    _, _, pV = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, V, c.z_bar, want=("pos",))
    torch.cuda.synchronize()
    lw, rw = _dot(gw, V), _dot(pos_dot, pV)
    sw = _l2_terms(gw, V) + _l2_terms(pos_dot, pV)
    note(f"  <dL/dW,V> {lw:.6e} vs {rw:.6e} (scale {sw:.3e})")
    assert _close(lw, rw, sw, 1e-3)
