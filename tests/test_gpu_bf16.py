"""GPU parity of the reduced-precision channel GEMMs (bf16 or fp16 operands, fp32
accumulation).

Only the channel-space GEMMs round (z = S W, Xt = x W, x_bar = P W^T, W_bar = x^T P);
traversals and reductions stay fp32.  Tolerance, from the arithmetic: each operand is
rounded with unit roundoff u (bf16: 2^-9, fp16: 2^-11), so each product carries a
relative error of at most 2u and the K rounding errors of one output add up like
independent terms, about 2u times the root-sum-square of the products, which is of the
order of the output's own size for the largest outputs.  The test measure
max|d| / max|ref| is therefore a few times 2u (bf16 3.9e-3, fp16 9.8e-4); it is held to
about 2.5 times 2u for forward and backward (bf16 1e-2, fp16 2.5e-3) and twice that for
double backward, whose outputs pass through two rounded GEMMs.  Each case also checks
that the reduced-precision result differs from the fp32 one (so those kernels ran) by
less than the same bound.
"""
import numpy as np
import pytest
import torch

from oracle import conv
from tests.gpu_helpers import make_case, note, rel_err
from workloads import small_variant

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp16": 2.5e-3}
TOL_DBL = {"bf16": 2e-2, "fp16": 5e-3}
PRECISIONS = ("bf16", "fp16")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _etpc():
    import equivariant_gnn_tensor_amd as etpc
    return etpc


def _differs(a, b):
    a = a.detach().double().cpu()
    b = b.detach().double().cpu()
    return float((a - b).abs().max() / b.abs().max())


@pytest.mark.parametrize("prec", PRECISIONS)
@pytest.mark.parametrize("name,n", [("cfg2", 256), ("cfg4_d64", 300), ("cfg3", 128)])
def test_reduced_precision_forward_backward(name, n, prec):
    etpc = _etpc()
    cfg = small_variant(name, n)
    c = make_case(cfg, gemm_precision=prec)
    c32 = make_case(cfg)
    note(f"{prec} forward/backward {cfg.name} N={cfg.n_nodes}")
    z = etpc.etpc_forward(c.plan, c.graph, c.x, c.pos, c.w)
    z32 = etpc.etpc_forward(c32.plan, c32.graph, c32.x, c32.pos, c32.w)
    torch.cuda.synchronize()
    ref = conv.forward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst)
    ez = rel_err(z, ref)
    if cfg.mode == "uvw":
        assert 1e-6 < _differs(z, z32) <= TOL[prec]
    xb, wb, pb = etpc.etpc_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar)
    xb32, _, _ = etpc.etpc_backward(c32.plan, c32.graph, c32.x, c32.pos, c32.w, c32.z_bar)
    torch.cuda.synchronize()
    rx, rw, rp = conv.backward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst, c.wl.z_bar)
    errs = (ez, rel_err(xb, rx), rel_err(wb, rw), rel_err(pb, rp))
    note(f"  {prec} rel err z {errs[0]:.2e} x_bar {errs[1]:.2e} w_bar {errs[2]:.2e} pos_bar {errs[3]:.2e}")
    assert max(errs) <= TOL[prec]
    if cfg.mode == "uvw":
        assert 1e-6 < _differs(xb, xb32)


@pytest.mark.parametrize("prec", PRECISIONS)
def test_reduced_precision_double_backward(prec):
    etpc = _etpc()
    cfg = small_variant("cfg5", 128)
    c = make_case(cfg, gemm_precision=prec)
    note(f"{prec} double backward {cfg.name}")
    rng = np.random.default_rng(21)
    xd = rng.standard_normal(c.wl.x.shape).astype(np.float32)
    wd = rng.standard_normal(c.wl.w.shape).astype(np.float32)
    pd = rng.standard_normal(c.wl.pos.shape).astype(np.float32)
    T = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    gz, gx, gw, gp = etpc.etpc_double_backward(c.plan, c.graph, c.x, c.pos, c.w, c.z_bar, x_dot=T(xd),
                                               w_dot=T(wd), pos_dot=T(pd))
    torch.cuda.synchronize()
    rz, rx, rw, rp = conv.double_backward(c.spec, c.wl.x, c.wl.pos, c.wl.w, c.wl.src, c.wl.dst, c.wl.z_bar,
                                          x_dot=xd, w_dot=wd, pos_dot=pd)
    errs = (rel_err(gz, rz), rel_err(gx, rx), rel_err(gw, rw), rel_err(gp, rp))
    note(f"  {prec} double backward rel err {['%.2e' % e for e in errs]}")
    assert max(errs) <= TOL_DBL[prec]
