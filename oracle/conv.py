"""Materialized edge-conditioned tensor-product convolution, float64, CPU.

Definition (the Sobek paper, Sec. 2): for an edge e = (j -> i) with
r_e = p_j - p_i (Eq. 8; minimum image when the box is periodic), distance r and
direction u = r_e / r, radial embedding phi(r) and harmonics Y(u):

  per-edge weights   W_e,pi = sum_q phi_q A_q,pi                      (Eq. 12-13)
  angular product    T_pi[u', m_o] = sum_{a,b} c^pi[a,b,m_o] x_j[k(pi),u',a] Y_ls[b]
  uvw message        M_e[g(pi), w, m_o] += sum_u' W_e,pi[u',w] T_pi[u',m_o]  (Eq. 6, 11)
  uvu message        M_e[g(pi), u', m_o] += W_e,pi[u'] T_pi[u',m_o]          (Eq. 7)
  output             z_i = sum_{e -> i} M_e

This is the conventional schedule the paper contrasts with streaming (the
paragraph after Eq. 13): W_e and M_e are formed explicitly, chunk by chunk.
Backward is float64 autograd of <z_bar, z>; double backward is autograd of
<x_dot, x_bar> + <w_dot, w_bar> + <pos_dot, pos_bar> (PyTorch double-backward
semantics; the paper's directional second adjoints, Eq. 23-31).  Every loss is
a sum over edges, so chunks are differentiated independently and summed.

Pinned by tests/test_oracle_conv.py and tests/test_oracle_grad.py: brute force
on tiny graphs, O(3) equivariance, translation/permutation invariance,
linearity, uvu == uvw with diagonal weights, the streaming reassociation
(Eq. 33-35) in float64, central finite differences, sum of forces = 0, torque
balance, and the exact structure of the force-loss weight gradient.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import cg as _cg
from . import irreps as _ir
from . import radial as _rad
from . import sh as _sh

f64 = torch.float64


@dataclasses.dataclass
class Spec:
    plan: _ir.Plan
    radial: str
    r_lo: float
    r_hi: float
    poly_p: int
    box: Optional[Tuple[float, float, float]]

    @property
    def n_basis(self) -> int:
        return self.plan.n_basis


def spec_from_config(cfg) -> Spec:
    """Build the oracle's own plan from a workload description."""
    plan = _ir.make_plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.n_basis,
                         out_per_path=cfg.out_per_path)
    box = None if cfg.box is None else (cfg.box, cfg.box, cfg.box)
    return Spec(plan, cfg.radial, cfg.r_lo, cfg.r_hi, cfg.poly_p, box)


def _t(a) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a.detach().to(f64)
    return torch.from_numpy(np.asarray(a)).to(f64)


def edge_vectors(ps: torch.Tensor, pd: torch.Tensor, box) -> torch.Tensor:
    """r_e = p_sender - p_receiver, minimum image in an orthorhombic box."""
    rv = ps - pd
    if box is not None:
        L = torch.tensor(box, dtype=rv.dtype)
        rv = rv - L * torch.round(rv / L)
    return rv


def messages(spec: Spec, xs: torch.Tensor, ps: torch.Tensor, pd: torch.Tensor,
             w: torch.Tensor) -> torch.Tensor:
    """Edge messages M_e [Ec, z_dim] from gathered sender rows xs [Ec, x_dim] and
    sender/receiver positions.  Materializes the per-edge weights W_e."""
    plan = spec.plan
    ec = xs.shape[0]
    rv = edge_vectors(ps, pd, spec.box)
    r = torch.linalg.vector_norm(rv, dim=-1)
    u = rv / r[:, None]
    phi = _rad.radial(spec.radial, r, spec.n_basis, spec.r_lo, spec.r_hi, spec.poly_p)  # [Ec, B]
    ys = _sh.sh_all(plan.lmax_sh, u)
    xoff = _ir.offsets(plan.irreps_in)
    zoff = _ir.offsets(plan.irreps_out)
    contrib: Dict[int, torch.Tensor] = {}
    B = spec.n_basis
    for p in plan.paths:
        ni, no = 2 * p.l_in + 1, 2 * p.l_out + 1
        c = torch.from_numpy(_cg.real_cg(p.l_in, p.l_sh, p.l_out)).to(f64)
        xin = xs[:, xoff[p.in_block]: xoff[p.in_block] + ni * p.c_in].reshape(ec, ni, p.c_in)
        cy = torch.einsum("abm,eb->eam", c, ys[p.l_sh])                 # [Ec, ni, no]
        t = torch.einsum("eau,eam->eum", xin, cy)                        # [Ec, C_in, no]
        wp = w[p.w_off: p.w_off + p.w_numel]
        if plan.mode == "uvw":
            we = torch.einsum("eq,quw->euw", phi, wp.reshape(B, p.c_in, p.c_out))   # materialized
            msg = torch.einsum("euw,eum->emw", we, t)                                 # [Ec, no, C_out]
        else:
            we = phi @ wp.reshape(B, p.c_in)                                          # [Ec, C_in]
            msg = (we[:, :, None] * t).permute(0, 2, 1)                               # [Ec, no, C_in]
        msg = msg.reshape(ec, no * p.c_out)
        contrib[p.out_block] = contrib[p.out_block] + msg if p.out_block in contrib else msg
    cols = []
    for g, (mul, l, _) in enumerate(plan.irreps_out):
        width = mul * (2 * l + 1)
        cols.append(contrib[g] if g in contrib else xs.new_zeros(ec, width))
    return torch.cat(cols, dim=1) if cols else xs.new_zeros(ec, 0)


def _chunks(spec: Spec, edges: np.ndarray, budget: int) -> List[np.ndarray]:
    per_edge = sum(p.c_in * p.c_out for p in spec.plan.paths) + spec.plan.z_dim + 1
    step = max(1, budget // per_edge)
    return [edges[i:i + step] for i in range(0, len(edges), step)]


def _edge_index(n_edges: int, edges) -> np.ndarray:
    return np.arange(n_edges) if edges is None else np.asarray(edges, dtype=np.int64)


def forward(spec: Spec, x, pos, w, src, dst, edges=None, budget: int = 1 << 22) -> np.ndarray:
    """z [N, z_dim] (float64).  ``edges``: optional subset of edge indices whose
    messages are summed (rows of z touched only by that subset are exact)."""
    x, pos, w = _t(x), _t(pos), _t(w)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    n = x.shape[0]
    z = torch.zeros(n, spec.plan.z_dim, dtype=f64)
    with torch.no_grad():
        for ch in _chunks(spec, _edge_index(len(src), edges), budget):
            s, d = torch.from_numpy(src[ch]), torch.from_numpy(dst[ch])
            m = messages(spec, x[s], pos[s], pos[d], w)
            z.index_add_(0, d, m)
    return z.numpy()


def backward(spec: Spec, x, pos, w, src, dst, z_bar, edges=None, budget: int = 1 << 21):
    """Gradients of <z_bar, z> w.r.t. x, W and positions (float64)."""
    x, pos, w, zb = _t(x), _t(pos), _t(w), _t(z_bar)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    gx = torch.zeros_like(x)
    gw = torch.zeros_like(w)
    gp = torch.zeros_like(pos)
    for ch in _chunks(spec, _edge_index(len(src), edges), budget):
        s, d = torch.from_numpy(src[ch]), torch.from_numpy(dst[ch])
        xs = x[s].clone().requires_grad_(True)
        ps = pos[s].clone().requires_grad_(True)
        pd = pos[d].clone().requires_grad_(True)
        wl = w.clone().requires_grad_(True)
        m = messages(spec, xs, ps, pd, wl)
        loss = (zb[d] * m).sum()
        axs, aw, aps, apd = torch.autograd.grad(loss, (xs, wl, ps, pd))
        gx.index_add_(0, s, axs)
        gw += aw
        gp.index_add_(0, s, aps)
        gp.index_add_(0, d, apd)
    return gx.numpy(), gw.numpy(), gp.numpy()


def double_backward(spec: Spec, x, pos, w, src, dst, z_bar, x_dot=None, w_dot=None, pos_dot=None,
                    edges=None, budget: int = 1 << 20):
    """VJP of (x, W, pos, z_bar) -> (x_bar, W_bar, pos_bar) with cotangents
    (x_dot, w_dot, pos_dot); returns (d/dz_bar, d/dx, d/dW, d/dpos), float64."""
    x, pos, w, zb = _t(x), _t(pos), _t(w), _t(z_bar)
    xd = None if x_dot is None else _t(x_dot)
    wd = None if w_dot is None else _t(w_dot)
    pdot = None if pos_dot is None else _t(pos_dot)
    src, dst = np.asarray(src, np.int64), np.asarray(dst, np.int64)
    g_zb = torch.zeros_like(zb)
    g_x = torch.zeros_like(x)
    g_w = torch.zeros_like(w)
    g_p = torch.zeros_like(pos)
    for ch in _chunks(spec, _edge_index(len(src), edges), budget):
        s, d = torch.from_numpy(src[ch]), torch.from_numpy(dst[ch])
        xs = x[s].clone().requires_grad_(True)
        ps = pos[s].clone().requires_grad_(True)
        pd = pos[d].clone().requires_grad_(True)
        zbl = zb[d].clone().requires_grad_(True)
        wl = w.clone().requires_grad_(True)
        m = messages(spec, xs, ps, pd, wl)
        loss = (zbl * m).sum()
        axs, aw, aps, apd = torch.autograd.grad(loss, (xs, wl, ps, pd), create_graph=True)
        L = zbl.new_zeros(())
        if xd is not None:
            L = L + (xd[s] * axs).sum()
        if wd is not None:
            L = L + (wd * aw).sum()
        if pdot is not None:
            L = L + (pdot[s] * aps).sum() + (pdot[d] * apd).sum()
        if not L.requires_grad:
            continue
        outs = torch.autograd.grad(L, (zbl, xs, wl, ps, pd), allow_unused=True)
        bz, bx, bw, bps, bpd = [o if o is not None else None for o in outs]
        if bz is not None:
            g_zb.index_add_(0, d, bz)
        if bx is not None:
            g_x.index_add_(0, s, bx)
        if bw is not None:
            g_w += bw
        if bps is not None:
            g_p.index_add_(0, s, bps)
        if bpd is not None:
            g_p.index_add_(0, d, bpd)
    return g_zb.numpy(), g_x.numpy(), g_w.numpy(), g_p.numpy()


def edges_into(dst, nodes: Sequence[int]) -> np.ndarray:
    """Edge indices whose receiver is in ``nodes`` (rows of z they complete)."""
    return np.nonzero(np.isin(np.asarray(dst), np.asarray(nodes)))[0]


def edges_touching(src, dst, nodes: Sequence[int]) -> np.ndarray:
    """Edge indices incident to ``nodes`` as sender or receiver (completes their
    rows of x_bar and pos_bar)."""
    nodes = np.asarray(nodes)
    return np.nonzero(np.isin(np.asarray(src), nodes) | np.isin(np.asarray(dst), nodes))[0]
