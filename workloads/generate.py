"""Seeded input draws for the synthetic workloads.

Draw order is fixed: positions, graph (including the COO shuffle), x, W,
cotangents.  Every value is drawn in float64 with ``numpy.random.default_rng``
and then rounded to float32; both the GPU path and the oracle receive the same
float32 values.  Nothing here evaluates the convolution: weight scaling per
path block and the output width are passed in by the caller.
"""
from __future__ import annotations

import dataclasses
import re
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .configs import WorkloadConfig

_IRREP_RE = re.compile(r"^\s*(?:(\d+)\s*x\s*)?(\d+)([eo])\s*$")


def parse_irreps(s: str) -> List[Tuple[int, int, int]]:
    """"64x0e+64x1o" -> [(64, 0, +1), (64, 1, -1)] as (mul, l, parity)."""
    out = []
    for tok in s.split("+"):
        m = _IRREP_RE.match(tok)
        if not m:
            raise ValueError(f"bad irrep token {tok!r}")
        mul = int(m.group(1)) if m.group(1) else 1
        out.append((mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def irreps_dim(irreps: Sequence[Tuple[int, int, int]]) -> int:
    return sum(mul * (2 * l + 1) for mul, l, _ in irreps)


def irreps_offsets(irreps: Sequence[Tuple[int, int, int]]) -> List[int]:
    offs, o = [], 0
    for mul, l, _ in irreps:
        offs.append(o)
        o += mul * (2 * l + 1)
    return offs


@dataclasses.dataclass
class Workload:
    cfg: WorkloadConfig
    pos: np.ndarray          # [N,3] float32
    src: np.ndarray          # [E] int32 sender j of edge j->i
    dst: np.ndarray          # [E] int32 receiver i
    x: np.ndarray            # [N, C_x] float32, ir_mul layout
    w: Optional[np.ndarray]  # [w_numel] float32
    z_bar: Optional[np.ndarray]   # [N, C_z] float32
    force_c: Optional[np.ndarray]  # [N,3] float32 (energy/force workloads)

    @property
    def n_nodes(self) -> int:
        return self.pos.shape[0]

    @property
    def n_edges(self) -> int:
        return int(self.src.shape[0])


def _positions(rng, cfg: WorkloadConfig) -> np.ndarray:
    return rng.uniform(0.0, cfg.pos_extent, size=(cfg.n_nodes, 3))


def _indegree_graph(rng, n: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    if d > n - 1:
        raise ValueError("in-degree larger than n-1")
    src = np.empty(n * d, dtype=np.int64)
    for i in range(n):
        s = rng.choice(n - 1, size=d, replace=False)
        s = s + (s >= i)                     # uniform over V \ {i}
        src[i * d:(i + 1) * d] = s
    dst = np.repeat(np.arange(n, dtype=np.int64), d)
    return src, dst


def _radius_graph(pos: np.ndarray, cutoff: float, box: Optional[float]) -> Tuple[np.ndarray, np.ndarray]:
    from scipy.spatial import cKDTree
    tree = cKDTree(pos, boxsize=box) if box else cKDTree(pos)
    pairs = tree.query_pairs(cutoff, output_type="ndarray").astype(np.int64)
    a, b = pairs[:, 0], pairs[:, 1]
    return np.concatenate([a, b]), np.concatenate([b, a])


def draw_weights(rng, w_blocks: Sequence[Tuple[int, float]]) -> np.ndarray:
    """One standard-normal draw for all of W, scaled block-wise by the given stds."""
    total = sum(n for n, _ in w_blocks)
    raw = rng.standard_normal(total)
    scale = np.concatenate([np.full(n, s, dtype=np.float64) for n, s in w_blocks]) if w_blocks else raw[:0]
    return raw * scale


def make_workload(cfg: WorkloadConfig,
                  w_blocks: Optional[Sequence[Tuple[int, float]]] = None,
                  z_dim: Optional[int] = None,
                  scalar_out_mask: Optional[np.ndarray] = None) -> Workload:
    """Draw one workload.

    w_blocks: [(numel, std), ...] per weight block in storage order (None: no W).
    z_dim: output width; needed for random cotangents (cotangent="normal").
    scalar_out_mask: bool [z_dim], True on scalar (0e) output columns; needed for
        cotangent="energy", where z_bar = 1 on those columns and 0 elsewhere.
    """
    rng = np.random.default_rng(cfg.seed)
    pos = _positions(rng, cfg)
    if cfg.graph == "indegree":
        src, dst = _indegree_graph(rng, cfg.n_nodes, cfg.degree)
    elif cfg.graph == "radius" and cfg.n_graphs > 1:
        # block-diagonal batch: each cell's radius graph on its own atoms, indices offset
        per = cfg.n_nodes // cfg.n_graphs
        if per * cfg.n_graphs != cfg.n_nodes:
            raise ValueError("n_nodes must be a multiple of n_graphs")
        parts = [_radius_graph(pos[b * per:(b + 1) * per], cfg.cutoff, cfg.box) for b in range(cfg.n_graphs)]
        src = np.concatenate([s + b * per for b, (s, _) in enumerate(parts)])
        dst = np.concatenate([d + b * per for b, (_, d) in enumerate(parts)])
    elif cfg.graph == "radius":
        src, dst = _radius_graph(pos, cfg.cutoff, cfg.box)
    else:
        raise ValueError(cfg.graph)
    perm = rng.permutation(src.shape[0])
    src, dst = src[perm], dst[perm]
    c_x = irreps_dim(parse_irreps(cfg.irreps_in))
    x = rng.standard_normal((cfg.n_nodes, c_x))
    w = draw_weights(rng, w_blocks) if w_blocks is not None else None
    z_bar = None
    force_c = None
    if cfg.cotangent == "normal":
        if z_dim is not None:
            z_bar = rng.standard_normal((cfg.n_nodes, z_dim))
    elif cfg.cotangent == "energy":
        if scalar_out_mask is not None:
            z_bar = np.broadcast_to(scalar_out_mask.astype(np.float64), (cfg.n_nodes, scalar_out_mask.shape[0])).copy()
        force_c = rng.standard_normal((cfg.n_nodes, 3))
    else:
        raise ValueError(cfg.cotangent)
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)  # noqa: E731
    return Workload(cfg=cfg, pos=f32(pos), src=src.astype(np.int32), dst=dst.astype(np.int32),
                    x=f32(x), w=f32(w), z_bar=f32(z_bar), force_c=f32(force_c))


def scalar_mask(irreps_out: str) -> np.ndarray:
    """True on the columns of 0e output blocks (layout only)."""
    irr = parse_irreps(irreps_out)
    mask = np.zeros(irreps_dim(irr), dtype=bool)
    for (mul, l, p), off in zip(irr, irreps_offsets(irr)):
        if l == 0 and p == 1:
            mask[off:off + mul] = True
    return mask
