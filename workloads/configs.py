"""The synthetic workloads (sizes, irreps, radial basis, graph recipe).

Each workload stands in for one of the scaling sweeps of the Sobek paper
("Sobek: Streaming Equivariant Tensor Product Convolutions", Sec. 5: memory and
throughput scaling under degree and graph-count scaling).  The paper publishes
no dataset and no absolute workload; these are seeded synthetic graphs of the
stated shapes.  Irreps strings use the usual "MULxLP" notation (P = e/o).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    index: int                      # 1..5
    mode: str                       # "uvw" | "uvu"
    n_nodes: int
    graph: str                      # "indegree" | "radius"
    degree: int                     # in-degree for "indegree" graphs
    cutoff: float                   # radius-graph cutoff [A] (also Bessel cutoff)
    box: Optional[float]            # periodic cube side [A] or None (open)
    pos_extent: float               # positions drawn U[0, pos_extent)^3
    irreps_in: str
    irreps_out: str                 # for uvu per-path outputs: the allowed output irreps
    out_per_path: bool              # uvu: one output block per path, mult tied to input
    lmax_sh: int
    radial: str                     # "gaussian" | "bessel"
    n_basis: int
    r_lo: float
    r_hi: float
    poly_p: int
    passes: Tuple[str, ...]         # subset of ("fwd", "bwd", "dbl")
    cotangent: str                  # "normal" | "energy" (z_bar = 1 on 0e outputs)
    w_std: str                      # "fan_in" (1/sqrt(B * sum C_in of group)) | "uvu" (1/sqrt(B*C_sh))
    seed_k: int = 0
    n_graphs: int = 1               # > 1: that many independent radius graphs of n_nodes / n_graphs
                                    # atoms each (block-diagonal batch), all in the same box

    @property
    def seed(self) -> int:
        return 1000 + 10 * self.index + self.seed_k


def _box(n: int, density: float = 0.1) -> float:
    return (n / density) ** (1.0 / 3.0)


def _cfg1() -> WorkloadConfig:
    return WorkloadConfig(
        name="tiny_uvw_fwd", index=1, mode="uvw", n_nodes=64, graph="indegree", degree=8,
        cutoff=5.0, box=None, pos_extent=4.0,
        irreps_in="8x0e+8x1o", irreps_out="8x0e+8x1o+8x2e", out_per_path=False,
        lmax_sh=2, radial="gaussian", n_basis=8, r_lo=0.0, r_hi=5.0, poly_p=6,
        passes=("fwd",), cotangent="normal", w_std="fan_in")


def _cfg2(n: int = 4096) -> WorkloadConfig:
    L = _box(n)
    return WorkloadConfig(
        name="mace_uvw_fwd_bwd", index=2, mode="uvw", n_nodes=n, graph="radius", degree=0,
        cutoff=5.0, box=L, pos_extent=L,
        irreps_in="64x0e+64x1o+64x2e", irreps_out="64x0e+64x1o+64x2e+64x3o", out_per_path=False,
        lmax_sh=3, radial="bessel", n_basis=8, r_lo=0.0, r_hi=5.0, poly_p=6,
        passes=("fwd", "bwd"), cotangent="normal", w_std="fan_in")


def _cfg3(n: int = 16384) -> WorkloadConfig:
    L = _box(n)
    return WorkloadConfig(
        name="channelwise_uvu_fwd_bwd", index=3, mode="uvu", n_nodes=n, graph="radius", degree=0,
        cutoff=5.0, box=L, pos_extent=L,
        irreps_in="128x0e+128x1o+128x2e+128x3o", irreps_out="0e+1o+2e+3o", out_per_path=True,
        lmax_sh=3, radial="gaussian", n_basis=16, r_lo=0.0, r_hi=5.0, poly_p=6,
        passes=("fwd", "bwd"), cotangent="normal", w_std="uvu")


def _cfg4(degree: int, n: int = 32768) -> WorkloadConfig:
    k = {16: 0, 64: 1, 256: 2, 512: 3}.get(degree, 0)
    return WorkloadConfig(
        name=f"edge_sweep_uvw_d{degree}", index=4, mode="uvw", n_nodes=n, graph="indegree",
        degree=degree, cutoff=5.0, box=None, pos_extent=30.0,
        irreps_in="32x0e+32x1o+32x2e", irreps_out="32x0e+32x1o+32x2e", out_per_path=False,
        lmax_sh=2, radial="gaussian", n_basis=8, r_lo=0.0, r_hi=30.0 * math.sqrt(3.0), poly_p=6,
        passes=("fwd", "bwd"), cotangent="normal", w_std="fan_in", seed_k=k)


def _cfg5(n: int = 8192) -> WorkloadConfig:
    L = _box(n)
    return WorkloadConfig(
        name="force_dbl_uvw", index=5, mode="uvw", n_nodes=n, graph="radius", degree=0,
        cutoff=5.0, box=L, pos_extent=L,
        irreps_in="64x0e+64x1o+64x2e", irreps_out="64x0e+64x1o+64x2e", out_per_path=False,
        lmax_sh=2, radial="bessel", n_basis=8, r_lo=0.0, r_hi=5.0, poly_p=6,
        passes=("fwd", "bwd", "dbl"), cotangent="energy", w_std="fan_in")


GRAPH_COUNTS = (1, 4, 16, 64, 256, 511)


def _cfg6(n_graphs: int, atoms: int = 128) -> WorkloadConfig:
    """Graph-count scaling (Sobek Sec. 5): a batch of independent periodic cells of
    `atoms` atoms at 0.1 / A^3 (side 10.86 A > 2 x cutoff), MACE-like features."""
    L = _box(atoms)
    return WorkloadConfig(
        name=f"graph_count_uvw_b{n_graphs}", index=6, mode="uvw", n_nodes=atoms * n_graphs, graph="radius",
        degree=0, cutoff=5.0, box=L, pos_extent=L,
        irreps_in="64x0e+64x1o+64x2e", irreps_out="64x0e+64x1o+64x2e+64x3o", out_per_path=False,
        lmax_sh=3, radial="bessel", n_basis=8, r_lo=0.0, r_hi=5.0, poly_p=6,
        passes=("fwd", "bwd"), cotangent="normal", w_std="fan_in",
        seed_k=GRAPH_COUNTS.index(n_graphs) if n_graphs in GRAPH_COUNTS else 9, n_graphs=n_graphs)


CONFIGS = {
    "cfg1": _cfg1(),
    "cfg2": _cfg2(),
    "cfg3": _cfg3(),
    "cfg4_d16": _cfg4(16),
    "cfg4_d64": _cfg4(64),
    "cfg4_d256": _cfg4(256),
    "cfg4_d512": _cfg4(512),
    "cfg5": _cfg5(),
    **{f"cfg6_b{b}": _cfg6(b) for b in GRAPH_COUNTS},
}


def get_config(name: str) -> WorkloadConfig:
    return CONFIGS[name]


def small_variant(name: str, n_nodes: int, degree: Optional[int] = None) -> WorkloadConfig:
    """Same recipe at fewer nodes (radius graphs keep the density, so the box shrinks).

    Used for parity cases the oracle finishes in seconds.  Periodic boxes stay
    larger than twice the cutoff so the minimum image is unique.
    """
    c = CONFIGS[name]
    kw = {"n_nodes": n_nodes}
    if c.n_graphs > 1:
        raise ValueError("graph-count batches scale through n_graphs, not n_nodes")
    if c.graph == "radius":
        L = _box(n_nodes)
        if L <= 2.0 * c.cutoff:
            raise ValueError("box too small for the minimum-image convention")
        kw.update(box=L, pos_extent=L)
    if degree is not None:
        kw["degree"] = degree
    return dataclasses.replace(c, name=f"{c.name}_n{n_nodes}", **kw)
