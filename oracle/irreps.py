"""Irreps bookkeeping and path enumeration.

Follows the Sobek paper, Sec. 2: a feature field is a direct sum of irreps
(Eq. 3) of flattened width sum C (2l+1) (Eq. 4); a tensor-product path couples an
input irrep with a spherical-harmonic irrep into an output irrep allowed by the
Clebsch-Gordan selection rule (Eq. 5): |l_in - l_sh| <= l_out <= l_in + l_sh and
parity_out = parity_in * parity_sh, with the harmonic of degree l having parity
(-1)^l.  A uvw path has C_in * C_out weights per radial basis (Eq. 6, 9), a uvu
path C_in and requires C_out = C_in (Eq. 7).

Layout (ir_mul): irrep block k of a feature row is stored as [2l+1][C] with the
channel index fastest.  Weight storage: paths in plan order (out_block,
in_block, l_sh); each uvw path block is [B][C_in][C_out], each uvu block [B][C_in].

Pinned by tests/test_oracle_irreps.py (closed-form path counts and widths).
"""
from __future__ import annotations

import dataclasses
import re
from typing import List, Optional, Sequence, Tuple

Irrep = Tuple[int, int, int]   # (mul, l, parity +1/-1)

_TOK = re.compile(r"^\s*(?:(\d+)\s*x\s*)?(\d+)([eo])\s*$")


def parse(s: str) -> List[Irrep]:
    out = []
    for tok in s.split("+"):
        m = _TOK.match(tok)
        if not m:
            raise ValueError(tok)
        out.append((int(m.group(1) or 1), int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def dim(irreps: Sequence[Irrep]) -> int:
    return sum(mul * (2 * l + 1) for mul, l, _ in irreps)


def offsets(irreps: Sequence[Irrep]) -> List[int]:
    o, out = 0, []
    for mul, l, _ in irreps:
        out.append(o)
        o += mul * (2 * l + 1)
    return out


def selection_ok(l_in: int, p_in: int, l_sh: int, l_out: int, p_out: int) -> bool:
    """Eq. 5 with the harmonic's parity (-1)^l_sh."""
    return abs(l_in - l_sh) <= l_out <= l_in + l_sh and p_out == p_in * (-1) ** l_sh


@dataclasses.dataclass(frozen=True)
class Path:
    in_block: int
    l_sh: int
    out_block: int
    l_in: int
    l_out: int
    c_in: int
    c_out: int
    w_off: int
    w_numel: int


@dataclasses.dataclass
class Plan:
    irreps_in: List[Irrep]
    irreps_out: List[Irrep]
    lmax_sh: int
    mode: str
    n_basis: int
    paths: List[Path]

    @property
    def x_dim(self) -> int:
        return dim(self.irreps_in)

    @property
    def z_dim(self) -> int:
        return dim(self.irreps_out)

    @property
    def w_numel(self) -> int:
        return sum(p.w_numel for p in self.paths)

    def fan_in(self, p: Path) -> int:
        """uvw: B times the summed input multiplicity of the output group (D_g, Sec. 4)."""
        if self.mode == "uvw":
            return self.n_basis * sum(q.c_in for q in self.paths if q.out_block == p.out_block)
        return self.n_basis      # uvu: B * C_sh with C_sh = 1

    def w_blocks(self) -> List[Tuple[int, float]]:
        """(numel, std) per path block with std = 1/sqrt(fan_in)."""
        return [(p.w_numel, 1.0 / (self.fan_in(p) ** 0.5)) for p in self.paths]


def make_plan(irreps_in, irreps_out, lmax_sh: int, mode: str, n_basis: int,
              out_per_path: bool = False,
              instructions: Optional[Sequence[Tuple[int, int, int]]] = None) -> Plan:
    """Enumerate paths.

    irreps_out: explicit output irreps, or with ``out_per_path`` (uvu only) the
    allowed output (l, parity) list: one output block per valid
    (in_block, l_sh, allowed out) in that nested order, multiplicity = C_in.
    instructions: optional explicit (in_block, l_sh, out_block) list; default is
    every CG-valid triple.
    """
    if isinstance(irreps_in, str):
        irreps_in = parse(irreps_in)
    if isinstance(irreps_out, str):
        irreps_out = parse(irreps_out)
    if mode not in ("uvw", "uvu"):
        raise ValueError(mode)
    if out_per_path:
        if mode != "uvu":
            raise ValueError("per-path outputs are a uvu construction")
        allowed = [(l, p) for _, l, p in irreps_out]
        outs, instr = [], []
        for k, (mul, li, pi) in enumerate(irreps_in):
            for ls in range(lmax_sh + 1):
                for lo, po in allowed:
                    if selection_ok(li, pi, ls, lo, po):
                        instr.append((k, ls, len(outs)))
                        outs.append((mul, lo, po))
        irreps_out = outs
        instructions = instr
    if instructions is None:
        instructions = []
        for g, (_, lo, po) in enumerate(irreps_out):
            for k, (_, li, pi) in enumerate(irreps_in):
                for ls in range(lmax_sh + 1):
                    if selection_ok(li, pi, ls, lo, po):
                        instructions.append((k, ls, g))
    for k, ls, g in instructions:
        ci, li, pi = irreps_in[k]
        co, lo, po = irreps_out[g]
        if not (0 <= ls <= lmax_sh) or not selection_ok(li, pi, ls, lo, po):
            raise ValueError(f"instruction {(k, ls, g)} violates the selection rule")
        if mode == "uvu" and ci != co:
            raise ValueError("uvu requires C_out == C_in")
    order = sorted(set(instructions), key=lambda t: (t[2], t[0], t[1]))
    paths, off = [], 0
    for k, ls, g in order:
        ci, li, _ = irreps_in[k]
        co, lo, _ = irreps_out[g]
        n = n_basis * ci * co if mode == "uvw" else n_basis * ci
        paths.append(Path(k, ls, g, li, lo, ci, co, off, n))
        off += n
    return Plan(list(irreps_in), list(irreps_out), lmax_sh, mode, n_basis, paths)
