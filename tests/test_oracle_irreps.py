"""Pins for oracle/irreps.py: path counts and widths fixed by Eq. 4, 5, 9-10."""
import pytest

from oracle import irreps as ir
from workloads import CONFIGS

# (paths, sum over paths of (2l_out+1), x_dim, z_dim, |W|) counted by hand from Eq. 5
EXPECT = {
    "cfg1": (7, 21, 32, 72, 3584),
    "cfg2": (17, 71, 576, 1024, 557056),
    "cfg3": (23, 99, 2048, 12672, 47104),
    "cfg4_d16": (11, 35, 288, 288, 90112),
    "cfg5": (11, 35, 576, 576, 360448),
}


@pytest.mark.parametrize("name", sorted(EXPECT))
def test_config_plans(name):
    c = CONFIGS[name]
    plan = ir.make_plan(c.irreps_in, c.irreps_out, c.lmax_sh, c.mode, c.n_basis, out_per_path=c.out_per_path)
    n, so, xd, zd, wn = EXPECT[name]
    assert len(plan.paths) == n
    assert sum(2 * p.l_out + 1 for p in plan.paths) == so
    assert (plan.x_dim, plan.z_dim, plan.w_numel) == (xd, zd, wn)
    keys = [(p.out_block, p.in_block, p.l_sh) for p in plan.paths]
    assert keys == sorted(keys)
    off = 0
    for p in plan.paths:
        assert p.w_off == off
        off += p.w_numel


def test_cfg2_first_paths_by_hand():
    plan = ir.make_plan("64x0e+64x1o+64x2e", "64x0e+64x1o+64x2e+64x3o", 3, "uvw", 8)
    # output 0e receives 0e x Y0, 1o x Y1, 2e x Y2
    got = [(p.in_block, p.l_sh) for p in plan.paths if p.out_block == 0]
    assert got == [(0, 0), (1, 1), (2, 2)]
    # output 3o receives 0e x Y3, 1o x Y2, 2e x Y1, 2e x Y3
    got = [(p.in_block, p.l_sh) for p in plan.paths if p.out_block == 3]
    assert got == [(0, 3), (1, 2), (2, 1), (2, 3)]
    assert plan.fan_in(plan.paths[0]) == 8 * 3 * 64


def test_selection_rule_violations_rejected():
    with pytest.raises(ValueError):
        ir.make_plan("4x0e", "4x1e", 1, "uvw", 4, instructions=[(0, 1, 0)])  # parity
    with pytest.raises(ValueError):
        ir.make_plan("4x0e", "4x2e", 1, "uvw", 4, instructions=[(0, 1, 0)])  # triangle
    with pytest.raises(ValueError):
        ir.make_plan("4x0e", "8x0e", 0, "uvu", 4, instructions=[(0, 0, 0)])  # uvu width
