"""Pins for oracle/layout.py: a hand-indexed example, identities, round trips."""
import numpy as np

from oracle import irreps as oi
from oracle import layout


def test_hand_indexed_example():
    # 1x0e + 2x1o: width 1 + 6.  mul_ir: [s, (u0: m0 m1 m2), (u1: m0 m1 m2)]
    #                           ir_mul: [s, (m0: u0 u1), (m1: u0 u1), (m2: u0 u1)]
    ir = oi.parse("1x0e+2x1o")
    mul_ir = np.array([[9, 10, 11, 12, 20, 21, 22]], np.float32)
    want = np.array([[9, 10, 20, 11, 21, 12, 22]], np.float32)
    assert np.array_equal(layout.mul_ir_to_ir_mul(mul_ir, ir), want)
    assert np.array_equal(layout.ir_mul_to_mul_ir(want, ir), mul_ir)


def test_identity_on_scalars_and_single_channels():
    rng = np.random.default_rng(1)
    ir = oi.parse("7x0e+1x1o+1x2e+3x0o+1x3o")
    only_scalar_or_single = rng.standard_normal((4, oi.dim(ir)))
    assert np.array_equal(layout.mul_ir_to_ir_mul(only_scalar_or_single, ir), only_scalar_or_single)


def test_round_trips():
    rng = np.random.default_rng(2)
    ir = oi.parse("64x0e+64x1o+32x2e+16x3o")
    x = rng.standard_normal((5, oi.dim(ir)))
    a = layout.mul_ir_to_ir_mul(x, ir)
    assert np.array_equal(layout.ir_mul_to_mul_ir(a, ir), x)
    assert np.array_equal(layout.mul_ir_to_ir_mul(layout.ir_mul_to_mul_ir(x, ir), ir), x)
    assert not np.array_equal(a, x)


def test_element_positions():
    # component m of channel u of block k: mul_ir column off + u (2l+1) + m, ir_mul off + m C + u
    ir = oi.parse("3x0e+5x2e+4x1o")
    offs = oi.offsets(ir)
    n = oi.dim(ir)
    x = np.arange(n, dtype=np.float64)[None, :]
    y = layout.mul_ir_to_ir_mul(x, ir)
    for (mul, l, _), off in zip(ir, offs):
        d = 2 * l + 1
        for u in range(mul):
            for m in range(d):
                assert y[0, off + m * mul + u] == off + u * d + m
