"""Seeded synthetic workloads shared by the GPU path's tests/bench and the oracle.

This package holds only input *data*: the five workload descriptions and the
seeded random draws (positions, graphs, features, weights, cotangents).  It
contains none of the convolution's arithmetic (no spherical harmonics, no
Clebsch-Gordan coefficients, no radial bases, no path enumeration), so both the
HIP path and the CPU oracle can consume it without sharing method code.
"""
from .configs import CONFIGS, WorkloadConfig, get_config, small_variant  # noqa: F401
from .generate import (  # noqa: F401
    Workload,
    make_workload,
    parse_irreps,
    irreps_dim,
    irreps_offsets,
    draw_weights,
)
