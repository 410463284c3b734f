"""Small workloads for oracle self-checks (CPU, seconds)."""
import dataclasses

import numpy as np

from oracle import conv
from workloads import CONFIGS, make_workload


def tiny_config(base="cfg1", **kw):
    c = CONFIGS[base]
    return dataclasses.replace(c, **kw)


def tiny_workload(cfg, with_cot=True):
    spec = conv.spec_from_config(cfg)
    wl = make_workload(cfg, w_blocks=spec.plan.w_blocks(), z_dim=spec.plan.z_dim if with_cot else None)
    return spec, wl


def o3_transform_features(x, irreps, D_of_l, det):
    """Apply an O(3) element to an ir_mul feature matrix [N, dim]."""
    out = np.empty_like(x)
    off = 0
    for mul, l, par in irreps:
        n = 2 * l + 1
        blk = x[:, off:off + n * mul].reshape(-1, n, mul)
        s = par if det < 0 else 1
        out[:, off:off + n * mul] = (s * np.einsum("mn,Nnu->Nmu", D_of_l(l), blk)).reshape(x.shape[0], -1)
        off += n * mul
    return out
