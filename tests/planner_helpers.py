"""Build a library plan from a workload description (test/bench helper)."""
from equivariant_gnn_tensor_amd import Plan


def plan_from_config(cfg, gemm_precision="fp32", lanes=0):
    return Plan(cfg.irreps_in, cfg.irreps_out, cfg.lmax_sh, cfg.mode, cfg.radial, cfg.n_basis, cfg.r_lo, cfg.r_hi,
                cfg.poly_p, box=cfg.box, out_per_path=cfg.out_per_path, gemm_precision=gemm_precision, lanes=lanes)
