"""Streaming edge-conditioned O(3) tensor-product convolution for MI355X (gfx950).

The compute path is the HIP library ``_lib/libetpc.so`` (C ABI in
``include/etpc.h``); this package is its thin Python binding.  Importing it
without the built library raises ImportError.
"""
from ._binding import (  # noqa: F401
    BESSEL, GAUSSIAN, KINDS, PASS_BWD, PASS_DBL, PASS_FWD, SYMBOLS, UVU, UVW,
    EtpcError, Graph, Plan,
    etpc_backward, etpc_csr_build, etpc_csr_workspace_size, etpc_double_backward, etpc_forward, etpc_forward_noalloc,
    etpc_graph_validate, etpc_plan_cg, etpc_plan_info, etpc_plan_out_irrep, etpc_plan_path,
    etpc_profile_enable, etpc_profile_read, etpc_workspace_size, lib, parse_irreps,
    etpc_layout_convert, etpc_radius_graph, etpc_radius_graph_workspace_size,
    etpc_degree_order, etpc_degree_order_workspace_size, RECV_ORDER_WINDOW, SEND_ORDER_WINDOW,
    etpc_spatial_order, etpc_spatial_order_workspace_size,
)
