"""ctypes binding of libetpc.so (argument marshalling only).

Every computation runs in the HIP library; this module converts Python/torch
arguments to the C ABI of ``include/etpc.h`` and allocates caller-owned buffers
(outputs, workspaces) with torch on the current device.  Function names mirror
the C entry points.  If the shared library is missing, importing this module
raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_LIB_PATH = os.environ.get("ETPC_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                                                            "libetpc.so")

ETPC_OK = 0
UVW, UVU = 0, 1
GAUSSIAN, BESSEL = 0, 1
PASS_FWD, PASS_BWD, PASS_DBL = 0, 1, 2
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "INVALID_PATH", 4: "WORKSPACE", 5: "OVERFLOW",
           6: "GRAPH", 7: "HIP", 8: "CAPACITY"}
ERR_CAPACITY = 8
TO_IR_MUL, TO_MUL_IR = 0, 1
FEATURES_IN, FEATURES_OUT = 0, 1
GEMM_FP32, GEMM_BF16, GEMM_FP16 = 0, 1, 2
SEND_ORDER_WINDOW, RECV_ORDER_WINDOW = 4096, 512   # ETPC_SEND_ORDER_WINDOW, ETPC_RECV_ORDER_WINDOW


class EtpcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"etpc {_STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


class etpc_irrep(C.Structure):
    _fields_ = [("mul", C.c_int32), ("l", C.c_int32), ("parity", C.c_int32)]


class etpc_instr(C.Structure):
    _fields_ = [("in_block", C.c_int32), ("l_sh", C.c_int32), ("out_block", C.c_int32)]


class etpc_spec(C.Structure):
    _fields_ = [
        ("n_in", C.c_int32), ("in_", C.POINTER(etpc_irrep)),
        ("n_out", C.c_int32), ("out", C.POINTER(etpc_irrep)),
        ("out_per_path", C.c_int32), ("lmax_sh", C.c_int32), ("mode", C.c_int32),
        ("n_instr", C.c_int32), ("instr", C.POINTER(etpc_instr)),
        ("radial", C.c_int32), ("n_basis", C.c_int32), ("r_lo", C.c_float), ("r_hi", C.c_float),
        ("poly_p", C.c_int32), ("box", C.c_float * 3), ("gemm_precision", C.c_int32), ("lanes", C.c_int32),
    ]


class etpc_graph(C.Structure):
    _fields_ = [
        ("n_nodes", C.c_int32), ("n_edges", C.c_int64),
        ("rowptr", C.c_void_p), ("col", C.c_void_p),
        ("s_rowptr", C.c_void_p), ("s_col", C.c_void_p), ("s_slot", C.c_void_p), ("s_order", C.c_void_p),
        ("r_order", C.c_void_p),
    ]


SYMBOLS = (
    "etpc_plan_create", "etpc_plan_destroy", "etpc_plan_info", "etpc_plan_path", "etpc_plan_out_irrep",
    "etpc_plan_cg", "etpc_workspace_size", "etpc_csr_workspace_size", "etpc_csr_build", "etpc_graph_validate",
    "etpc_forward", "etpc_forward_noalloc", "etpc_backward", "etpc_double_backward",
    "etpc_profile_enable", "etpc_profile_read", "etpc_radius_graph_workspace_size", "etpc_radius_graph",
    "etpc_layout_convert", "etpc_last_error", "etpc_degree_order_workspace_size", "etpc_degree_order",
    "etpc_degree_order_within", "etpc_spatial_order_workspace_size", "etpc_spatial_order",
)
KINDS = ("csr", "fwd_traverse", "channel_gemm", "bwd_traverse", "node_gemm", "aux", "prep")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built (python equivariant_gnn_tensor_amd/build.py)")
    lib = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    P = C.POINTER
    lib.etpc_last_error.restype = C.c_char_p
    lib.etpc_last_error.argtypes = []
    sig = {
        "etpc_plan_create": [P(etpc_spec), P(vp)],
        "etpc_plan_info": [vp, P(i64), P(i64), P(i64), P(i32)],
        "etpc_plan_path": [vp, i32, P(i32), P(i32), P(i32), P(i32), P(i32), P(i64), P(i64), P(i64), P(i64),
                           P(i32)],
        "etpc_plan_out_irrep": [vp, i32, P(i32), P(etpc_irrep)],
        "etpc_plan_cg": [vp, i32, P(C.c_double)],
        "etpc_workspace_size": [vp, i32, i32, i64, sz, P(sz)],
        "etpc_csr_workspace_size": [i32, i64, P(sz)],
        "etpc_csr_build": [i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "etpc_graph_validate": [P(etpc_graph), vp],
        "etpc_degree_order_workspace_size": [i32, P(sz)],
        "etpc_degree_order": [i32, vp, i32, vp, vp, sz, vp],
        "etpc_degree_order_within": [i32, vp, i32, vp, vp, vp, sz, vp],
        "etpc_spatial_order_workspace_size": [i32, P(sz)],
        "etpc_spatial_order": [i32, vp, P(C.c_float), vp, vp, sz, vp],
        "etpc_forward": [vp, P(etpc_graph), vp, vp, vp, vp, vp, sz, vp],
        "etpc_forward_noalloc": [vp, P(etpc_graph), vp, vp, vp, vp, vp],
        "etpc_backward": [vp, P(etpc_graph), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "etpc_double_backward": [vp, P(etpc_graph), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "etpc_profile_enable": [i32],
        "etpc_profile_read": [i32, P(C.c_double), P(i64)],
        "etpc_radius_graph_workspace_size": [i32, i64, P(sz)],
        "etpc_radius_graph": [i32, vp, C.c_float, P(C.c_float), i64, vp, vp, P(i64), vp, sz, vp],
        "etpc_layout_convert": [vp, i32, i32, i32, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.etpc_plan_destroy.argtypes = [vp]
    lib.etpc_plan_destroy.restype = None
    return lib


lib = _load()


def _check(status: int):
    if status != ETPC_OK:
        raise EtpcError(status, lib.etpc_last_error().decode())


_TOK = re.compile(r"^\s*(?:(\d+)\s*x\s*)?(\d+)([eo])\s*$")


def parse_irreps(s) -> List[Tuple[int, int, int]]:
    if not isinstance(s, str):
        return [tuple(t) for t in s]
    out = []
    for tok in s.split("+"):
        m = _TOK.match(tok)
        if not m:
            raise ValueError(f"bad irrep token {tok!r}")
        out.append((int(m.group(1) or 1), int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def _ptr(t: Optional[torch.Tensor], dtype=torch.float32) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _torch_stream(stream, device):
    """The torch stream object of a call's stream (current stream, a torch stream, or a raw
    HIP stream handle)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _check_shape(name: str, t: Optional[torch.Tensor], shape: Tuple[int, ...], device=None):
    """Raise ValueError unless t is None or has exactly `shape` (and lives on `device`)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class Plan:
    """Owns an etpc_plan handle (host tables only)."""

    def __init__(self, irreps_in, irreps_out, lmax_sh: int, mode: str = "uvw", radial: str = "gaussian",
                 n_basis: int = 8, r_lo: float = 0.0, r_hi: float = 5.0, poly_p: int = 6,
                 box: Optional[Sequence[float]] = None, out_per_path: bool = False,
                 instructions: Optional[Sequence[Tuple[int, int, int]]] = None, gemm_precision: str = "fp32",
                 lanes: int = 0):
        ins, outs = parse_irreps(irreps_in), parse_irreps(irreps_out)
        self.irreps_in = ins
        self._in = (etpc_irrep * len(ins))(*[etpc_irrep(*t) for t in ins])
        self._out = (etpc_irrep * len(outs))(*[etpc_irrep(*t) for t in outs])
        n_instr = 0 if instructions is None else len(instructions)
        self._instr = (etpc_instr * max(1, n_instr))(*[etpc_instr(*t) for t in (instructions or [])])
        spec = etpc_spec()
        spec.n_in, spec.in_ = len(ins), self._in
        spec.n_out, spec.out = len(outs), self._out
        spec.out_per_path = 1 if out_per_path else 0
        spec.lmax_sh = lmax_sh
        spec.mode = {"uvw": UVW, "uvu": UVU}[mode] if isinstance(mode, str) else int(mode)
        spec.n_instr = n_instr
        spec.instr = self._instr if n_instr else None
        spec.radial = {"gaussian": GAUSSIAN, "bessel": BESSEL}[radial] if isinstance(radial, str) else int(radial)
        spec.n_basis, spec.r_lo, spec.r_hi, spec.poly_p = n_basis, r_lo, r_hi, poly_p
        b = (0.0, 0.0, 0.0) if box is None else (tuple(box) if hasattr(box, "__len__") else (box, box, box))
        spec.box = (C.c_float * 3)(*b)
        spec.gemm_precision = {"fp32": GEMM_FP32, "bf16": GEMM_BF16, "fp16": GEMM_FP16}[gemm_precision]
        spec.lanes = int(lanes)
        self.spec = spec
        self.handle = C.c_void_p()
        self.handle = etpc_plan_create(spec)
        self.mode = "uvw" if spec.mode == UVW else "uvu"

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            lib.etpc_plan_destroy(h)
            self.handle = None

    def info(self) -> Dict[str, int]:
        return etpc_plan_info(self)

    def paths(self) -> List[Dict[str, int]]:
        return [etpc_plan_path(self, p) for p in range(self.info()["n_paths"])]

    def out_irreps(self) -> List[Tuple[int, int, int]]:
        return etpc_plan_out_irrep(self)

    def cg(self, p: int):
        return etpc_plan_cg(self, p)

    def w_blocks(self) -> List[Tuple[int, float]]:
        return [(q["w_numel"], 1.0 / q["fan_in"] ** 0.5) for q in self.paths()]


def etpc_plan_create(spec: etpc_spec) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib.etpc_plan_create(C.byref(spec), C.byref(h)))
    return h


def etpc_plan_info(plan: Plan) -> Dict[str, int]:
    x, z, w = C.c_int64(), C.c_int64(), C.c_int64()
    n = C.c_int32()
    _check(lib.etpc_plan_info(plan.handle, C.byref(x), C.byref(z), C.byref(w), C.byref(n)))
    return dict(x_dim=x.value, z_dim=z.value, w_numel=w.value, n_paths=n.value)


def etpc_plan_path(plan: Plan, p: int) -> Dict[str, int]:
    ib, ls, ob, li, lo, fi = (C.c_int32() for _ in range(6))
    xo, zo, wo, wn = (C.c_int64() for _ in range(4))
    _check(lib.etpc_plan_path(plan.handle, p, C.byref(ib), C.byref(ls), C.byref(ob), C.byref(li), C.byref(lo),
                              C.byref(xo), C.byref(zo), C.byref(wo), C.byref(wn), C.byref(fi)))
    return dict(in_block=ib.value, l_sh=ls.value, out_block=ob.value, l_in=li.value, l_out=lo.value,
                x_off=xo.value, z_off=zo.value, w_off=wo.value, w_numel=wn.value, fan_in=fi.value)


def etpc_plan_out_irrep(plan: Plan) -> List[Tuple[int, int, int]]:
    n = C.c_int32()
    _check(lib.etpc_plan_out_irrep(plan.handle, 0, C.byref(n), None))
    out = []
    for b in range(n.value):
        ir = etpc_irrep()
        _check(lib.etpc_plan_out_irrep(plan.handle, b, None, C.byref(ir)))
        out.append((ir.mul, ir.l, ir.parity))
    return out


def etpc_plan_cg(plan: Plan, p: int):
    import numpy as np
    q = etpc_plan_path(plan, p)
    li, ls, lo = q["l_in"], q["l_sh"], q["l_out"]
    buf = (C.c_double * ((2 * li + 1) * (2 * ls + 1) * (2 * lo + 1)))()
    _check(lib.etpc_plan_cg(plan.handle, p, buf))
    return np.array(buf[:], dtype=np.float64).reshape(2 * li + 1, 2 * ls + 1, 2 * lo + 1)


def parse_irreps_of(plan: Plan, which: str) -> List[Tuple[int, int, int]]:
    arr, n = (plan.spec.in_, plan.spec.n_in) if which == "in" else (plan.spec.out, plan.spec.n_out)
    return [(arr[i].mul, arr[i].l, arr[i].parity) for i in range(n)]


def etpc_workspace_size(plan: Plan, pass_: int, n_nodes: int, n_edges: int, budget: int = 0) -> int:
    """Workspace bytes of a pass; budget > 0 caps the node-state scratch (node chunks)."""
    b = C.c_size_t()
    _check(lib.etpc_workspace_size(plan.handle, pass_, n_nodes, n_edges, int(budget), C.byref(b)))
    return b.value


def etpc_csr_workspace_size(n_nodes: int, n_edges: int) -> int:
    b = C.c_size_t()
    _check(lib.etpc_csr_workspace_size(n_nodes, n_edges, C.byref(b)))
    return b.value


class Graph:
    """Device CSR views (receiver and sender) of one graph."""

    def __init__(self, n_nodes: int, rowptr, col, s_rowptr, s_col, s_slot, eid=None, s_order=None, r_order=None):
        self.n_nodes = int(n_nodes)
        self.rowptr, self.col, self.eid = rowptr, col, eid
        self.s_rowptr, self.s_col, self.s_slot = s_rowptr, s_col, s_slot
        self.s_order, self.r_order = s_order, r_order
        self.n_edges = int(col.shape[0])
        g = etpc_graph()
        g.n_nodes, g.n_edges = self.n_nodes, self.n_edges
        g.rowptr = _ptr(rowptr, torch.int32)
        g.col = _ptr(col, torch.int32) if self.n_edges else None
        g.s_rowptr = _ptr(s_rowptr, torch.int32)
        g.s_col = _ptr(s_col, torch.int32) if self.n_edges else None
        g.s_slot = _ptr(s_slot, torch.int32) if self.n_edges else None
        g.s_order = _ptr(s_order, torch.int32) if s_order is not None and self.n_nodes else None
        g.r_order = _ptr(r_order, torch.int32) if r_order is not None and self.n_nodes else None
        self.c = g

    def without_order(self) -> "Graph":
        """The same views with s_order and r_order unset (nodes dispatched in index order)."""
        return Graph(self.n_nodes, self.rowptr, self.col, self.s_rowptr, self.s_col, self.s_slot, eid=self.eid)


def _empty_i32(n, device):
    return torch.empty(max(n, 0), dtype=torch.int32, device=device)


def _workspace(nbytes: int, device, stream=None) -> Tuple[Optional[torch.Tensor], int]:
    """A library-call scratch buffer, allocated on the call's stream so that the caching
    allocator does not hand its memory out again before that stream's kernels are done
    with it (it is dropped as soon as the call has been enqueued)."""
    if nbytes <= 0:
        return None, 0
    with torch.cuda.stream(_torch_stream(stream, device)):
        t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, nbytes


def etpc_csr_build(n_nodes: int, src: torch.Tensor, dst: torch.Tensor, stream=None, order: bool = True,
                   pos: torch.Tensor = None, box=None) -> Graph:
    """Both CSR views of the COO list; with `order`, also the sender and receiver
    dispatch orders (etpc_degree_order of s_rowptr and rowptr, or, given positions,
    etpc_degree_order_within along their etpc_spatial_order, box = periodic lengths or None)."""
    dev = src.device
    e = int(src.shape[0])
    _check_shape("dst", dst, (e,), dev)
    rowptr, s_rowptr = _empty_i32(n_nodes + 1, dev), _empty_i32(n_nodes + 1, dev)
    col, eid, s_col, s_slot = (_empty_i32(e, dev) for _ in range(4))
    ws, nb = _workspace(etpc_csr_workspace_size(n_nodes, e), dev, stream)
    _check(lib.etpc_csr_build(n_nodes, e, _ptr(src, torch.int32), _ptr(dst, torch.int32), _ptr(rowptr, torch.int32),
                              _ptr(col, torch.int32), _ptr(eid, torch.int32), _ptr(s_rowptr, torch.int32),
                              _ptr(s_col, torch.int32), _ptr(s_slot, torch.int32),
                              None if ws is None else ws.data_ptr(), nb, _stream(stream)))
    base = etpc_spatial_order(pos, box, stream=stream) if (order and pos is not None) else None
    s_order = etpc_degree_order(s_rowptr, window=SEND_ORDER_WINDOW, base=base, stream=stream) if order else None
    r_order = etpc_degree_order(rowptr, window=RECV_ORDER_WINDOW, base=base, stream=stream) if order else None
    return Graph(n_nodes, rowptr, col, s_rowptr, s_col, s_slot, eid=eid, s_order=s_order, r_order=r_order)


def etpc_degree_order_workspace_size(n_nodes: int) -> int:
    b = C.c_size_t()
    _check(lib.etpc_degree_order_workspace_size(n_nodes, C.byref(b)))
    return b.value


def etpc_degree_order(rowptr: torch.Tensor, window: int = 0, base: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Nodes by decreasing row length rowptr[v+1] - rowptr[v], ties by index (int32 [N]);
    with window > 0, within each aligned window of that many nodes.  With `base` (a
    permutation, e.g. etpc_spatial_order), windows and ties follow the base sequence."""
    n = int(rowptr.shape[0]) - 1
    order = _empty_i32(n, rowptr.device)
    ws, nb = _workspace(etpc_degree_order_workspace_size(n), rowptr.device, stream)
    wsp = None if ws is None else ws.data_ptr()
    out = _ptr(order, torch.int32) if n > 0 else None
    if base is None:
        _check(lib.etpc_degree_order(n, _ptr(rowptr, torch.int32), window, out, wsp, nb, _stream(stream)))
    else:
        _check_shape("base", base, (n,), rowptr.device)
        _check(lib.etpc_degree_order_within(n, _ptr(rowptr, torch.int32), window, _ptr(base, torch.int32), out, wsp,
                                            nb, _stream(stream)))
    return order


def etpc_spatial_order_workspace_size(n_nodes: int) -> int:
    b = C.c_size_t()
    _check(lib.etpc_spatial_order_workspace_size(n_nodes, C.byref(b)))
    return b.value


def etpc_spatial_order(pos: torch.Tensor, box=None, stream=None) -> torch.Tensor:
    """Nodes by the Morton code of their position (int32 [N]): over the periodic box
    (box = three lengths) or the bounding box (box = None); ties by index."""
    n = int(pos.shape[0])
    _check_shape("pos", pos, (n, 3), pos.device)
    order = _empty_i32(n, pos.device)
    ws, nb = _workspace(etpc_spatial_order_workspace_size(n), pos.device, stream)
    bx = None if box is None else (C.c_float * 3)(*[float(v) for v in box])
    _check(lib.etpc_spatial_order(n, _ptr(pos, torch.float32) if n > 0 else None, bx,
                                  _ptr(order, torch.int32) if n > 0 else None,
                                  None if ws is None else ws.data_ptr(), nb, _stream(stream)))
    return order


def etpc_graph_validate(graph: Graph, stream=None) -> None:
    _check(lib.etpc_graph_validate(C.byref(graph.c), _stream(stream)))


def etpc_radius_graph_workspace_size(n_nodes: int, max_edges: int) -> int:
    b = C.c_size_t()
    _check(lib.etpc_radius_graph_workspace_size(n_nodes, max_edges, C.byref(b)))
    return b.value


def etpc_radius_graph(pos: torch.Tensor, cutoff: float, box=None, max_edges: Optional[int] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(src, dst) int32 device tensors of the radius graph, sorted by (receiver, sender).

    Without max_edges the capacity starts at 64 edges per node; when the library reports
    that it was too small, the buffers are re-allocated at the returned size and the call
    is made once more."""
    n = int(pos.shape[0])
    dev = pos.device
    cap = int(max_edges) if max_edges is not None else 64 * n
    box_c = None if box is None else (C.c_float * 3)(*[float(b) for b in box])
    for attempt in range(2):
        src, dst = _empty_i32(cap, dev), _empty_i32(cap, dev)
        ws, nb = _workspace(etpc_radius_graph_workspace_size(n, cap), dev, stream)
        ne = C.c_int64()
        st = lib.etpc_radius_graph(n, _ptr(pos), float(cutoff), box_c, cap, _ptr(src, torch.int32),
                                   _ptr(dst, torch.int32), C.byref(ne), None if ws is None else ws.data_ptr(), nb,
                                   _stream(stream))
        if st == ERR_CAPACITY and max_edges is None and attempt == 0:
            cap = int(ne.value)
            continue
        _check(st)
        e = int(ne.value)
        return src[:e], dst[:e]
    raise AssertionError("unreachable")


def etpc_layout_convert(plan: Plan, features: str, direction: str, x: torch.Tensor, out=None,
                        stream=None) -> torch.Tensor:
    """features: "in" (x-like rows) or "out" (z-like rows); direction: "to_ir_mul" or "to_mul_ir"."""
    f = {"in": FEATURES_IN, "out": FEATURES_OUT}[features]
    d = {"to_ir_mul": TO_IR_MUL, "to_mul_ir": TO_MUL_IR}[direction]
    if out is None:
        out = torch.empty_like(x)
    _check_shape("out", out, tuple(x.shape), x.device)
    _check(lib.etpc_layout_convert(plan.handle, f, d, int(x.shape[0]) if x.dim() else 0, _ptr(x), _ptr(out),
                                   _stream(stream)))
    return out


def _ws_for(plan, pass_, graph, ws, stream, budget=0):
    if isinstance(ws, torch.Tensor):
        return ws.data_ptr(), ws.numel() * ws.element_size(), ws
    n = etpc_workspace_size(plan, pass_, graph.n_nodes, graph.n_edges, budget)
    t, nb = _workspace(n, graph.rowptr.device, stream)
    return (None if t is None else t.data_ptr()), nb, t


def _check_inputs(plan: Plan, graph: Graph, x, pos, w, z_bar=None, **extra):
    """Shapes of the dense operands against the plan and the graph (the library reads and
    writes exactly these extents, so a wrong size would be an out-of-bounds access)."""
    info = plan.info()
    N, dev = graph.n_nodes, graph.rowptr.device
    shapes = dict(x=(N, info["x_dim"]), pos=(N, 3), w=(info["w_numel"],), z_bar=(N, info["z_dim"]),
                  z=(N, info["z_dim"]), x_bar=(N, info["x_dim"]), w_bar=(info["w_numel"],), pos_bar=(N, 3),
                  x_dot=(N, info["x_dim"]), w_dot=(info["w_numel"],), pos_dot=(N, 3),
                  z_bar_grad=(N, info["z_dim"]), x_grad=(N, info["x_dim"]), w_grad=(info["w_numel"],),
                  pos_grad=(N, 3))
    for name, t in dict(x=x, pos=pos, w=w, z_bar=z_bar, **extra).items():
        _check_shape(name, t, shapes[name], dev)
    return info


def etpc_forward(plan: Plan, graph: Graph, x, pos, w, z=None, ws=None, stream=None, budget: int = 0):
    """z = conv(x, pos, W).  Without ws, a workspace is allocated for the call: the fast
    schedule's size, or the largest that fits `budget` bytes (the bounded schedule)."""
    _check_inputs(plan, graph, x, pos, w, z=z)
    if z is None:
        with torch.cuda.stream(_torch_stream(stream, x.device)):
            z = torch.empty(graph.n_nodes, plan.info()["z_dim"], dtype=torch.float32, device=x.device)
    wp, wn, _keep = _ws_for(plan, PASS_FWD, graph, ws, stream, budget)
    _check(lib.etpc_forward(plan.handle, C.byref(graph.c), _ptr(x), _ptr(pos), _ptr(w), _ptr(z), wp, wn,
                            _stream(stream)))
    return z


def etpc_forward_noalloc(plan: Plan, graph: Graph, x, pos, w, z, stream=None):
    """Forward into a caller-given z using the library's fixed device scratch: allocates
    nothing (not even here: z must be given).  Calls that overlap on one GPU race."""
    _check_inputs(plan, graph, x, pos, w, z=z)
    if z is None:
        raise ValueError("etpc_forward_noalloc writes into a caller-given z")
    _check(lib.etpc_forward_noalloc(plan.handle, C.byref(graph.c), _ptr(x), _ptr(pos), _ptr(w), _ptr(z),
                                    _stream(stream)))
    return z


def etpc_backward(plan: Plan, graph: Graph, x, pos, w, z_bar, want=("x", "w", "pos"), outs=None, ws=None,
                  stream=None, budget: int = 0):
    info = _check_inputs(plan, graph, x, pos, w, z_bar)
    dev = x.device
    if outs is None:
        with torch.cuda.stream(_torch_stream(stream, dev)):
            outs = (
                torch.empty(graph.n_nodes, info["x_dim"], dtype=torch.float32, device=dev) if "x" in want else None,
                torch.empty(info["w_numel"], dtype=torch.float32, device=dev) if "w" in want else None,
                torch.empty(graph.n_nodes, 3, dtype=torch.float32, device=dev) if "pos" in want else None,
            )
    xb, wb, pb = outs
    _check_inputs(plan, graph, x, pos, w, z_bar, x_bar=xb, w_bar=wb, pos_bar=pb)
    wp, wn, _keep = _ws_for(plan, PASS_BWD, graph, ws, stream, budget)
    _check(lib.etpc_backward(plan.handle, C.byref(graph.c), _ptr(x), _ptr(pos), _ptr(w), _ptr(z_bar), _ptr(xb),
                             _ptr(wb), _ptr(pb), wp, wn, _stream(stream)))
    return xb, wb, pb


def etpc_double_backward(plan: Plan, graph: Graph, x, pos, w, z_bar, x_dot=None, w_dot=None, pos_dot=None,
                         want=("z_bar", "x", "w", "pos"), outs=None, ws=None, stream=None, budget: int = 0):
    """Returns (d/dz_bar, d/dx, d/dW, d/dpos); outputs not in ``want`` are None."""
    info = _check_inputs(plan, graph, x, pos, w, z_bar, x_dot=x_dot, w_dot=w_dot, pos_dot=pos_dot)
    dev = x.device
    if outs is None:
        with torch.cuda.stream(_torch_stream(stream, dev)):
            outs = (
                torch.empty(graph.n_nodes, info["z_dim"], dtype=torch.float32, device=dev)
                if "z_bar" in want else None,
                torch.empty(graph.n_nodes, info["x_dim"], dtype=torch.float32, device=dev) if "x" in want else None,
                torch.empty(info["w_numel"], dtype=torch.float32, device=dev) if "w" in want else None,
                torch.empty(graph.n_nodes, 3, dtype=torch.float32, device=dev) if "pos" in want else None,
            )
    if len(outs) == 3:
        outs = tuple(outs) + (None,)
    gz, gx, gw, gp = outs
    _check_inputs(plan, graph, x, pos, w, z_bar, z_bar_grad=gz, x_grad=gx, w_grad=gw, pos_grad=gp)
    wp, wn, _keep = _ws_for(plan, PASS_DBL, graph, ws, stream, budget)
    _check(lib.etpc_double_backward(plan.handle, C.byref(graph.c), _ptr(x), _ptr(pos), _ptr(w), _ptr(z_bar),
                                    _ptr(x_dot), _ptr(w_dot), _ptr(pos_dot), _ptr(gz), _ptr(gx), _ptr(gw), _ptr(gp),
                                    wp, wn, _stream(stream)))
    return gz, gx, gw, gp


def etpc_profile_enable(enable: bool) -> None:
    _check(lib.etpc_profile_enable(1 if enable else 0))


def etpc_profile_read(kind) -> Tuple[float, int]:
    """(total milliseconds, launches) recorded for one kernel kind since the last enable."""
    k = KINDS.index(kind) if isinstance(kind, str) else int(kind)
    ms, n = C.c_double(), C.c_int64()
    _check(lib.etpc_profile_read(k, C.byref(ms), C.byref(n)))
    return ms.value, n.value
