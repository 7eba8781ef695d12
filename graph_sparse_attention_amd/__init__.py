"""Python binding of libgattn (fused graph sparse attention, MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libgattn.so``.  torch supplies device memory (``torch.empty``) and the
current stream.  Names follow the C ABI in ``include/gattn.h``:

    gattn_build_csr(src, dst, num_nodes)            -> (row_ptr, col_idx, edge_perm)
    gattn_build_rowwindows(row_ptr, col_idx, n)     -> RowWindows
    gattn_forward(row_ptr, col_idx, q, k, v, ...)   -> out [N, H, D]  (, e_out)
    gattn_build_hybrid(row_ptr, col_idx, rw, q)     -> Hybrid (per-window plan)
    gattn_forward_path(...)                         -> "gather" | "mfma" | "hybrid"
    gattn_forward_noalloc(row_ptr, col_idx, q, k, v, out, ...) -> out (no allocation)
    gattn_aggregate(row_ptr, col_idx, x, w, ...)    -> out [N, H, D]

and, on top of them, a graph object for callers that hold a COO edge list:

    g = Graph.from_coo(src, dst, num_nodes)         # CSR built on the device once
    g.rowwindows()                                  # the MFMA path's windows (built once)
    forward(g, q, k, v, e=None, mode=..., ...)      -> out [N, H, D]  (e in COO edge order)

Every call raises if ``libgattn.so`` is missing or stale: there is no
fallback implementation.  Build it with ``python -m
graph_sparse_attention_amd.build``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch  # loads the HIP runtime that libgattn.so then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GATTN_LIBRARY") or os.path.join(_HERE, "libgattn.so")

GATTN_OK, GATTN_ERR_INVALID_VALUE, GATTN_ERR_UNSUPPORTED, GATTN_ERR_BAD_GRAPH, \
    GATTN_ERR_DUPLICATE_EDGE, GATTN_ERR_BUFFER_TOO_SMALL, GATTN_ERR_HIP = range(7)
GATTN_F32, GATTN_F16, GATTN_BF16 = range(3)
GATTN_SOFTMAX_STANDARD, GATTN_SOFTMAX_CLIPPED = range(2)
GATTN_PATH_AUTO, GATTN_PATH_GATHER, GATTN_PATH_MFMA, GATTN_PATH_HYBRID = range(4)
GATTN_FLAG_VALIDATE = 1
GATTN_NOALLOC_SCRATCH_BYTES = 64 << 20

_DTYPES = {torch.float32: GATTN_F32, torch.float16: GATTN_F16, torch.bfloat16: GATTN_BF16}
_MODES = {"standard": GATTN_SOFTMAX_STANDARD, "clipped": GATTN_SOFTMAX_CLIPPED}
_PATHS = {"auto": GATTN_PATH_AUTO, "gather": GATTN_PATH_GATHER, "mfma": GATTN_PATH_MFMA, "hybrid": GATTN_PATH_HYBRID}
_PATH_NAMES = {GATTN_PATH_GATHER: "gather", GATTN_PATH_MFMA: "mfma", GATTN_PATH_HYBRID: "hybrid"}


class GattnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {gattn_status_string(status)} (status {status})")


class _RowWindows(ctypes.Structure):
    _fields_ = [("num_windows", ctypes.c_int32), ("num_cols", ctypes.c_int64),
                ("win_col_ptr", ctypes.c_void_p), ("win_cols", ctypes.c_void_p), ("tile_mask", ctypes.c_void_p)]


class _Hybrid(ctypes.Structure):
    _fields_ = [("num_dense", ctypes.c_int32), ("num_ranges", ctypes.c_int32), ("range_rows", ctypes.c_int32),
                ("dense_windows", ctypes.c_void_p), ("ranges", ctypes.c_void_p)]


class _ForwardArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("num_nodes", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("e", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("dtype", ctypes.c_int), ("mode", ctypes.c_int),
                ("scale", ctypes.c_float), ("clip_lo", ctypes.c_float), ("clip_hi", ctypes.c_float),
                ("eps", ctypes.c_float), ("path", ctypes.c_int), ("rw", ctypes.POINTER(_RowWindows)),
                ("flags", ctypes.c_uint32), ("edge_ids", ctypes.c_void_p), ("e_out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("hybrid", ctypes.POINTER(_Hybrid)), ("q_stride", ctypes.c_int64), ("kv_stride", ctypes.c_int64)]


class _AggregateArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("num_nodes", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("edge_ids", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("dtype", ctypes.c_int), ("normalize", ctypes.c_int32), ("eps", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class _Unloaded:
    """Stands in for a library that is missing, stale or unloadable: every use
    raises, so nothing can run without the HIP kernels (and the build script
    can still be imported to rebuild it)."""

    def __init__(self, err: Exception):
        self._err = err

    def __getattr__(self, name):
        raise ImportError(f"libgattn.so is not usable ({self._err}); "
                          "run `python -m graph_sparse_attention_amd.build`")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m graph_sparse_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    sz = ctypes.POINTER(ctypes.c_size_t)
    L.gattn_abi_version.restype = ctypes.c_int
    L.gattn_status_string.argtypes = [st]
    L.gattn_status_string.restype = ctypes.c_char_p
    L.gattn_build_csr_workspace.argtypes = [i32, i64, sz]
    L.gattn_build_csr.argtypes = [i32, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
    L.gattn_build_rowwindows_workspace.argtypes = [i32, i64, sz]
    L.gattn_build_rowwindows.argtypes = [i32, i64, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_int64), vp,
                                         ctypes.c_size_t, vp]
    L.gattn_forward.argtypes = [ctypes.POINTER(_ForwardArgs), vp]
    L.gattn_forward_path.argtypes = [ctypes.POINTER(_ForwardArgs), ctypes.POINTER(ctypes.c_int)]
    L.gattn_forward_noalloc.argtypes = [ctypes.POINTER(_ForwardArgs), vp]
    L.gattn_aggregate.argtypes = [ctypes.POINTER(_AggregateArgs), vp]
    L.gattn_forward_workspace.argtypes = [ctypes.POINTER(_ForwardArgs), sz]
    L.gattn_build_hybrid.argtypes = [ctypes.POINTER(_ForwardArgs), ctypes.c_float, vp, vp, ctypes.POINTER(_Hybrid), vp]
    L.gattn_aggregate_workspace.argtypes = [ctypes.POINTER(_AggregateArgs), sz]
    for f in (L.gattn_build_csr_workspace, L.gattn_build_csr, L.gattn_build_rowwindows_workspace,
              L.gattn_build_rowwindows, L.gattn_forward, L.gattn_forward_path, L.gattn_aggregate,
              L.gattn_forward_workspace, L.gattn_aggregate_workspace, L.gattn_build_hybrid, L.gattn_forward_noalloc):
        f.restype = st
    return L


try:
    _lib = _load()
except (ImportError, OSError, AttributeError) as _e:   # missing file, failed dlopen, missing symbol
    _lib = _Unloaded(_e)


def gattn_abi_version() -> int:
    return _lib.gattn_abi_version()


def gattn_status_string(status: int) -> str:
    return _lib.gattn_status_string(status).decode()


def _check(status: int, what: str):
    if status != GATTN_OK:
        raise GattnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32(t: torch.Tensor, name: str, device=None, numel=None) -> torch.Tensor:
    """A contiguous int32 GPU tensor, on `device` and of `numel` elements when
    given: the kernels read every index array over its full nominal length,
    so a short or misplaced one is refused here, before any launch."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor on the GPU")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t


def _csr(row_ptr, col_idx, num_nodes: int, device):
    """row_ptr [num_nodes + 1] and col_idx [nnz], int32, on `device`."""
    row_ptr = _i32(row_ptr, "row_ptr", device, num_nodes + 1)
    col_idx = _i32(col_idx, "col_idx", device)
    return row_ptr, col_idx


def gattn_build_csr(src: torch.Tensor, dst: torch.Tensor, num_nodes: int, validate: bool = True):
    """COO (src, dst) int32 on the GPU -> (row_ptr, col_idx, edge_perm),
    canonical order (destination, source, edge id).  validate=True checks
    indices and synchronizes; False keeps the call asynchronous (bad indices
    then give an unspecified CSR)."""
    src = _i32(src, "src")
    dev = src.device
    nnz = src.numel()
    dst = _i32(dst, "dst", dev, nnz)
    nbytes = ctypes.c_size_t()
    _check(_lib.gattn_build_csr_workspace(num_nodes, nnz, ctypes.byref(nbytes)), "gattn_build_csr_workspace")
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(num_nodes + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
    edge_perm = torch.empty(nnz, dtype=torch.int32, device=dev)
    status = None if validate else torch.empty(1, dtype=torch.int32, device=dev)
    _check(_lib.gattn_build_csr(num_nodes, nnz, _ptr(src), _ptr(dst), _ptr(row_ptr), _ptr(col_idx), _ptr(edge_perm),
                                _ptr(ws), nbytes.value, _ptr(status), _stream(dev)), "gattn_build_csr")
    return row_ptr, col_idx, edge_perm


class CsrBuilder:
    """Reusable buffers for repeated CSR builds of one graph size (no
    allocation per call); the device status is kept in ``status``."""

    def __init__(self, num_nodes: int, nnz: int, device):
        self.num_nodes, self.nnz = num_nodes, nnz
        nbytes = ctypes.c_size_t()
        _check(_lib.gattn_build_csr_workspace(num_nodes, nnz, ctypes.byref(nbytes)), "gattn_build_csr_workspace")
        self.ws_bytes = nbytes.value
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.row_ptr = torch.empty(num_nodes + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(nnz, dtype=torch.int32, device=device)
        self.edge_perm = torch.empty(nnz, dtype=torch.int32, device=device)
        self.status = torch.empty(1, dtype=torch.int32, device=device)

    def __call__(self, src: torch.Tensor, dst: torch.Tensor):
        src = _i32(src, "src", self.row_ptr.device, self.nnz)
        dst = _i32(dst, "dst", self.row_ptr.device, self.nnz)
        _check(_lib.gattn_build_csr(self.num_nodes, self.nnz, _ptr(src), _ptr(dst), _ptr(self.row_ptr),
                                    _ptr(self.col_idx), _ptr(self.edge_perm), _ptr(self.ws), self.ws_bytes,
                                    _ptr(self.status), _stream(src.device)), "gattn_build_csr")
        return self.row_ptr, self.col_idx, self.edge_perm


@dataclasses.dataclass
class RowWindows:
    num_nodes: int
    win_col_ptr: torch.Tensor   # int32 [W+1]
    win_cols: torch.Tensor      # int32 [C]
    tile_mask: torch.Tensor     # int16 bits [C/16, 16] (uint16 values)

    @property
    def num_windows(self):
        return self.win_col_ptr.numel() - 1

    @property
    def num_cols(self):
        return self.win_cols.numel()

    def _struct(self):
        return _RowWindows(self.num_windows, self.num_cols, self.win_col_ptr.data_ptr(),
                           self.win_cols.data_ptr() if self.num_cols else None,
                           self.tile_mask.data_ptr() if self.num_cols else None)


def gattn_build_rowwindows(row_ptr: torch.Tensor, col_idx: torch.Tensor, num_nodes: int) -> RowWindows:
    """16-row windows with 16x16 masked tiles (two calls of the C ABI)."""
    dev = row_ptr.device if isinstance(row_ptr, torch.Tensor) else None
    row_ptr, col_idx = _csr(row_ptr, col_idx, num_nodes, dev)
    nnz = col_idx.numel()
    nbytes = ctypes.c_size_t()
    _check(_lib.gattn_build_rowwindows_workspace(num_nodes, nnz, ctypes.byref(nbytes)),
           "gattn_build_rowwindows_workspace")
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    W = (num_nodes + 15) // 16
    wcp = torch.empty(W + 1, dtype=torch.int32, device=dev)
    ncols = ctypes.c_int64(0)
    _check(_lib.gattn_build_rowwindows(num_nodes, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(wcp), None, None,
                                       ctypes.byref(ncols), _ptr(ws), nbytes.value, _stream(dev)),
           "gattn_build_rowwindows (sizes)")
    C = ncols.value
    cols = torch.empty(max(C, 1), dtype=torch.int32, device=dev)
    mask = torch.empty(max(C, 1), dtype=torch.int16, device=dev)
    _check(_lib.gattn_build_rowwindows(num_nodes, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(wcp), _ptr(cols),
                                       _ptr(mask), ctypes.byref(ncols), _ptr(ws), nbytes.value, _stream(dev)),
           "gattn_build_rowwindows (fill)")
    return RowWindows(num_nodes, wcp, cols[:C], mask[:C].view(C // 16, 16) if C else mask[:0].view(0, 16))


@dataclasses.dataclass
class Hybrid:
    """Per-window dispatch plan of gattn_build_hybrid (device lists)."""
    num_dense: int
    num_ranges: int
    range_rows: int
    dense_windows: torch.Tensor   # int32 [ceil(N/16)], first num_dense used
    ranges: torch.Tensor          # int32 [2N], first 2*num_ranges used

    def _struct(self):
        return _Hybrid(self.num_dense, self.num_ranges, self.range_rows, self.dense_windows.data_ptr(),
                       self.ranges.data_ptr())


def gattn_build_hybrid(row_ptr: torch.Tensor, col_idx: torch.Tensor, rw: RowWindows, q: torch.Tensor,
                       min_density: float = 0.09) -> Hybrid:
    """Row windows whose tile density (edges / (16 * columns)) is at least
    min_density go to the MFMA path, the other rows to the gather path, in
    ranges sized like its workgroups.  q gives the geometry (N, H, D, dtype);
    the plan is for the standard mode without an edge tensor."""
    if q.dim() != 3 or not q.is_cuda or q.dtype not in _DTYPES:
        raise ValueError("q must be an [N, H, D] GPU tensor")
    N = q.shape[0]
    row_ptr, col_idx = _csr(row_ptr, col_idx, N, q.device)
    if rw.num_nodes != N or rw.win_col_ptr.device != q.device:
        raise ValueError("rw must be the row windows of this graph, on q's device")
    W = (N + 15) // 16
    dev = q.device
    dense = torch.empty(max(W, 1), dtype=torch.int32, device=dev)
    ranges = torch.empty(max(2 * N, 2), dtype=torch.int32, device=dev)
    a, keep = _forward_args(row_ptr, col_idx, q, q, q, None, None, "standard", None, (-5.0, 5.0), 1e-6, "hybrid", rw,
                            False)
    plan = _Hybrid()
    _check(_lib.gattn_build_hybrid(ctypes.byref(a), float(min_density), _ptr(dense), _ptr(ranges), ctypes.byref(plan),
                                   _stream(dev)), "gattn_build_hybrid")
    del keep
    return Hybrid(plan.num_dense, plan.num_ranges, plan.range_rows, dense, ranges)


def _forward_args(row_ptr, col_idx, q, k, v, e, out, mode, scale, clip, eps, path, rw, validate,
                  edge_ids=None, e_out=None, hybrid=None):
    N, H, D = q.shape
    a = _ForwardArgs()
    a.struct_size = ctypes.sizeof(_ForwardArgs)
    a.num_nodes, a.num_heads, a.head_dim = N, H, D
    a.nnz = col_idx.numel()
    a.row_ptr, a.col_idx = row_ptr.data_ptr(), col_idx.data_ptr()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.e = None if e is None else e.data_ptr()
    a.out = out.data_ptr() if out is not None else None
    a.dtype = _DTYPES[q.dtype]
    a.mode = _MODES[mode]
    a.scale = 1.0 / math.sqrt(D) if scale is None else scale
    a.clip_lo, a.clip_hi = clip
    a.eps = eps
    a.path = _PATHS[path]
    keep = []
    if rw is not None:
        keep.append(rw._struct())
        a.rw = ctypes.pointer(keep[-1])
    if hybrid is not None:
        keep.append(hybrid._struct())
        a.hybrid = ctypes.pointer(keep[-1])
    a.flags = GATTN_FLAG_VALIDATE if validate else 0
    a.edge_ids = None if edge_ids is None else edge_ids.data_ptr()
    a.e_out = None if e_out is None else e_out.data_ptr()
    a.q_stride = _row_stride(q)
    a.kv_stride = _row_stride(k)
    return a, keep


def _attach_workspace(a, query, workspace, device, what):
    """workspace: True -> allocate the queried size, a uint8 GPU tensor -> use
    it, None / False -> none (node partition)."""
    if workspace is None or workspace is False:
        return None
    nbytes = ctypes.c_size_t()
    _check(query(ctypes.byref(a), ctypes.byref(nbytes)), what)
    if nbytes.value == 0:
        return None
    if workspace is True:
        workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=device)
    elif workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < nbytes.value:
        raise ValueError(f"workspace must be a uint8 GPU tensor of at least {nbytes.value} bytes")
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return workspace


def gattn_forward_workspace(row_ptr, col_idx, q, k, v, e=None, mode="standard", e_out=False) -> int:
    """Bytes of the balanced-partition workspace for these tensors."""
    a, keep = _forward_args(row_ptr, col_idx, q, k, v, e, None, mode, None, (-5.0, 5.0), 1e-6, "gather", None,
                            False, None, None)
    if e_out:
        a.e_out = 256        # never dereferenced: only its presence sets the size
    nbytes = ctypes.c_size_t()
    _check(_lib.gattn_forward_workspace(ctypes.byref(a), ctypes.byref(nbytes)), "gattn_forward_workspace")
    del keep
    return nbytes.value


def gattn_aggregate_workspace(row_ptr, col_idx, x) -> int:
    """Bytes of the balanced-partition workspace of gattn_aggregate for these tensors."""
    N, H, D = x.shape
    a = _AggregateArgs()
    a.struct_size = ctypes.sizeof(_AggregateArgs)
    a.num_nodes, a.num_heads, a.head_dim, a.nnz = N, H, D, col_idx.numel()
    a.row_ptr, a.col_idx, a.x, a.out = row_ptr.data_ptr(), col_idx.data_ptr(), x.data_ptr(), None
    a.w = 256            # never dereferenced
    a.dtype = _DTYPES[x.dtype]
    nbytes = ctypes.c_size_t()
    _check(_lib.gattn_aggregate_workspace(ctypes.byref(a), ctypes.byref(nbytes)), "gattn_aggregate_workspace")
    return nbytes.value


def _check_node_tensor(t, name, like):
    if t.dtype != like.dtype or t.shape != like.shape or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"{name} must match q in dtype, shape and device and be contiguous")


def _row_stride(t):
    """Row stride of an [N, H, D] tensor for the C ABI: 0 when its rows are
    packed, else the stride of dim 0 in elements."""
    N, H, D = t.shape
    return 0 if t.stride(0) == H * D or N <= 1 else t.stride(0)


def _check_rows(t, name, like):
    """An [N, H, D] view whose rows may be strided (a fused projection's
    output): each row's H x D block packed, the row stride a multiple of 8
    elements, at least H x D."""
    if t.dim() != 3 or t.dtype != like.dtype or t.shape != like.shape or not t.is_cuda or t.device != like.device:
        raise ValueError(f"{name} must be an [N, H, D] GPU tensor matching q in dtype, shape and device")
    N, H, D = t.shape
    if t.stride(2) != 1 or (H > 1 and t.stride(1) != D) or (N > 1 and (t.stride(0) < H * D or t.stride(0) % 8)):
        raise ValueError(f"{name}: each row's [H, D] block must be packed and the row stride a multiple of 8 "
                         "elements, at least H * D")


def gattn_forward(row_ptr: torch.Tensor, col_idx: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  e: Optional[torch.Tensor] = None, mode: str = "standard", scale: Optional[float] = None,
                  clip=(-5.0, 5.0), eps: float = 1e-6, path: str = "auto", rw: Optional[RowWindows] = None,
                  out: Optional[torch.Tensor] = None, validate: bool = False,
                  edge_ids: Optional[torch.Tensor] = None, e_out=None, workspace=None,
                  hybrid: Optional[Hybrid] = None):
    """Fused SDDMM -> softmax -> SpMM over the CSR; q/k/v [N, H, D]; e
    [nnz, H, D] by CSR position (or row edge_ids[p] for position p) or None.
    Returns out [N, H, D]; with e_out (True, or an [nnz, H, D] tensor) the
    clipped mode also writes the per-edge update and returns (out, e_out).
    workspace: None (default) runs the node partition (equal destination
    counts per workgroup); True allocates the balanced-partition workspace
    and a uint8 tensor supplies it (equal edge shares, heavy rows cut across
    workgroups: for graphs whose hubs hold many times a workgroup's share).
    hybrid (with rw): a gattn_build_hybrid plan for path "hybrid" (or
    "auto"): dense row windows on the MFMA path, the other rows gathered."""
    if q.dim() != 3 or not q.is_cuda or q.dtype not in _DTYPES:
        raise ValueError("q must be an [N, H, D] GPU tensor")
    _check_rows(q, "q", q)
    _check_rows(k, "k", q)
    _check_rows(v, "v", q)
    if _row_stride(k) != _row_stride(v):
        raise ValueError("k and v must have the same row stride")
    N, H, D = q.shape
    row_ptr, col_idx = _csr(row_ptr, col_idx, N, q.device)
    if e is not None and (e.dtype != q.dtype or tuple(e.shape) != (col_idx.numel(), H, D) or not e.is_contiguous()
                          or e.device != q.device):
        raise ValueError("e must be a contiguous [nnz, H, D] tensor of q's dtype on q's device")
    if edge_ids is not None:
        edge_ids = _i32(edge_ids, "edge_ids", q.device, col_idx.numel())
    want_e_out = e_out is not None and e_out is not False
    if e_out is True:
        e_out = torch.empty((col_idx.numel(), H, D), dtype=q.dtype, device=q.device)
    elif want_e_out and (e_out.dtype != q.dtype or tuple(e_out.shape) != (col_idx.numel(), H, D)
                         or not e_out.is_contiguous() or e_out.device != q.device):
        raise ValueError("e_out must be a contiguous [nnz, H, D] tensor of q's dtype on q's device")
    for name, x in (("rw", rw), ("hybrid", hybrid)):
        t = None if x is None else (x.win_col_ptr if name == "rw" else x.dense_windows)
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if rw is not None and rw.num_nodes != N:
        raise ValueError(f"rw was built for {rw.num_nodes} nodes, q has {N}")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    else:
        _check_node_tensor(out, "out", q)
    a, keep = _forward_args(row_ptr, col_idx, q, k, v, e, out, mode, scale, clip, eps, path, rw, validate,
                            edge_ids, e_out if want_e_out else None, hybrid)
    ws = _attach_workspace(a, _lib.gattn_forward_workspace, workspace, q.device, "gattn_forward_workspace")
    _check(_lib.gattn_forward(ctypes.byref(a), _stream(q.device)), "gattn_forward")
    del keep, ws
    return (out, e_out) if want_e_out else out


def gattn_forward_noalloc(row_ptr: torch.Tensor, col_idx: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                          v: torch.Tensor, out: torch.Tensor, e: Optional[torch.Tensor] = None,
                          mode: str = "standard", scale: Optional[float] = None, clip=(-5.0, 5.0),
                          eps: float = 1e-6, path: str = "auto", rw: Optional[RowWindows] = None,
                          edge_ids: Optional[torch.Tensor] = None, e_out: Optional[torch.Tensor] = None,
                          hybrid: Optional[Hybrid] = None) -> torch.Tensor:
    """gattn_forward for callers that cannot allocate: the gather path runs
    the balanced partition with its workspace in the library's fixed scratch
    array (GATTN_NOALLOC_SCRATCH_BYTES per GPU).  `out` (and `e_out`, when
    wanted) must be given; nothing is allocated here or in the library.
    Calls whose executions overlap on one GPU race on the scratch array."""
    if out is None:
        raise ValueError("gattn_forward_noalloc writes into a given `out`")
    if q.dim() != 3 or not q.is_cuda or q.dtype not in _DTYPES:
        raise ValueError("q must be an [N, H, D] GPU tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_rows(t, name, q)
    if _row_stride(k) != _row_stride(v):
        raise ValueError("k and v must have the same row stride")
    _check_node_tensor(out, "out", q)
    N, H, D = q.shape
    row_ptr, col_idx = _csr(row_ptr, col_idx, N, q.device)
    nnz = col_idx.numel()
    if e is not None and (e.dtype != q.dtype or tuple(e.shape) != (nnz, H, D) or not e.is_contiguous()
                          or e.device != q.device):
        raise ValueError("e must be a contiguous [nnz, H, D] tensor of q's dtype on q's device")
    if e_out is not None and (e_out.dtype != q.dtype or tuple(e_out.shape) != (nnz, H, D)
                              or not e_out.is_contiguous() or e_out.device != q.device):
        raise ValueError("e_out must be a contiguous [nnz, H, D] tensor of q's dtype on q's device")
    if edge_ids is not None:
        edge_ids = _i32(edge_ids, "edge_ids", q.device, nnz)
    a, keep = _forward_args(row_ptr, col_idx, q, k, v, e, out, mode, scale, clip, eps, path, rw, False,
                            edge_ids, e_out, hybrid)
    _check(_lib.gattn_forward_noalloc(ctypes.byref(a), _stream(q.device)), "gattn_forward_noalloc")
    del keep
    return out


def gattn_forward_path(row_ptr, col_idx, q, k, v, e=None, mode="standard", path="auto",
                       rw: Optional[RowWindows] = None, hybrid: Optional[Hybrid] = None) -> str:
    a, keep = _forward_args(row_ptr, col_idx, q, k, v, e, None, mode, None, (-5.0, 5.0), 1e-6, path, rw, False,
                            hybrid=hybrid)
    res = ctypes.c_int(0)
    _check(_lib.gattn_forward_path(ctypes.byref(a), ctypes.byref(res)), "gattn_forward_path")
    del keep
    return _PATH_NAMES[res.value]


def gattn_aggregate(row_ptr: torch.Tensor, col_idx: torch.Tensor, x: torch.Tensor, w: torch.Tensor,
                    normalize: bool = False, eps: float = 1e-6, edge_ids: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, validate: bool = False, workspace=None) -> torch.Tensor:
    """Weighted aggregation over the CSR: x [N, H, D], w [nnz, H] fp32 (row
    edge_ids[p] for position p when given); out[i] = sum_p w x[src], divided
    by (sum_p w + eps) when normalize.  workspace as in gattn_forward."""
    if x.dim() != 3 or not x.is_contiguous() or not x.is_cuda or x.dtype not in _DTYPES:
        raise ValueError("x must be a contiguous [N, H, D] GPU tensor")
    N, H, D = x.shape
    row_ptr, col_idx = _csr(row_ptr, col_idx, N, x.device)
    nnz = col_idx.numel()
    if w.dtype != torch.float32 or tuple(w.shape) != (nnz, H) or not w.is_contiguous() or w.device != x.device:
        raise ValueError("w must be a contiguous fp32 [nnz, H] tensor on x's device")
    if edge_ids is not None:
        edge_ids = _i32(edge_ids, "edge_ids", x.device, nnz)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_node_tensor(out, "out", x)
    a = _AggregateArgs()
    a.struct_size = ctypes.sizeof(_AggregateArgs)
    a.num_nodes, a.num_heads, a.head_dim, a.nnz = N, H, D, nnz
    a.row_ptr, a.col_idx = row_ptr.data_ptr(), col_idx.data_ptr()
    a.x, a.w, a.out = x.data_ptr(), w.data_ptr(), out.data_ptr()
    a.edge_ids = None if edge_ids is None else edge_ids.data_ptr()
    a.dtype = _DTYPES[x.dtype]
    a.normalize = 1 if normalize else 0
    a.eps = eps
    a.flags = GATTN_FLAG_VALIDATE if validate else 0
    ws = _attach_workspace(a, _lib.gattn_aggregate_workspace, workspace, x.device, "gattn_aggregate_workspace")
    _check(_lib.gattn_aggregate(ctypes.byref(a), _stream(x.device)), "gattn_aggregate")
    del ws
    return out


@dataclasses.dataclass
class Graph:
    """A graph as the kernels read it: CSR by destination in canonical order
    (destination, source, edge id), plus edge_perm[p] = the original COO id
    of the edge at CSR position p.  Built on the device by from_coo; the row
    windows of the MFMA path are built on the first rowwindows() call and
    kept (that build synchronizes once, for its size query)."""
    num_nodes: int
    row_ptr: torch.Tensor      # int32 [N + 1]
    col_idx: torch.Tensor      # int32 [nnz]
    edge_perm: torch.Tensor    # int32 [nnz]
    _rw: Optional[RowWindows] = dataclasses.field(default=None, repr=False)
    _max_degree: Optional[int] = dataclasses.field(default=None, repr=False)

    @classmethod
    def from_coo(cls, src: torch.Tensor, dst: torch.Tensor, num_nodes: int, validate: bool = True) -> "Graph":
        """Edges src[i] -> dst[i] (int32 GPU tensors); validate=True rejects
        indices outside [0, num_nodes) (and synchronizes)."""
        row_ptr, col_idx, edge_perm = gattn_build_csr(src, dst, num_nodes, validate)
        return cls(num_nodes, row_ptr, col_idx, edge_perm)

    @property
    def nnz(self) -> int:
        return self.col_idx.numel()

    def rowwindows(self) -> RowWindows:
        if self._rw is None:
            self._rw = gattn_build_rowwindows(self.row_ptr, self.col_idx, self.num_nodes)
        return self._rw

    @property
    def max_degree(self) -> int:
        """Largest in-degree (read back once)."""
        if self._max_degree is None:
            self._max_degree = int((self.row_ptr[1:] - self.row_ptr[:-1]).max().item()) if self.num_nodes else 0
        return self._max_degree

    def skewed(self) -> bool:
        """Whether hubs would set the gather kernel's end under equal
        destination counts per workgroup (Graph.skewed_degrees on this
        graph's sizes and largest in-degree, which is read back only when
        the sizes leave the rule open)."""
        if Graph.skewed_degrees(self.num_nodes, self.nnz, 1 << 31) is False:
            return False
        return Graph.skewed_degrees(self.num_nodes, self.nnz, self.max_degree)

    @staticmethod
    def skewed_degrees(num_nodes: int, nnz: int, max_degree: int) -> bool:
        """The rule behind Graph.skewed: the largest in-degree is above 32x
        the mean, and the graph is small enough (below 2^24 edges) that its
        workgroups run in few rounds (in many rounds the other workgroups
        absorb a hub's)."""
        if num_nodes == 0 or nnz == 0 or nnz >= (1 << 24):
            return False
        return max_degree > 32.0 * nnz / num_nodes


def forward(graph: Graph, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, e: Optional[torch.Tensor] = None,
            mode: str = "standard", scale: Optional[float] = None, clip=(-5.0, 5.0), eps: float = 1e-6,
            path: str = "auto", out: Optional[torch.Tensor] = None, e_out=None, workspace="auto"):
    """gattn_forward on a Graph.  e (and e_out, when asked for) are indexed
    by the caller's original edge ids -- the COO order from_coo was given --
    and reached through graph.edge_perm, as the gattn-triton article reaches
    its edge tensor through the CSC edge ids.  With fp16 / bf16 inputs, the
    standard mode and no e, paths "auto" and "mfma" use the graph's row
    windows (built on first use); "auto" then takes the MFMA path for dense
    windows, else the gather path.  workspace "auto" runs the gather path's
    balanced partition (heavy rows cut across workgroups) on skewed graphs
    (Graph.skewed) and the node partition otherwise; None, True or a tensor
    are passed on to gattn_forward."""
    rw = None
    if path in ("auto", "mfma") and q.dtype != torch.float32 and mode == "standard" and e is None:
        rw = graph.rowwindows()
    ids = graph.edge_perm if (e is not None or (e_out is not None and e_out is not False)) else None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None, True or a uint8 tensor')
        workspace = True if graph.skewed() else None
    return gattn_forward(graph.row_ptr, graph.col_idx, q, k, v, e, mode=mode, scale=scale, clip=clip, eps=eps,
                         path=path, rw=rw, out=out, edge_ids=ids, e_out=e_out, workspace=workspace)


__all__ = ["Graph", "forward", "gattn_build_csr", "gattn_build_rowwindows", "gattn_build_hybrid", "gattn_forward", "gattn_forward_path",
           "gattn_forward_noalloc", "gattn_aggregate",
           "gattn_forward_workspace", "gattn_aggregate_workspace",
           "gattn_status_string", "gattn_abi_version", "CsrBuilder", "RowWindows", "Hybrid", "GattnError", "LIB_PATH"]
