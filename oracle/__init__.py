"""CPU oracle for fused graph sparse attention (fp64, plain C via ctypes).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library and
its Python binding never do.  ``build()`` compiles ``oracle.c`` with gcc
(``-O2 -fopenmp``, no fast-math, no FP contraction).

All float inputs are float64 numpy arrays: callers widen the stored fp32 /
fp16 / bf16 values exactly (``widen``).  See ``oracle.c`` for the passages
of the pages each function restates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ORC_OK, ORC_INVALID, ORC_BAD_GRAPH, ORC_DUPLICATE, ORC_NOMEM = range(5)
_NAMES = {1: "INVALID", 2: "BAD_GRAPH", 3: "DUPLICATE", 4: "NOMEM"}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code} ({_NAMES.get(code, '?')})")
        self.code = code


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def load(path: str):
    """ctypes handle with argument types declared (any build of oracle.c)."""
    L = ctypes.CDLL(path)
    i32p = ctypes.c_void_p
    L.orc_build_csr.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p, i32p, i32p, i32p]
    L.orc_rowwindow_sizes.argtypes = [ctypes.c_int32, i32p, i32p, i32p]
    L.orc_build_rowwindows.argtypes = [ctypes.c_int32, i32p, i32p, i32p, i32p, i32p]
    L.orc_forward.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                              i32p, i32p, i32p, i32p, i32p, i32p, i32p,
                              ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                              ctypes.c_double, i32p, ctypes.c_int64, i32p, i32p, i32p, i32p, ctypes.c_int]
    L.orc_aggregate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                i32p, i32p, i32p, i32p, i32p, ctypes.c_int, ctypes.c_double, i32p, ctypes.c_int]
    for f in (L.orc_build_csr, L.orc_rowwindow_sizes, L.orc_build_rowwindows, L.orc_forward, L.orc_aggregate):
        f.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = load(_LIB_PATH)
    return _lib


class use_library:
    """Context manager: route this module's calls to another build of
    oracle.c (the mutation tests compile deliberately broken copies)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _check(rc):
    if rc != ORC_OK:
        raise OracleError(rc)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def widen(x) -> np.ndarray:
    """Exact widening of a torch tensor or numpy array to float64 numpy."""
    if hasattr(x, "detach"):
        return np.ascontiguousarray(x.detach().cpu().double().numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def build_csr(n: int, src, dst):
    """Canonical destination-grouped CSR: (row_ptr, col_idx, edge_perm)."""
    src, dst = _i32(src), _i32(dst)
    nnz = src.shape[0]
    row_ptr = np.empty(n + 1, np.int32)
    col_idx = np.empty(max(nnz, 0), np.int32)
    perm = np.empty(max(nnz, 0), np.int32)
    _check(lib().orc_build_csr(n, nnz, _p(src), _p(dst), _p(row_ptr), _p(col_idx), _p(perm)))
    return row_ptr, col_idx, perm


def rowwindows(n: int, row_ptr, col_idx):
    """(win_col_ptr [W+1], win_cols [C], tile_mask [C/16, 16] uint16)."""
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    W = (n + 15) // 16
    wcp = np.empty(W + 1, np.int32)
    _check(lib().orc_rowwindow_sizes(n, _p(row_ptr), _p(col_idx), _p(wcp)))
    C = int(wcp[-1])
    cols = np.empty(C, np.int32)
    mask = np.empty((C // 16, 16), np.uint16)
    _check(lib().orc_build_rowwindows(n, _p(row_ptr), _p(col_idx), _p(wcp), _p(cols), _p(mask)))
    return wcp, cols, mask


def forward(row_ptr, col_idx, q, k, v, e=None, mode="standard", scale=None, clip=(-5.0, 5.0),
            eps=1e-6, rows=None, want_mag=False, want_alpha=False, threads=1, edge_ids=None,
            want_e_out=False):
    """fp64 fused 3S forward.  q/k/v: float64 [N,H,D]; e: float64 [nnz,H,D]
    or None, row edge_ids[p] for CSR position p (row p without edge_ids).
    Returns out [nrows,H,D] (and mag, alpha, e_out when asked)."""
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    n, h, d = q.shape
    nnz = int(col_idx.shape[0])
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(d)))
    if e is not None:
        e = np.ascontiguousarray(e, dtype=np.float64)
        assert e.shape == (nnz, h, d)
    if rows is not None:
        rows = _i32(rows)
        nrows = rows.shape[0]
    else:
        nrows = n
    out = np.empty((nrows, h, d), np.float64)
    mag = np.empty((nrows, h, d), np.float64) if want_mag else None
    alpha = np.full((nnz, h), np.nan, np.float64) if want_alpha else None
    e_out = np.full((nnz, h, d), np.nan, np.float64) if want_e_out else None
    if edge_ids is not None:
        edge_ids = _i32(edge_ids)
    clipped = {"standard": 0, "clipped": 1}[mode]
    _check(lib().orc_forward(n, h, d, nnz, _p(row_ptr), _p(col_idx), _p(q), _p(k), _p(v), _p(e),
                             _p(edge_ids), clipped, float(scale), float(clip[0]), float(clip[1]), float(eps),
                             _p(rows), nrows, _p(out), _p(mag), _p(alpha), _p(e_out), int(threads)))
    res = [out]
    if want_mag:
        res.append(mag)
    if want_alpha:
        res.append(alpha)
    if want_e_out:
        res.append(e_out)
    return res[0] if len(res) == 1 else tuple(res)


def aggregate(row_ptr, col_idx, x, w, normalize=False, eps=1e-6, edge_ids=None, threads=1):
    """fp64 weighted aggregation: x float64 [N,H,D], w float64 [nnz,H]
    (row edge_ids[p] for CSR position p).  Returns out [N,H,D]."""
    row_ptr, col_idx = _i32(row_ptr), _i32(col_idx)
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n, h, d = x.shape
    nnz = int(col_idx.shape[0])
    assert w.shape == (nnz, h)
    if edge_ids is not None:
        edge_ids = _i32(edge_ids)
    out = np.empty((n, h, d), np.float64)
    _check(lib().orc_aggregate(n, h, d, nnz, _p(row_ptr), _p(col_idx), _p(x), _p(w), _p(edge_ids),
                               int(bool(normalize)), float(eps), _p(out), int(threads)))
    return out
