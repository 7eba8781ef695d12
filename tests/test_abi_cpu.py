"""The C ABI without a GPU: every symbol of include/gattn.h is exported, and
argument errors come back before anything touches the HIP runtime.  No
compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gattn.h")


@pytest.fixture(scope="module")
def gsa():
    from graph_sparse_attention_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    import graph_sparse_attention_amd as g
    return g


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"GATTN_API\s+[\w\s\*]+?\b(gattn_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported(gsa):
    names = declared_functions()
    assert len(names) == 13, names
    lib = ctypes.CDLL(gsa.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gattn.h but not exported"


def test_only_the_c_abi_is_exported(gsa):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gsa.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert sorted(text_syms) == sorted(declared_functions())


def test_enums_and_strings(gsa):
    text = open(HEADER).read()
    for name in ["GATTN_OK", "GATTN_ERR_INVALID_VALUE", "GATTN_ERR_UNSUPPORTED", "GATTN_ERR_BAD_GRAPH",
                 "GATTN_ERR_DUPLICATE_EDGE", "GATTN_ERR_BUFFER_TOO_SMALL", "GATTN_ERR_HIP"]:
        m = re.search(name + r"\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(gsa, name)
    assert gsa.gattn_abi_version() == 5
    assert gsa.gattn_status_string(gsa.GATTN_ERR_DUPLICATE_EDGE).startswith("repeated")
    assert gsa.gattn_status_string(99) == "unknown status"
    assert ctypes.sizeof(gsa._ForwardArgs) == 184
    assert ctypes.sizeof(gsa._Hybrid) == 32
    assert ctypes.sizeof(gsa._AggregateArgs) == 104


def fake_args(gsa, **kw):
    a = gsa._ForwardArgs()
    a.struct_size = ctypes.sizeof(gsa._ForwardArgs)
    a.num_nodes, a.num_heads, a.head_dim, a.nnz = 100, 8, 64, 1000
    base = 1 << 32   # aligned, never dereferenced: only host checks run
    a.row_ptr, a.col_idx = base, base + (1 << 20)
    a.q, a.k, a.v, a.out = base + (2 << 20), base + (4 << 20), base + (6 << 20), base + (8 << 20)
    a.e = None
    a.dtype, a.mode, a.path = gsa.GATTN_F16, gsa.GATTN_SOFTMAX_STANDARD, gsa.GATTN_PATH_AUTO
    a.scale, a.clip_lo, a.clip_hi, a.eps = 0.125, -5.0, 5.0, 1e-6
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def path_of(gsa, a):
    r = ctypes.c_int(-1)
    st = gsa._lib.gattn_forward_path(ctypes.byref(a), ctypes.byref(r))
    return st, r.value


def test_forward_argument_errors(gsa):
    L = gsa._lib
    cases = [
        (dict(struct_size=12), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(num_nodes=-1), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(num_heads=0), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(head_dim=48), gsa.GATTN_ERR_UNSUPPORTED),
        (dict(dtype=7), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(mode=5), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(path=9), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(scale=0.0), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(scale=float("nan")), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(mode=gsa.GATTN_SOFTMAX_CLIPPED, clip_lo=1.0, clip_hi=-1.0), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(mode=gsa.GATTN_SOFTMAX_CLIPPED, eps=-1.0), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(q=(1 << 32) + 8), gsa.GATTN_ERR_INVALID_VALUE),          # misaligned
        (dict(row_ptr=None), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(out=None), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(out=(1 << 32) + (2 << 20)), gsa.GATTN_ERR_INVALID_VALUE),  # aliases q
        (dict(flags=8), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(path=gsa.GATTN_PATH_MFMA), gsa.GATTN_ERR_INVALID_VALUE),  # no row windows
        (dict(path=gsa.GATTN_PATH_MFMA, dtype=gsa.GATTN_F32), gsa.GATTN_ERR_UNSUPPORTED),
        (dict(path=gsa.GATTN_PATH_MFMA, mode=gsa.GATTN_SOFTMAX_CLIPPED), gsa.GATTN_ERR_UNSUPPORTED),
        (dict(path=gsa.GATTN_PATH_MFMA, head_dim=16), gsa.GATTN_ERR_UNSUPPORTED),
        # the edge update needs the clipped mode and an edge tensor, no aliasing
        (dict(e_out=(1 << 32) + (16 << 20)), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(e_out=(1 << 32) + (16 << 20), mode=gsa.GATTN_SOFTMAX_CLIPPED), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(e_out=(1 << 32) + (16 << 20), e=(1 << 32) + (14 << 20)), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(e_out=(1 << 32) + (14 << 20) + 64, e=(1 << 32) + (14 << 20), mode=gsa.GATTN_SOFTMAX_CLIPPED),
         gsa.GATTN_ERR_INVALID_VALUE),                                 # aliases e
        (dict(e_out=(1 << 32) + (16 << 20) + 8, e=(1 << 32) + (14 << 20), mode=gsa.GATTN_SOFTMAX_CLIPPED),
         gsa.GATTN_ERR_INVALID_VALUE),                                 # misaligned
        (dict(edge_ids=(1 << 32) + 2), gsa.GATTN_ERR_INVALID_VALUE),   # misaligned
        # row strides of q and of k / v: at least H * D, multiples of 8, at most 2^24
        (dict(q_stride=256), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(kv_stride=516), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(kv_stride=(1 << 24) + 8), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(q_stride=1024, out=(1 << 32) + (2 << 20) + 102400), gsa.GATTN_ERR_INVALID_VALUE),  # in q's span
        (dict(kv_stride=2048, out=(1 << 32) + (6 << 20) + 102400), gsa.GATTN_ERR_INVALID_VALUE),  # in v's span
        (dict(workspace=(1 << 32) + (20 << 20) + 64, workspace_bytes=4096), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(workspace=(1 << 32) + (8 << 20), workspace_bytes=4096), gsa.GATTN_ERR_INVALID_VALUE),  # aliases out
    ]
    for kw, want in cases:
        a = fake_args(gsa, **kw)
        assert L.gattn_forward(ctypes.byref(a), None) == want, kw
    assert L.gattn_forward(None, None) == gsa.GATTN_ERR_INVALID_VALUE


def test_strided_rows_accepted(gsa):
    # strided q / k / v pass the host checks (out just past q's packed rows is
    # fine while q is packed); the MFMA path needs the strided spans under 2^31
    a = fake_args(gsa, out=(1 << 32) + (2 << 20) + 102400, q_stride=0, kv_stride=1024)
    assert path_of(gsa, a)[0] == gsa.GATTN_OK
    rw = gsa._RowWindows(7, 16 * 10, (1 << 32) + (10 << 20), (1 << 32) + (11 << 20), (1 << 32) + (12 << 20))
    a = fake_args(gsa, kv_stride=1024, path=gsa.GATTN_PATH_MFMA)
    a.rw = ctypes.pointer(rw)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_MFMA)
    # 2^17 rows 2^15 bytes apart: K and V each span (2^17 - 1) * 2^15 + 1024 bytes > 2^31
    a.num_nodes, a.kv_stride = 1 << 17, 1 << 14
    a.k, a.v, a.out = (1 << 40), (1 << 41), (1 << 39)
    a.rw.contents.num_windows = (1 << 17) // 16
    assert path_of(gsa, a)[0] == gsa.GATTN_ERR_UNSUPPORTED
    a.path = gsa.GATTN_PATH_AUTO
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)


def test_path_resolution(gsa):
    base = 1 << 32
    rw = gsa._RowWindows(7, 16 * 80, base + (10 << 20), base + (11 << 20), base + (12 << 20))  # density 1000/(16*1280)
    a = fake_args(gsa)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)           # no row windows
    a.rw = ctypes.pointer(rw)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)           # density 0.049 < 0.09
    rw.num_cols = 16 * 60                                                     # density 0.065 < 0.09
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)
    rw.num_cols = 16 * 40                                                     # density 0.098
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_MFMA)
    rw.num_cols = 16 * 10                                                     # density 0.39
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_MFMA)
    a.e = base + (14 << 20)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)           # edge tensor: gather only
    a.e = None
    a.out = None                                                              # the query needs no output
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_MFMA)
    rw.num_windows = 3
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)           # inconsistent windows ignored
    a.path = gsa.GATTN_PATH_MFMA
    assert path_of(gsa, a)[0] == gsa.GATTN_ERR_INVALID_VALUE


def fake_hybrid(gsa, **kw):
    base = 1 << 32
    h = gsa._Hybrid(3, 4, 8, base + (30 << 20), base + (31 << 20))   # this geometry stages 12 Q rows
    for k, v in kw.items():
        setattr(h, k, v)
    return h


def test_hybrid_path_checks(gsa):
    L = gsa._lib
    base = 1 << 32
    rw = gsa._RowWindows(7, 16 * 10, base + (10 << 20), base + (11 << 20), base + (12 << 20))
    hy = fake_hybrid(gsa)
    # the hybrid path needs the MFMA path's conditions, row windows and a plan
    a = fake_args(gsa, path=gsa.GATTN_PATH_HYBRID)
    assert path_of(gsa, a)[0] == gsa.GATTN_ERR_INVALID_VALUE                  # no row windows
    a.rw = ctypes.pointer(rw)
    assert path_of(gsa, a)[0] == gsa.GATTN_ERR_INVALID_VALUE                  # no plan
    a.hybrid = ctypes.pointer(hy)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_HYBRID)
    for kw in (dict(num_dense=8), dict(num_dense=-1), dict(num_ranges=101), dict(range_rows=0),
               dict(range_rows=100000), dict(dense_windows=None), dict(ranges=None), dict(ranges=base + 2)):
        bad = fake_hybrid(gsa, **kw)
        a.hybrid = ctypes.pointer(bad)
        assert path_of(gsa, a)[0] == gsa.GATTN_ERR_INVALID_VALUE, kw
        assert L.gattn_forward(ctypes.byref(a), None) == gsa.GATTN_ERR_INVALID_VALUE, kw
    a.hybrid = ctypes.pointer(hy)
    a.dtype = gsa.GATTN_F32
    assert path_of(gsa, a)[0] == gsa.GATTN_ERR_UNSUPPORTED
    # AUTO takes a plan when the MFMA path applies, and ignores it otherwise
    a = fake_args(gsa, rw=ctypes.pointer(rw), hybrid=ctypes.pointer(hy))
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_HYBRID)
    a.e = base + (14 << 20)
    assert path_of(gsa, a) == (gsa.GATTN_OK, gsa.GATTN_PATH_GATHER)


def test_build_hybrid_argument_errors(gsa):
    L = gsa._lib
    base = 1 << 32
    rw = gsa._RowWindows(7, 16 * 10, base + (10 << 20), base + (11 << 20), base + (12 << 20))
    plan = gsa._Hybrid()
    dw, rg = ctypes.c_void_p(base + (30 << 20)), ctypes.c_void_p(base + (31 << 20))
    a = fake_args(gsa, rw=ctypes.pointer(rw))
    assert L.gattn_build_hybrid(ctypes.byref(a), 0.25, dw, rg, None, None) == gsa.GATTN_ERR_INVALID_VALUE
    for d in (-0.5, float("nan"), float("inf")):
        assert L.gattn_build_hybrid(ctypes.byref(a), d, dw, rg, ctypes.byref(plan), None) == gsa.GATTN_ERR_INVALID_VALUE
    assert L.gattn_build_hybrid(ctypes.byref(a), 0.25, None, rg, ctypes.byref(plan), None) == gsa.GATTN_ERR_INVALID_VALUE
    assert L.gattn_build_hybrid(ctypes.byref(a), 0.25, dw, ctypes.c_void_p(base + 2), ctypes.byref(plan),
                                None) == gsa.GATTN_ERR_INVALID_VALUE
    b = fake_args(gsa)                                                        # no row windows
    assert L.gattn_build_hybrid(ctypes.byref(b), 0.25, dw, rg, ctypes.byref(plan), None) == gsa.GATTN_ERR_INVALID_VALUE
    b = fake_args(gsa, rw=ctypes.pointer(rw), dtype=gsa.GATTN_F32)            # no MFMA path for fp32
    assert L.gattn_build_hybrid(ctypes.byref(b), 0.25, dw, rg, ctypes.byref(plan), None) == gsa.GATTN_ERR_UNSUPPORTED
    b = fake_args(gsa, rw=ctypes.pointer(rw), mode=gsa.GATTN_SOFTMAX_CLIPPED)
    assert L.gattn_build_hybrid(ctypes.byref(b), 0.25, dw, rg, ctypes.byref(plan), None) == gsa.GATTN_ERR_UNSUPPORTED
    # an empty graph: an empty plan, no HIP call
    rw0 = gsa._RowWindows(0, 0, base + (10 << 20), None, None)
    z = fake_args(gsa, num_nodes=0, nnz=0, rw=ctypes.pointer(rw0))
    assert L.gattn_build_hybrid(ctypes.byref(z), 0.25, None, None, ctypes.byref(plan), None) == gsa.GATTN_OK
    assert (plan.num_dense, plan.num_ranges) == (0, 0)


def test_build_argument_errors(gsa):
    L = gsa._lib
    sz = ctypes.c_size_t()
    assert L.gattn_build_csr_workspace(10, 20, ctypes.byref(sz)) == 0 and sz.value > 0
    assert L.gattn_build_csr_workspace(-1, 20, ctypes.byref(sz)) == gsa.GATTN_ERR_INVALID_VALUE
    assert L.gattn_build_csr_workspace(10, 1 << 31, ctypes.byref(sz)) == gsa.GATTN_ERR_INVALID_VALUE
    need = sz.value if L.gattn_build_csr_workspace(10, 20, ctypes.byref(sz)) == 0 else 0
    base = 1 << 32
    p = lambda i: ctypes.c_void_p(base + (i << 20))
    # null row_ptr, null COO with edges, misaligned workspace, workspace too small
    assert L.gattn_build_csr(10, 20, p(1), p(2), None, p(4), p(5), p(6), need, None, None) == 1
    assert L.gattn_build_csr(10, 20, None, p(2), p(3), p(4), p(5), p(6), need, None, None) == 1
    assert L.gattn_build_csr(10, 20, p(1), p(2), p(3), p(4), p(5), ctypes.c_void_p(base + 64), need, None, None) == 1
    assert L.gattn_build_csr(10, 20, p(1), p(2), p(3), p(4), p(5), p(6), need - 1, None, None) == 5
    assert L.gattn_build_rowwindows_workspace(10, 20, ctypes.byref(sz)) == 0
    need = sz.value
    nc = ctypes.c_int64(0)
    assert L.gattn_build_rowwindows(10, 20, p(1), p(2), p(3), None, None, None, p(6), need, None) == 1
    assert L.gattn_build_rowwindows(10, 20, None, p(2), p(3), None, None, ctypes.byref(nc), p(6), need, None) == 1
    assert L.gattn_build_rowwindows(10, 20, p(1), p(2), p(3), None, None, ctypes.byref(nc), p(6), need - 8, None) == 5
    # padded column counts that an int32 win_col_ptr could not hold
    n_big, m_big = 1 << 27, (1 << 31) - (1 << 20)
    assert L.gattn_build_rowwindows_workspace(n_big, m_big, ctypes.byref(sz)) == 0
    assert L.gattn_build_rowwindows(n_big, m_big, p(1), p(2), p(3), None, None, ctypes.byref(nc), p(6), sz.value,
                                    None) == gsa.GATTN_ERR_UNSUPPORTED


def test_csr_workspace_per_build(gsa, monkeypatch):
    # the counting build needs about 16 bytes per edge (sort keys and the merge
    # buffer of long rows), the radix build (chosen from 2^18 edges, or forced)
    # about 25: keys and values twice, plus 8-byte look-back words per tile
    # (and group of tiles), digit and pass
    L = gsa._lib
    sz = ctypes.c_size_t()

    def need(n, m):
        assert L.gattn_build_csr_workspace(n, m, ctypes.byref(sz)) == 0
        return sz.value

    small, large = (1 << 18) - 1, 1 << 18
    assert 16 * small <= need(100000, small) < 18 * small
    assert 24 * large <= need(100000, large) < 28 * large
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    assert 24 * small <= need(100000, small) < 28 * small
    assert need(100000, 0) < 4096 + 4 * 100000 + 8192   # no edges: the counting build
    monkeypatch.setenv("GATTN_CSR_PATH", "atomic")
    assert 16 * large <= need(100000, large) < 18 * large
    monkeypatch.delenv("GATTN_CSR_PATH")
    # 4 radix passes (31-bit keys) take more look-back words than 3
    assert need((1 << 31) - 1, large) > need(1 << 20, large)


def fake_aggregate(gsa, **kw):
    a = gsa._AggregateArgs()
    a.struct_size = ctypes.sizeof(gsa._AggregateArgs)
    a.num_nodes, a.num_heads, a.head_dim, a.nnz = 100, 8, 64, 1000
    base = 1 << 32
    a.row_ptr, a.col_idx, a.x, a.w = base, base + (1 << 20), base + (2 << 20), base + (4 << 20)
    a.edge_ids, a.out = None, base + (6 << 20)
    a.dtype, a.normalize, a.eps, a.flags = gsa.GATTN_F32, 0, 1e-6, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_aggregate_argument_errors(gsa):
    L = gsa._lib
    base = 1 << 32
    cases = [
        (dict(struct_size=8), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(num_nodes=-2), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(num_heads=0), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(nnz=1 << 31), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(dtype=3), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(normalize=2), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(eps=-1e-3), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(eps=float("inf")), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(flags=4), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(head_dim=8), gsa.GATTN_ERR_UNSUPPORTED),
        (dict(w=None), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(x=None), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(out=None), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(x=base + (2 << 20) + 4), gsa.GATTN_ERR_INVALID_VALUE),     # misaligned
        (dict(w=base + (4 << 20) + 2), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(out=base + (2 << 20) + 4096), gsa.GATTN_ERR_INVALID_VALUE),  # aliases x
        (dict(out=base + (4 << 20)), gsa.GATTN_ERR_INVALID_VALUE),         # aliases w
        (dict(workspace=base + (8 << 20) + 128, workspace_bytes=4096), gsa.GATTN_ERR_INVALID_VALUE),
        (dict(workspace=base + (2 << 20), workspace_bytes=4096), gsa.GATTN_ERR_INVALID_VALUE),  # aliases x
    ]
    for kw, want in cases:
        a = fake_aggregate(gsa, **kw)
        assert L.gattn_aggregate(ctypes.byref(a), None) == want, kw
    assert L.gattn_aggregate(None, None) == gsa.GATTN_ERR_INVALID_VALUE
    # nothing to do: no launch, no HIP call
    a = fake_aggregate(gsa, num_nodes=0, nnz=0, row_ptr=None, x=None, w=None, out=None)
    assert L.gattn_aggregate(ctypes.byref(a), None) == gsa.GATTN_OK


def test_workspace_query_errors(gsa):
    L = gsa._lib
    nb = ctypes.c_size_t(7)
    a = fake_args(gsa)
    assert L.gattn_forward_workspace(ctypes.byref(a), None) == gsa.GATTN_ERR_INVALID_VALUE
    assert L.gattn_forward_workspace(None, ctypes.byref(nb)) == gsa.GATTN_ERR_INVALID_VALUE
    a = fake_args(gsa, head_dim=24)
    assert L.gattn_forward_workspace(ctypes.byref(a), ctypes.byref(nb)) == gsa.GATTN_ERR_UNSUPPORTED
    g = fake_aggregate(gsa, normalize=3)
    assert L.gattn_aggregate_workspace(ctypes.byref(g), ctypes.byref(nb)) == gsa.GATTN_ERR_INVALID_VALUE
    assert nb.value == 7   # untouched on error
    # nothing to compute: no workspace, no HIP call
    a = fake_args(gsa, num_nodes=0, nnz=0)
    assert L.gattn_forward_workspace(ctypes.byref(a), ctypes.byref(nb)) == gsa.GATTN_OK and nb.value == 0


def test_noalloc_host_checks(gsa):
    # gattn_forward_noalloc refuses, before touching a device: a caller
    # workspace, the validating flag (a host copy), and a problem whose
    # balanced-partition workspace exceeds the library's scratch array
    L = gsa._lib
    text = open(HEADER).read()
    m = re.search(r"#define GATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gsa.GATTN_NOALLOC_SCRATCH_BYTES
    base = 1 << 32
    a = fake_args(gsa, workspace=base + (20 << 20), workspace_bytes=4096)
    assert L.gattn_forward_noalloc(ctypes.byref(a), None) == gsa.GATTN_ERR_INVALID_VALUE
    a = fake_args(gsa, flags=gsa.GATTN_FLAG_VALIDATE)
    assert L.gattn_forward_noalloc(ctypes.byref(a), None) == gsa.GATTN_ERR_INVALID_VALUE
    a = fake_args(gsa, head_dim=40)
    assert L.gattn_forward_noalloc(ctypes.byref(a), None) == gsa.GATTN_ERR_UNSUPPORTED
    assert L.gattn_forward_noalloc(None, None) == gsa.GATTN_ERR_INVALID_VALUE
    # a huge graph (tensors far apart so that none overlaps): its workspace
    # exceeds the scratch array
    big = fake_args(gsa, num_nodes=400_000_000, nnz=2_000_000_000, num_heads=1, head_dim=64,
                    row_ptr=1 << 40, col_idx=2 << 40, q=3 << 40, k=4 << 40, v=5 << 40, out=6 << 40)
    nb = ctypes.c_size_t(0)
    assert L.gattn_forward_workspace(ctypes.byref(big), ctypes.byref(nb)) == gsa.GATTN_OK
    assert nb.value > gsa.GATTN_NOALLOC_SCRATCH_BYTES
    assert L.gattn_forward_noalloc(ctypes.byref(big), None) == gsa.GATTN_ERR_BUFFER_TOO_SMALL
    # nothing to compute
    a = fake_args(gsa, num_nodes=0, nnz=0)
    assert L.gattn_forward_noalloc(ctypes.byref(a), None) == gsa.GATTN_OK


def test_skewed_degree_rule(gsa):
    # the graph layer's choice of the balanced gather partition (and bench.py's)
    rule = gsa.Graph.skewed_degrees
    assert rule(100, 1000, 321) and not rule(100, 1000, 320)      # above 32x the mean in-degree
    assert not rule(1 << 20, 1 << 24, 1 << 20)                     # 2^24 edges or more: many rounds
    assert rule(1 << 20, (1 << 24) - 1, 1 << 20)
    assert not rule(0, 0, 0) and not rule(10, 0, 0)
