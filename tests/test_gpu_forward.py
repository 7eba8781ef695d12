"""GPU: fused forward (gather and MFMA row-window paths) against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import FP32_TOL, REL_L2_TOL, TORCH_DTYPE, ForwardCheck, case, check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


def gpu_forward(gsa, c, path="gather", rw=None, rp=None, ci=None, workspace=True):
    wl = c.wl
    rp_t = torch.from_numpy(c.rp if rp is None else rp).cuda()
    ci_t = torch.from_numpy(c.ci if ci is None else ci).cuda()
    return gsa.gattn_forward(rp_t, ci_t, c.q, c.k, c.v, c.e, mode=wl.mode, scale=wl.scale, clip=wl.clip,
                             eps=wl.eps, path=path, rw=rw, workspace=workspace)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
@pytest.mark.parametrize("partition", ["balanced", "node"])
def test_configs_gather(gsa, cfg, partition):
    c = case(cfg)
    ref, mag = c.oracle_forward()
    out = gpu_forward(gsa, c, "gather", workspace=partition == "balanced")
    err = check_forward(out, ref, mag, c.wl.dtype)
    print(f"config {cfg} gather ({partition} partition): error {err:.3e}")


def test_config5_mfma(gsa):
    c = case(5)
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    rw = gsa.gattn_build_rowwindows(rp, ci, c.n)
    assert gsa.gattn_forward_path(rp, ci, c.q, c.k, c.v, rw=rw) == "mfma"
    ref, mag = c.oracle_forward()
    out = gpu_forward(gsa, c, "mfma", rw=rw)
    err = check_forward(out, ref, mag, "f16")
    print(f"config 5 mfma: rel-L2 {err:.3e}")


@pytest.mark.slow
def test_config4_full(gsa):
    # the full path on the large power-law graph (2.45M destinations, 101M
    # edges, bf16): device CSR, then the forward; every output row is compared
    # with the oracle, in chunks of rows
    c = case(4)
    rp, ci, _ = gsa.gattn_build_csr(c.src, c.dst, c.n)
    assert torch.equal(rp.cpu(), torch.from_numpy(c.rp)) and torch.equal(ci.cpu(), torch.from_numpy(c.ci))
    out = gsa.gattn_forward(rp, ci, c.q, c.k, c.v, mode="standard", scale=c.wl.scale, path="gather")
    y_all = out.cpu()
    chk = ForwardCheck("bf16")
    step = 400_000
    for r0 in range(0, c.n, step):
        rows = np.arange(r0, min(r0 + step, c.n), dtype=np.int32)
        ref, mag = c.oracle_forward(rows=rows, threads=16)
        chk.add(y_all[r0:r0 + rows.shape[0]].double().numpy(), ref, mag)
    assert chk.rows == c.n
    err = chk.finish()
    print(f"config 4, all {c.n} rows: rel-L2 {err:.3e}, worst element at {chk.elem:.3f} of its bound")


# ---- a matrix of small random cases ------------------------------------------------

def small_case(n, deg_max, h, d, dtype, mode, with_e, seed, multi=False):
    src, dst = W.random_graph(800 + seed, seed, n, deg_max, multi=multi)
    rp, ci, pe = oracle.build_csr(n, src, dst)
    g = np.random.default_rng(seed)
    mk = lambda *s: W.cast(g.standard_normal(s, dtype=np.float32) * 1.5, dtype)
    q, k, v = mk(n, h, d), mk(n, h, d), mk(n, h, d)
    e = mk(src.shape[0], h, d) if with_e else None
    return rp, ci, q, k, v, e


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode", ["standard", "clipped"])
@pytest.mark.parametrize("with_e", [False, True])
@pytest.mark.parametrize("hd", [(1, 16), (3, 32), (8, 64), (2, 128), (8, 16), (5, 128)])
@pytest.mark.parametrize("ws", [None, True], ids=["node", "balanced"])
def test_matrix_gather(gsa, dtype, mode, with_e, hd, ws):
    h, d = hd
    seed = (h * 131 + d) % 97 + (7 if with_e else 0) + (3 if mode == "clipped" else 0)
    n = 203
    rp, ci, q, k, v, e = small_case(n, 40, h, d, dtype, mode, with_e, seed)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v),
                              None if e is None else oracle.widen(e), mode=mode, scale=scale, want_mag=True)
    out = gsa.gattn_forward(torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), q.cuda(), k.cuda(), v.cuda(),
                            None if e is None else e.cuda(), mode=mode, scale=scale, path="gather", workspace=ws)
    check_forward(out, ref, mag, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [(1, 32), (8, 64), (3, 128), (2, 64)])
@pytest.mark.parametrize("n", [16, 45, 300])
def test_matrix_mfma(gsa, dtype, hd, n):
    h, d = hd
    rp, ci, q, k, v, _ = small_case(n, min(n, 48), h, d, dtype, "standard", False, n + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), scale=scale, want_mag=True)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    out = gsa.gattn_forward(rp_t, ci_t, q.cuda(), k.cuda(), v.cuda(), scale=scale, path="mfma", rw=rw)
    check_forward(out, ref, mag, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", ["wide", "rising"])
def test_mfma_logit_ranges(gsa, dtype, shape):
    # The MFMA kernel moves a row's reference max only when a logit exceeds it
    # by more than 2^8 (log2 units), rescaling the row's sums then.  "wide":
    # logits with a spread of tens of natural units, so references move on
    # most tiles; "rising": every later column (sorted, so every later tile)
    # has a larger logit, so every tile of a long row moves the reference.
    n, h, d = 300, 2, 64
    rp, ci, q, k, v, _ = small_case(n, 48 if shape == "wide" else 150, h, d, dtype, "standard", False, 71)
    if shape == "wide":
        q, k = W.cast(q.float().numpy() * 4, dtype), W.cast(k.float().numpy() * 4, dtype)
    else:
        u = np.random.default_rng(5).standard_normal((h, d)).astype(np.float32)
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        q = W.cast(np.broadcast_to(u * 8.0, (n, h, d)).copy(), dtype)
        ramp = np.linspace(0.0, 60.0, n, dtype=np.float32)[:, None, None]
        k = W.cast(ramp * u[None], dtype)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), scale=scale, want_mag=True)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    out = gsa.gattn_forward(rp_t, ci_t, q.cuda(), k.cuda(), v.cuda(), scale=scale, path="mfma", rw=rw)
    assert torch.isfinite(out).all()
    check_forward(out, ref, mag, dtype)


@pytest.mark.parametrize("path", ["gather", "gather-node", "mfma"])
def test_hubs_and_isolated(gsa, path):
    # destinations far above a workgroup's share (split over all slots and
    # merged in LDS), isolated destinations, single in-edges
    n = 6000
    g = np.random.default_rng(11)
    srcs, dsts = [], []
    for hub, deg in [(5, 5000), (17, 2000), (5500, 300), (5501, 70)]:
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, hub))
    for i in range(100, 5000, 3):
        deg = 1 + (i // 3) % 9
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, i))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    rp, ci, pe = oracle.build_csr(n, src, dst)
    h, d, dtype = (1, 64, "f16") if path == "mfma" else (2, 32, "f32")
    mk = lambda *s: W.cast(g.standard_normal(s, dtype=np.float32), dtype)
    q, k, v = mk(n, h, d), mk(n, h, d), mk(n, h, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), scale=scale, want_mag=True)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n) if path == "mfma" else None
    out = gsa.gattn_forward(rp_t, ci_t, q.cuda(), k.cuda(), v.cuda(), scale=scale, path=path.split("-")[0], rw=rw,
                            workspace=path != "gather-node")
    check_forward(out, ref, mag, dtype)
    deg = np.diff(rp)
    one = np.flatnonzero(deg == 1)
    assert one.size > 0
    # a single in-edge has weight exactly 1: the output is v of its source
    assert torch.equal(out[torch.from_numpy(one).cuda()].cpu(), v[torch.from_numpy(ci[rp[one]]).long()])


def test_empty_and_edge_cases(gsa):
    for n in (0, 1, 15, 17):
        rp = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
        ci = torch.zeros(0, dtype=torch.int32, device="cuda")
        q = torch.randn(n, 2, 16, device="cuda")
        for ws in (None, True):
            out = gsa.gattn_forward(rp, ci, q, q.clone(), q.clone(), mode="clipped", path="gather", workspace=ws)
            assert out.shape == q.shape and torch.all(out == 0)


@pytest.mark.parametrize("cfg", [2, 3])
def test_deterministic(gsa, cfg):
    c = case(cfg)
    for workspace in (True, None):
        a = gpu_forward(gsa, c, workspace=workspace)
        b = gpu_forward(gsa, c, workspace=workspace)
        assert torch.equal(a, b)


def test_argument_errors(gsa):
    c = case(1)
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    bad = torch.empty(c.q.numel() + 4, dtype=torch.float32, device="cuda")[1:1 + c.q.numel()].view(c.q.shape)
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(rp, ci, bad, c.k, c.v)
    assert ei.value.status == gsa.GATTN_ERR_INVALID_VALUE
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(rp, ci, c.q, c.k, c.v, path="mfma")      # fp32 has no MFMA path
    assert ei.value.status == gsa.GATTN_ERR_UNSUPPORTED
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(rp, ci, c.q, c.k, c.v, out=c.q)          # output aliases an input
    assert ei.value.status == gsa.GATTN_ERR_INVALID_VALUE
    ci_bad = ci.clone()
    ci_bad[0] = c.n + 3
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(rp, ci_bad, c.q, c.k, c.v, validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    # the device-side check: every kind of malformed CSR, and a valid one passes
    bad_rps = []
    r1 = rp.clone(); r1[0] = 1; bad_rps.append(r1)                        # row_ptr[0] != 0
    r2 = rp.clone(); r2[-1] = r2[-1] - 1; bad_rps.append(r2)              # row_ptr[N] != nnz
    r3 = rp.clone(); r3[c.n // 2] = r3[c.n // 2 + 1] + 1; bad_rps.append(r3)  # decreasing
    for r in bad_rps:
        with pytest.raises(gsa.GattnError) as ei:
            gsa.gattn_forward(r, ci, c.q, c.k, c.v, validate=True)
        assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    ci_neg = ci.clone()
    ci_neg[-1] = -1
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(rp, ci_neg, c.q, c.k, c.v, validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    assert torch.equal(gsa.gattn_forward(rp, ci, c.q, c.k, c.v, validate=True), gsa.gattn_forward(rp, ci, c.q, c.k, c.v))
    # without validation a bad index is clamped: wrong numbers, no fault
    out = gsa.gattn_forward(rp, ci_bad, c.q, c.k, c.v)
    torch.cuda.synchronize()
    assert out.shape == c.q.shape


def test_binding_refuses_bad_index_tensors(gsa):
    # The kernels read row_ptr [N + 1], col_idx [nnz], src / dst [nnz] and
    # edge_ids [nnz] over their full nominal length: the binding refuses a
    # short, mistyped or misplaced one before anything is launched.
    c = case(1)
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    with pytest.raises(ValueError, match="row_ptr"):
        gsa.gattn_forward(rp[:-1], ci, c.q, c.k, c.v)
    with pytest.raises(ValueError, match="row_ptr"):
        gsa.gattn_forward(rp.cpu(), ci, c.q, c.k, c.v)
    with pytest.raises(ValueError, match="col_idx"):
        gsa.gattn_forward(rp, ci.long(), c.q, c.k, c.v)
    with pytest.raises(ValueError, match="row_ptr"):
        gsa.gattn_aggregate(rp[:-2], ci, c.v, torch.ones(ci.numel(), c.h, device="cuda"))
    with pytest.raises(ValueError, match="row_ptr"):
        gsa.gattn_build_rowwindows(rp[:-1], ci, c.n)
    b = gsa.CsrBuilder(c.n, c.wl.nnz, "cuda")
    with pytest.raises(ValueError, match="src"):
        b(c.src[:-1], c.dst)
    with pytest.raises(ValueError, match="dst"):
        b(c.src, c.dst.long())
    with pytest.raises(ValueError, match="dst"):
        gsa.gattn_build_csr(c.src, c.dst[:-3], c.n)
    c2 = case(2)
    rp2, ci2 = torch.from_numpy(c2.rp).cuda(), torch.from_numpy(c2.ci).cuda()
    with pytest.raises(ValueError, match="edge_ids"):
        gsa.gattn_forward(rp2, ci2, c2.q, c2.k, c2.v, c2.e, mode="clipped", edge_ids=ci2[:-1])
    torch.cuda.synchronize()
