"""GPU: q, k and v as strided row views (rows of a fused projection's output,
[N, 3, H, D] or [N, 2, H, D]) give the same bits as packed copies on every
path: gather (node and balanced partitions), MFMA, hybrid, edge features with
edge_ids and e_out, and the entry point that allocates nothing.  One case per
path is also checked against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


def graph(num_pairs, seed):
    wl = W.gen_mixed(seed=seed, num_pairs=num_pairs)
    rp, ci, _ = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
    return wl.num_nodes, rp, ci


def fused(n, parts, h, d, dtype, seed, pad=0):
    """An [N, parts, H, D] buffer (each row padded by `pad` elements) and its
    per-part [N, H, D] views, with packed copies of those views."""
    g = np.random.default_rng(seed)
    x = W.cast(g.standard_normal((n, parts * h * d + pad), dtype=np.float32), dtype).cuda()
    views = [x[:, i * h * d:(i + 1) * h * d].view(n, h, d) for i in range(parts)]
    assert all(t.stride(0) == parts * h * d + pad and not t.is_contiguous() for t in views)
    return views, [t.contiguous() for t in views]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ws", [None, True], ids=["node", "balanced"])
@pytest.mark.parametrize("hd", [(8, 64), (3, 32), (1, 128)])
def test_gather_strided_qkv(gsa, dtype, ws, hd):
    h, d = hd
    n, rp, ci = graph(16, 7 + h)
    (q, k, v), (qc, kc, vc) = fused(n, 3, h, d, dtype, 11 + d)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    scale = float(np.float32(1 / math.sqrt(d)))
    got = gsa.gattn_forward(rp_t, ci_t, q, k, v, scale=scale, path="gather", workspace=ws)
    want = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, scale=scale, path="gather", workspace=ws)
    assert torch.equal(got, want)
    if hd == (8, 64):
        ref, mag = oracle.forward(rp, ci, oracle.widen(qc.cpu()), oracle.widen(kc.cpu()), oracle.widen(vc.cpu()),
                                  scale=scale, want_mag=True, threads=8)
        check_forward(got, ref, mag, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pad", [0, 8])
def test_gather_strided_kv_padded_rows(gsa, dtype, pad):
    # k and v from [N, 2, H, D] with padded rows, q packed
    h, d = 4, 64
    n, rp, ci = graph(20, 3)
    (k, v), (kc, vc) = fused(n, 2, h, d, dtype, 5, pad)
    q = W.cast(np.random.default_rng(6).standard_normal((n, h, d), dtype=np.float32), dtype).cuda()
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    for ws in (None, True):
        got = gsa.gattn_forward(rp_t, ci_t, q, k, v, path="gather", workspace=ws)
        assert torch.equal(got, gsa.gattn_forward(rp_t, ci_t, q, kc, vc, path="gather", workspace=ws))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [(8, 64), (2, 32), (3, 128)])
def test_mfma_and_hybrid_strided(gsa, dtype, hd):
    h, d = hd
    n, rp, ci = graph(20, 9 + h)
    (q, k, v), (qc, kc, vc) = fused(n, 3, h, d, dtype, 13 + d)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    got = gsa.gattn_forward(rp_t, ci_t, q, k, v, path="mfma", rw=rw)
    want = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="mfma", rw=rw)
    assert torch.equal(got, want)
    ref, mag = oracle.forward(rp, ci, oracle.widen(qc.cpu()), oracle.widen(kc.cpu()), oracle.widen(vc.cpu()),
                              scale=1 / math.sqrt(d), want_mag=True, threads=8)
    check_forward(got, ref, mag, dtype)
    hy = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc, min_density=0.25)
    assert hy.num_dense > 0 and hy.num_ranges > 0
    got = gsa.gattn_forward(rp_t, ci_t, q, k, v, path="hybrid", rw=rw, hybrid=hy)
    assert torch.equal(got, gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw, hybrid=hy))
    check_forward(got, ref, mag, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_features_strided(gsa, dtype):
    # clipped mode with e addressed through edge_ids, and the e_out update
    h, d = 8, 32
    n, rp, ci = graph(12, 21)
    (q, k, v), (qc, kc, vc) = fused(n, 3, h, d, dtype, 17)
    nnz = ci.size
    g = np.random.default_rng(4)
    e = W.cast(g.standard_normal((nnz, h, d), dtype=np.float32), dtype).cuda()
    ids = torch.from_numpy(g.permutation(nnz).astype(np.int32)).cuda()
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    for ws in (None, True):
        kw = dict(mode="clipped", scale=0.125, edge_ids=ids, e_out=True, path="gather", workspace=ws)
        o1, e1 = gsa.gattn_forward(rp_t, ci_t, q, k, v, e, **kw)
        o2, e2 = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, e, **kw)
        assert torch.equal(o1, o2) and torch.equal(e1, e2)


def test_noalloc_strided(gsa):
    h, d = 8, 64
    n, rp, ci = graph(16, 2)
    (q, k, v), (qc, kc, vc) = fused(n, 3, h, d, "f16", 23)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    want = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="gather", workspace=True)
    out = torch.empty_like(qc)
    got = gsa.gattn_forward_noalloc(rp_t, ci_t, q, k, v, out, path="gather")
    assert torch.equal(got, want)


def test_strided_views_refused(gsa):
    n, rp, ci = graph(4, 1)
    h, d = 2, 32
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    (q, k, v), _ = fused(n, 3, h, d, "f16", 1)
    (k2, v2), _ = fused(n, 2, h, d, "f16", 2)
    with pytest.raises(ValueError, match="same row stride"):
        gsa.gattn_forward(rp_t, ci_t, q, k, v2)
    (kp,), _ = fused(n, 1, h, d, "f16", 3, pad=4)   # row stride 68: not a multiple of 8
    with pytest.raises(ValueError, match="multiple of 8"):
        gsa.gattn_forward(rp_t, ci_t, q, kp, kp)
    with pytest.raises(ValueError, match="packed"):
        gsa.gattn_forward(rp_t, ci_t, q.transpose(1, 2).contiguous().transpose(1, 2), k, v)


def test_graph_layer_strided_kv(gsa):
    # the Python graph layer passes strided views through (AUTO path: row windows)
    h, d = 4, 64
    n, rp, ci = graph(16, 8)
    (k, v), (kc, vc) = fused(n, 2, h, d, "bf16", 31)
    q = W.cast(np.random.default_rng(32).standard_normal((n, h, d), dtype=np.float32), "bf16").cuda()
    dst = torch.from_numpy(np.repeat(np.arange(n, dtype=np.int32), np.diff(rp)))   # the CSR's edges as COO
    g = gsa.Graph.from_coo(torch.from_numpy(ci).cuda(), dst.cuda(), n)
    assert torch.equal(gsa.forward(g, q, k, v), gsa.forward(g, q, kc, vc))


@pytest.mark.parametrize("seed", range(12))
def test_strided_fuzz(gsa, seed):
    # random geometry, dtype, row padding and path: strided views give the packed copies' bits
    g = np.random.default_rng(1000 + seed)
    h, d = [(1, 16), (2, 32), (4, 64), (8, 16), (3, 128), (1, 64)][g.integers(6)]
    dtype = ["f32", "f16", "bf16"][g.integers(3)]
    n, rp, ci = graph(int(g.integers(2, 10)), 50 + seed)
    parts, pad = int(g.integers(2, 4)), 8 * int(g.integers(0, 4))
    views, packed = fused(n, parts, h, d, dtype, 60 + seed, pad)
    k, v = views[-2], views[-1]
    kc, vc = packed[-2], packed[-1]
    if parts == 3:
        q, qc = views[0], packed[0]
    else:
        qc = W.cast(g.standard_normal((n, h, d), dtype=np.float32), dtype).cuda()
        q = qc
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    paths = [("gather", None), ("gather", True)] + ([("mfma", None)] if dtype != "f32" and d >= 32 else [])
    for path, ws in paths:
        rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n) if path == "mfma" else None
        got = gsa.gattn_forward(rp_t, ci_t, q, k, v, path=path, rw=rw, workspace=ws)
        want = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path=path, rw=rw, workspace=ws)
        assert torch.equal(got, want), f"{path} ws={ws} H={h} D={d} {dtype} parts={parts} pad={pad}"
