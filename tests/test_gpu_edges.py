"""GPU: the per-edge extensions of the gather path against the oracle --
the RTMScore edge update (e_out), the edge-id indirection of per-edge rows,
and weighted aggregation with given per-edge weights (gattn_aggregate).

Tolerances are those of the forward (tests/parity.py): fp32 componentwise
against the oracle's magnitude of the same sum, fp16 / bf16 relative L2 plus
the per-element bound.  The edge update is one product per element, so its
bounds are relative to the element itself."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import FP32_TOL, REL_L2_TOL, case, check_forward, componentwise, half_elementwise, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


def check_edges(y_gpu, ref, dtype):
    y = y_gpu.detach().float().cpu().double().numpy()
    assert not np.isnan(ref).any(), "the oracle left an edge row unwritten"
    if dtype == "f32":
        err = componentwise(y, ref, np.abs(ref))
        assert err <= FP32_TOL, f"fp32 edge-update error {err:.3e} > {FP32_TOL}"
    else:
        err = rel_l2(y, ref)
        assert err <= REL_L2_TOL[dtype], f"{dtype} edge-update rel-L2 {err:.3e} > {REL_L2_TOL[dtype]}"
        elem = half_elementwise(y, ref, np.abs(ref), dtype)
        assert elem <= 1.0, f"{dtype} edge-update element error {elem:.3f} of its bound"
    return err


def random_inputs(n, deg_max, h, d, dtype, seed, multi=False):
    """A shuffled COO graph with isolated destinations, node features and an
    edge tensor in the COO's own edge order."""
    src, dst = W.random_graph(900 + seed, seed, n, deg_max, multi=multi)
    g = np.random.default_rng(seed)
    mk = lambda *s: W.cast(g.standard_normal(s, dtype=np.float32) * 1.5, dtype)
    return src, dst, mk(n, h, d), mk(n, h, d), mk(n, h, d), mk(src.shape[0], h, d)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("hd", [(1, 16), (3, 32), (8, 64), (2, 128)])
@pytest.mark.parametrize("ws", [None, True], ids=["node", "balanced"])
def test_edge_update_with_edge_ids(gsa, dtype, hd, ws):
    # E stays in COO order; the device CSR's edge_perm addresses it
    h, d = hd
    n = 203
    src, dst, q, k, v, e = random_inputs(n, 40, h, d, dtype, h * 7 + d)
    rp, ci, pe = gsa.gattn_build_csr(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), n)
    orp, oci, ope = oracle.build_csr(n, src, dst)
    assert np.array_equal(pe.cpu().numpy(), ope)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag, ref_e = oracle.forward(orp, oci, *(oracle.widen(t) for t in (q, k, v, e)), mode="clipped",
                                     scale=scale, edge_ids=ope, want_mag=True, want_e_out=True)
    out, e_out = gsa.gattn_forward(rp, ci, q.cuda(), k.cuda(), v.cuda(), e.cuda(), mode="clipped", scale=scale,
                                   path="gather", edge_ids=pe, e_out=True, validate=True, workspace=ws)
    check_forward(out, ref, mag, dtype)
    check_edges(e_out, ref_e, dtype)
    # the same arithmetic as E laid out by CSR position: identical bits
    e_csr = e.cuda()[pe.long()].contiguous()
    out2, e_out2 = gsa.gattn_forward(rp, ci, q.cuda(), k.cuda(), v.cuda(), e_csr, mode="clipped", scale=scale,
                                     path="gather", e_out=True, workspace=ws)
    assert torch.equal(out, out2)
    assert torch.equal(e_out, e_out2[torch.argsort(pe.long())])


@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_edge_ids_without_edge_update(gsa, mode):
    h, d, n = 4, 32, 150
    src, dst, q, k, v, e = random_inputs(n, 30, h, d, "f32", 41 if mode == "standard" else 42)
    rp, ci, pe = gsa.gattn_build_csr(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), n)
    orp, oci, ope = oracle.build_csr(n, src, dst)
    ref, mag = oracle.forward(orp, oci, *(oracle.widen(t) for t in (q, k, v, e)), mode=mode, edge_ids=ope,
                              want_mag=True)
    out = gsa.gattn_forward(rp, ci, q.cuda(), k.cuda(), v.cuda(), e.cuda(), mode=mode, path="gather", edge_ids=pe)
    check_forward(out, ref, mag, "f32")


def test_edge_update_rtmscore_batch(gsa):
    # the whole RTMScore batch (64 kNN graphs, H=8, D=16, fp32, clipped with E)
    c = case(2)
    ref, mag, ref_e = oracle.forward(c.rp, c.ci, c.q64, c.k64, c.v64, c.e64, mode="clipped", scale=c.wl.scale,
                                     clip=c.wl.clip, eps=c.wl.eps, want_mag=True, want_e_out=True, threads=8)
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    out, e_out = gsa.gattn_forward(rp, ci, c.q, c.k, c.v, c.e, mode="clipped", scale=c.wl.scale, clip=c.wl.clip,
                                   eps=c.wl.eps, path="gather", e_out=True)
    err = check_forward(out, ref, mag, "f32")
    err_e = check_edges(e_out, ref_e, "f32")
    # the output does not depend on whether the edge update is written
    out_plain = gsa.gattn_forward(rp, ci, c.q, c.k, c.v, c.e, mode="clipped", scale=c.wl.scale, clip=c.wl.clip,
                                  eps=c.wl.eps, path="gather")
    assert torch.equal(out, out_plain)
    print(f"RTMScore batch: out {err:.3e}, edge update {err_e:.3e}")


def test_edge_ids_validation(gsa):
    n, h, d = 64, 2, 16
    src, dst, q, k, v, e = random_inputs(n, 8, h, d, "f32", 77)
    rp, ci, pe = gsa.gattn_build_csr(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), n)
    args = (rp, ci, q.cuda(), k.cuda(), v.cuda(), e.cuda())
    bad = pe.clone()
    bad[3] = pe.numel()                                    # out of range
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(*args, mode="clipped", edge_ids=bad, validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    dup = pe.clone()
    dup[1] = dup[0]                                        # not a permutation: fine to read, not to write
    gsa.gattn_forward(*args, mode="clipped", edge_ids=dup, validate=True)
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_forward(*args, mode="clipped", edge_ids=dup, e_out=True, validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    with pytest.raises(gsa.GattnError):                   # no edge update in the standard mode
        gsa.gattn_forward(*args, mode="standard", e_out=True)
    with pytest.raises(gsa.GattnError):                   # nor without an edge tensor
        gsa.gattn_forward(*args[:5], None, mode="clipped", e_out=True)
    # unchecked out-of-range ids are clamped: no fault, finite numbers
    wild = pe.clone()
    wild[::5] = -7
    wild[1::5] = 1 << 30
    out, e_out = gsa.gattn_forward(*args, mode="clipped", edge_ids=wild, e_out=torch.zeros_like(e.cuda()))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(e_out).all()


# ---- weighted aggregation -----------------------------------------------------------

def agg_case(n, deg_max, h, d, dtype, normalize, seed, multi=False):
    src, dst = W.random_graph(700 + seed, seed, n, deg_max, multi=multi)
    rp, ci, pe = oracle.build_csr(n, src, dst)
    g = np.random.default_rng(seed)
    x = W.cast(g.standard_normal((n, h, d), dtype=np.float32) * 1.5, dtype)
    w = g.standard_normal((src.shape[0], h), dtype=np.float32)
    if normalize:
        w = np.exp(w).astype(np.float32)                   # scores: positive
    return rp, ci, pe, x, w


def oracle_aggregate(rp, ci, x, w, normalize, eps, edge_ids=None):
    x64, w64 = oracle.widen(x), w.astype(np.float64)
    ref = oracle.aggregate(rp, ci, x64, w64, normalize=normalize, eps=eps, edge_ids=edge_ids, threads=8)
    # magnitude of the same sum: |w| |x| (positive weights when normalized)
    mag = oracle.aggregate(rp, ci, np.abs(x64), np.abs(w64), normalize=normalize, eps=eps, edge_ids=edge_ids,
                           threads=8)
    return ref, mag


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("with_ids", [False, True])
@pytest.mark.parametrize("hd", [(1, 16), (3, 32), (8, 64), (2, 128)])
@pytest.mark.parametrize("ws", [None, True], ids=["node", "balanced"])
def test_aggregate_matrix(gsa, dtype, normalize, with_ids, hd, ws):
    h, d = hd
    seed = (h * 31 + d) % 53 + (5 if normalize else 0) + (11 if with_ids else 0)
    n = 211
    rp, ci, pe, x, w = agg_case(n, 40, h, d, dtype, normalize, seed)
    ids = pe if with_ids else None
    ref, mag = oracle_aggregate(rp, ci, x, w, normalize, 1e-6, ids)
    out = gsa.gattn_aggregate(torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), x.cuda(),
                              torch.from_numpy(w).cuda(), normalize=normalize, eps=1e-6,
                              edge_ids=None if ids is None else torch.from_numpy(ids).cuda(), validate=True,
                              workspace=ws)
    check_forward(out, ref, mag, dtype)


@pytest.mark.parametrize("cfg", [2, 3])
def test_aggregate_workload_graphs(gsa, cfg):
    # the RTMScore batch and the power-law graph, V as features, seeded weights
    c = case(cfg)
    g = np.random.default_rng(100 + cfg)
    w = np.exp(g.standard_normal((c.ci.shape[0], c.h), dtype=np.float32)).astype(np.float32)
    x = c.v.cpu()
    for normalize in (False, True):
        ref, mag = oracle_aggregate(c.rp, c.ci, x, w, normalize, 1e-6)
        out = gsa.gattn_aggregate(torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda(), c.v,
                                  torch.from_numpy(w).cuda(), normalize=normalize)
        err = check_forward(out, ref, mag, c.wl.dtype)
        print(f"config {cfg} aggregate normalize={normalize}: error {err:.3e}")


def test_aggregate_reproduces_attention(gsa):
    # weights = the oracle's attention weights alpha: the aggregation is the
    # forward's SpMM step alone, so it must give the forward's output
    n, h, d = 180, 4, 32
    rp, ci, pe, x, _ = agg_case(n, 30, h, d, "f32", False, 3)
    g = np.random.default_rng(9)
    q, k = (W.cast(g.standard_normal((n, h, d), dtype=np.float32), "f32") for _ in range(2))
    ref, alpha = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(x), want_alpha=True)
    w = alpha.astype(np.float32)
    out = gsa.gattn_aggregate(torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), x.cuda(),
                              torch.from_numpy(w).cuda())
    _, mag = oracle_aggregate(rp, ci, x, w, False, 0.0)
    err = componentwise(out.cpu().double().numpy(), ref, mag)
    assert err <= 2 * FP32_TOL   # alpha rounded to fp32 adds one rounding per term


def test_aggregate_edge_cases(gsa):
    dev = "cuda"
    # no edges at all: exact zeros
    x = torch.randn(10, 2, 16, device=dev)
    rp = torch.zeros(11, dtype=torch.int32, device=dev)
    ci = torch.zeros(0, dtype=torch.int32, device=dev)
    w = torch.zeros(0, 2, dtype=torch.float32, device=dev)
    for normalize in (False, True):
        out = gsa.gattn_aggregate(rp, ci, x, w, normalize=normalize, validate=True)
        assert torch.equal(out, torch.zeros_like(x))
    # no nodes
    out = gsa.gattn_aggregate(torch.zeros(1, dtype=torch.int32, device=dev), ci, x[:0], w)
    assert out.shape == (0, 2, 16)
    # one edge, weight 1, no normalization: the source row itself, bit for bit
    rp = torch.tensor([0, 0, 1, 1], dtype=torch.int32, device=dev)
    ci = torch.tensor([2], dtype=torch.int32, device=dev)
    x = torch.randn(3, 4, 64, device=dev).half()
    out = gsa.gattn_aggregate(rp, ci, x, torch.ones(1, 4, device=dev))
    assert torch.equal(out[1], x[2]) and torch.equal(out[0], torch.zeros_like(x[0]))
    # a malformed graph is reported with validation
    bad = torch.tensor([0, 0, 1, 2], dtype=torch.int32, device=dev)
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_aggregate(bad, ci, x, torch.ones(1, 4, device=dev), validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    with pytest.raises(gsa.GattnError) as ei:
        gsa.gattn_aggregate(rp, ci, x, torch.ones(1, 4, device=dev), edge_ids=torch.tensor(
            [1], dtype=torch.int32, device=dev), validate=True)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH


def test_aggregate_hubs_deterministic(gsa):
    # destinations spread over many slots and workgroups; two runs, identical bits
    n = 5000
    g = np.random.default_rng(21)
    srcs, dsts = [], []
    for hub, deg in [(3, 4000), (4000, 900)]:
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, hub))
    for i in range(10, 3900, 2):
        deg = 1 + i % 7
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, i))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    rp, ci, pe = oracle.build_csr(n, src, dst)
    x = W.cast(g.standard_normal((n, 2, 64), dtype=np.float32), "bf16")
    w = np.exp(g.standard_normal((src.shape[0], 2), dtype=np.float32)).astype(np.float32)
    ref, mag = oracle_aggregate(rp, ci, x, w, True, 1e-6, pe)
    args = (torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), x.cuda(), torch.from_numpy(w).cuda())
    out = gsa.gattn_aggregate(*args, normalize=True, edge_ids=torch.from_numpy(pe).cuda())
    out2 = gsa.gattn_aggregate(*args, normalize=True, edge_ids=torch.from_numpy(pe).cuda())
    assert torch.equal(out, out2)
    check_forward(out, ref, mag, "bf16")
