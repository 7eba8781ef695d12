"""GPU: the graph layer of the binding (Graph.from_coo, Graph.rowwindows,
forward) against the oracle and against the C-ABI-named calls it wraps.

forward(graph, ...) takes the edge tensor in the caller's COO edge order and
reaches it through the CSR's edge_perm; its results must be the oracle's (to
the forward's tolerances) and bit-identical to gattn_forward given the same
edge-id map, and to gattn_forward with E laid out by CSR position."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import case, check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_forward_with_coo_edge_tensor(gsa, dtype, mode):
    n, h, d = 181, 4, 32
    seed = 5 if mode == "standard" else 6
    src, dst = W.random_graph(700 + seed, seed, n, 25)
    g = np.random.default_rng(seed)
    mk = lambda *s: W.cast(g.standard_normal(s, dtype=np.float32), dtype)
    q, k, v, e = mk(n, h, d), mk(n, h, d), mk(n, h, d), mk(src.shape[0], h, d)
    graph = gsa.Graph.from_coo(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), n)
    orp, oci, ope = oracle.build_csr(n, src, dst)
    assert graph.nnz == src.shape[0]
    assert np.array_equal(graph.row_ptr.cpu().numpy(), orp) and np.array_equal(graph.col_idx.cpu().numpy(), oci)
    assert np.array_equal(graph.edge_perm.cpu().numpy(), ope)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(orp, oci, *(oracle.widen(t) for t in (q, k, v, e)), mode=mode, scale=scale,
                              edge_ids=ope, want_mag=True)
    qd, kd, vd, ed = q.cuda(), k.cuda(), v.cuda(), e.cuda()
    out = gsa.forward(graph, qd, kd, vd, ed, mode=mode, scale=scale)
    check_forward(out, ref, mag, dtype)
    same = gsa.gattn_forward(graph.row_ptr, graph.col_idx, qd, kd, vd, ed, mode=mode, scale=scale,
                             edge_ids=graph.edge_perm)
    assert torch.equal(out, same)
    by_position = gsa.gattn_forward(graph.row_ptr, graph.col_idx, qd, kd, vd, ed[graph.edge_perm.long()].contiguous(),
                                    mode=mode, scale=scale)
    assert torch.equal(out, by_position)


def test_forward_edge_update_in_coo_order(gsa):
    # the RTMScore batch: E and the edge update both indexed by original edge id
    c = case(2)
    graph = gsa.Graph.from_coo(torch.from_numpy(c.wl.src).cuda(), torch.from_numpy(c.wl.dst).cuda(), c.wl.num_nodes)
    # case(2) holds E by CSR position; scatter it back to the COO order
    pe = graph.edge_perm.long()
    e_coo = torch.empty_like(c.e)
    e_coo[pe] = c.e
    out, e_out = gsa.forward(graph, c.q, c.k, c.v, e_coo, mode="clipped", scale=c.wl.scale, clip=c.wl.clip,
                             eps=c.wl.eps, e_out=True)
    ref_out, ref_e = gsa.gattn_forward(graph.row_ptr, graph.col_idx, c.q, c.k, c.v, c.e, mode="clipped",
                                       scale=c.wl.scale, clip=c.wl.clip, eps=c.wl.eps, path="gather", e_out=True)
    assert torch.equal(out, ref_out)
    assert torch.equal(e_out[pe], ref_e)


def test_auto_path_uses_row_windows(gsa):
    # complete digraphs in fp16: auto builds the windows once and runs the MFMA path
    c = case(5)
    graph = gsa.Graph.from_coo(torch.from_numpy(c.wl.src).cuda(), torch.from_numpy(c.wl.dst).cuda(), c.wl.num_nodes)
    out = gsa.forward(graph, c.q, c.k, c.v, scale=c.wl.scale)
    rw = graph.rowwindows()
    assert graph.rowwindows() is rw
    assert gsa.gattn_forward_path(graph.row_ptr, graph.col_idx, c.q, c.k, c.v, rw=rw) == "mfma"
    mf = gsa.gattn_forward(graph.row_ptr, graph.col_idx, c.q, c.k, c.v, scale=c.wl.scale, path="mfma", rw=rw)
    assert torch.equal(out, mf)
    ref, mag = oracle.forward(c.rp, c.ci, c.q64, c.k64, c.v64, scale=c.wl.scale, want_mag=True, threads=8)
    check_forward(out, ref, mag, c.wl.dtype)


def test_from_coo_rejects_bad_indices(gsa):
    src = torch.tensor([0, 1, 7], dtype=torch.int32, device="cuda")
    dst = torch.tensor([1, 2, 0], dtype=torch.int32, device="cuda")
    with pytest.raises(gsa.GattnError):
        gsa.Graph.from_coo(src, dst, 5)


def test_partition_follows_the_degree_skew(gsa):
    # the power-law graph (in-degrees up to 2000, mean 3.7) takes the balanced
    # partition, the kNN batch (in-degree 10 everywhere) the node partition;
    # both bit-identical to the explicit choice
    c3 = case(3)
    g3 = gsa.Graph.from_coo(c3.src, c3.dst, c3.wl.num_nodes)
    assert g3.skewed() and g3.max_degree == int(np.diff(c3.rp).max())
    out = gsa.forward(g3, c3.q, c3.k, c3.v, scale=c3.wl.scale, path="gather")
    bal = gsa.gattn_forward(g3.row_ptr, g3.col_idx, c3.q, c3.k, c3.v, scale=c3.wl.scale, path="gather",
                            workspace=True)
    assert torch.equal(out, bal)
    c2 = case(2)
    g2 = gsa.Graph.from_coo(c2.src, c2.dst, c2.wl.num_nodes)
    assert not g2.skewed() and g2.max_degree == 10
    pe = g2.edge_perm.long()
    e_coo = torch.empty_like(c2.e)
    e_coo[pe] = c2.e
    out2 = gsa.forward(g2, c2.q, c2.k, c2.v, e_coo, mode="clipped", scale=c2.wl.scale, clip=c2.wl.clip,
                       eps=c2.wl.eps)
    node = gsa.gattn_forward(g2.row_ptr, g2.col_idx, c2.q, c2.k, c2.v, c2.e, mode="clipped", scale=c2.wl.scale,
                             clip=c2.wl.clip, eps=c2.wl.eps)
    assert torch.equal(out2, node)
    with pytest.raises(ValueError):
        gsa.forward(g2, c2.q, c2.k, c2.v, workspace="balanced")
