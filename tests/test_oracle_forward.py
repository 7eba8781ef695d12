"""Pins of the oracle's fused forward (CPU only).

Each check below comes from outside the oracle's own code:
* dense all-pairs brute force on tiny simple graphs (masked N x N softmax);
* an edge-list gather / scatter-add formulation restated from the
  gattn-triton article's eager PyTorch attention (multigraphs);
* torch's scaled_dot_product_attention (fp64, CPU) on complete digraphs,
  where the standard sparse softmax is dense attention per graph;
* scipy.sparse D^-1 A V when every logit is equal;
* closed forms of the clipped mode (Q = 0, saturation at either bound);
* the hand-checked clip-order example under tests/golden/;
* invariants: edge order, node relabelling, head independence, linearity
  in V, weights summing to 1 (standard) or S/(S+eps) (clipped).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.sparse as sp
from hypothesis import given, settings, strategies as st

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def feats(seed, n, m, h, d, with_e):
    g = np.random.default_rng(seed)
    q = g.standard_normal((n, h, d))
    k = g.standard_normal((n, h, d))
    v = g.standard_normal((n, h, d))
    e = g.standard_normal((m, h, d)) if with_e else None
    return q, k, v, e


def dense_bruteforce(n, src, dst, q, k, v, e_by_edge, mode, scale, lo, hi, eps):
    """All-pairs masked attention; simple graphs only."""
    h, d = q.shape[1:]
    A = np.zeros((n, n), bool)
    A[dst, src] = True
    Ed = np.ones((n, n, h, d))
    if e_by_edge is not None:
        Ed[dst, src] = e_by_edge
    prod = q[:, None, :, :] * k[None, :, :, :]                      # [i, j, h, d]
    if mode == "standard":
        L = scale * (prod * Ed).sum(-1)                              # [i, j, h]
        L = np.where(A[..., None], L, -np.inf)
        m = L.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        w = np.where(A[..., None], np.exp(L - m), 0.0)
        Z = w.sum(axis=1, keepdims=True)
        alpha = np.divide(w, Z, out=np.zeros_like(w), where=Z > 0)
    else:
        T = np.clip(scale * prod, lo, hi) * Ed
        L = np.clip(T.sum(-1), lo, hi)
        s = np.where(A[..., None], np.exp(L), 0.0)
        Z = s.sum(axis=1, keepdims=True) + eps
        alpha = np.divide(s, Z, out=np.zeros_like(s), where=Z > 0)
    return np.einsum("ijh,jhd->ihd", alpha, v)


def edgelist_formulation(n, src, dst, q, k, v, e_by_edge, mode, scale, lo, hi, eps):
    """Gather by source / destination, score per edge, scatter-add per
    destination (the eager formulation of the gattn-triton article)."""
    h, d = q.shape[1:]
    prod = q[dst] * k[src]                                             # [M, h, d]
    ee = e_by_edge if e_by_edge is not None else 1.0
    if mode == "standard":
        L = scale * (prod * ee).sum(-1)                                  # [M, h]
        m = np.full((n, h), -np.inf)
        np.maximum.at(m, dst, L)
        w = np.exp(L - m[dst])
        Z = np.zeros((n, h))
        np.add.at(Z, dst, w)
    else:
        L = np.clip((np.clip(scale * prod, lo, hi) * ee).sum(-1), lo, hi)
        w = np.exp(L)
        Z = np.zeros((n, h))
        np.add.at(Z, dst, w)
        Z = Z + eps
    num = np.zeros((n, h, d))
    np.add.at(num, dst, w[..., None] * v[src])
    return np.divide(num, Z[..., None], out=np.zeros_like(num), where=Z[..., None] > 0)


def run_oracle(orc, n, src, dst, q, k, v, e_by_edge, mode, scale, clip=(-5.0, 5.0), eps=1e-6, **kw):
    rp, ci, pe = orc.build_csr(n, src, dst)
    e_csr = None if e_by_edge is None else e_by_edge[pe]
    return orc.forward(rp, ci, q, k, v, e_csr, mode=mode, scale=scale, clip=clip, eps=eps, **kw)


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 40), h=st.sampled_from([1, 3]), d=st.sampled_from([2, 4, 16]),
       mode=st.sampled_from(["standard", "clipped"]), with_e=st.booleans(),
       seed=st.integers(0, 10_000), self_loops=st.booleans())
def test_dense_bruteforce(orc, n, h, d, mode, with_e, seed, self_loops):
    src, dst = W.random_graph(900, seed, n, 10, allow_self=self_loops)
    q, k, v, e = feats(seed, n, src.shape[0], h, d, with_e)
    if mode == "clipped":
        q *= 3.0   # push some products and sums past the clip bounds
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = run_oracle(orc, n, src, dst, q, k, v, e, mode, scale)
    ref = dense_bruteforce(n, src, dst, q, k, v, e, mode, scale, -5.0, 5.0, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["standard", "clipped"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_magnitude_is_weighted_abs_sum(orc, mode, seed):
    """S = sum_p alpha_p |v_p|, the scale that the fp32 and half-precision
    tolerances are measured against, equals the dense brute force run on |V|
    (independent code, same weights) and, bit for bit, the oracle's own
    output with V replaced by |V| (same weights, same summation order)."""
    n = [9, 23, 37][seed]
    src, dst = W.random_graph(960, seed, n, 12)
    q, k, v, e = feats(seed, n, src.shape[0], 2, 8, True)
    q *= 2.0
    out, mag = run_oracle(orc, n, src, dst, q, k, v, e, mode, 0.3, want_mag=True)
    ref = dense_bruteforce(n, src, dst, q, k, np.abs(v), e, mode, 0.3, -5.0, 5.0, 1e-6)
    np.testing.assert_allclose(mag, ref, rtol=0, atol=1e-12)
    assert np.array_equal(mag, run_oracle(orc, n, src, dst, q, k, np.abs(v), e, mode, 0.3))
    assert np.all(mag >= np.abs(out) - 1e-12)
    # a row subset returns the same magnitudes
    rows = np.arange(n - 1, -1, -2, dtype=np.int32)
    _, mag_rows = run_oracle(orc, n, src, dst, q, k, v, e, mode, 0.3, want_mag=True, rows=rows)
    assert np.array_equal(mag_rows, mag[rows])


@settings(max_examples=40, deadline=None)
@given(n=st.integers(1, 30), h=st.sampled_from([1, 2]), d=st.sampled_from([4, 8]),
       mode=st.sampled_from(["standard", "clipped"]), with_e=st.booleans(), seed=st.integers(0, 10_000))
def test_edgelist_multigraph(orc, n, h, d, mode, with_e, seed):
    src, dst = W.random_graph(901, seed, n, 8, multi=True)
    q, k, v, e = feats(seed, n, src.shape[0], h, d, with_e)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    got = run_oracle(orc, n, src, dst, q, k, v, e, mode, scale)
    ref = edgelist_formulation(n, src, dst, q, k, v, e, mode, scale, -5.0, 5.0, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_sdpa_complete_digraphs(orc):
    import torch
    g = np.random.default_rng(5)
    sizes = [20, 33, 40, 1, 27]
    n = sum(sizes)
    src, dst, off = [], [], 0
    for s in sizes:
        a = np.arange(s) + off
        src.append(np.tile(a, s))
        dst.append(np.repeat(a, s))
        off += s
    src, dst = np.concatenate(src), np.concatenate(dst)
    h, d = 8, 64
    q, k, v = (g.standard_normal((n, h, d)) for _ in range(3))
    scale = float(np.float32(1.0 / 8.0))
    got = run_oracle(orc, n, src, dst, q, k, v, None, "standard", scale)
    off = 0
    for s in sizes:
        sl = slice(off, off + s)
        Q, K, V = (torch.from_numpy(np.ascontiguousarray(x[sl].transpose(1, 0, 2)))[None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(got[sl], ref, rtol=0, atol=1e-12)
        off += s


@pytest.mark.parametrize("cfg", [1, 3])
def test_equal_logits_give_scipy_mean(orc, cfg):
    wl = W.make(cfg)
    n, h, d = wl.num_nodes, wl.heads, wl.head_dim
    v = wl.v().astype(np.float64)
    q = np.zeros_like(v)
    k = wl.k().astype(np.float64)
    got = run_oracle(orc, n, wl.src, wl.dst, q, k, v, None, "standard", wl.scale)
    A = sp.csr_matrix((np.ones(wl.nnz), (wl.dst, wl.src)), shape=(n, n))
    deg = np.asarray(A.sum(axis=1)).ravel()
    Dinv = sp.diags(np.divide(1.0, deg, out=np.zeros_like(deg), where=deg > 0))
    for hh in range(h):
        ref = Dinv @ (A @ v[:, hh, :])
        np.testing.assert_allclose(got[:, hh, :], ref, rtol=0, atol=1e-12)


def neighbour_mean(n, src, dst, v):
    num = np.zeros_like(v)
    np.add.at(num, dst, v[src])
    deg = np.bincount(dst, minlength=n).astype(np.float64)
    return num / np.maximum(deg, 1)[:, None, None], deg


def test_clipped_closed_forms(orc):
    wl = W.make(2)
    n, h, d = wl.num_nodes, wl.heads, wl.head_dim
    v = wl.v().astype(np.float64)
    k = wl.k().astype(np.float64)
    e = wl.e().astype(np.float64)          # arbitrary E: with q = 0 every logit is 0
    mean, deg = neighbour_mean(n, wl.src, wl.dst, v)
    eps = 1e-6
    got = run_oracle(orc, n, wl.src, wl.dst, np.zeros_like(v), k, v, e, "clipped", wl.scale)
    np.testing.assert_allclose(got, (deg / (deg + eps))[:, None, None] * mean, rtol=1e-13, atol=1e-15)
    assert abs(10 / (10 + eps) - 0.99999990000001) < 1e-15
    # saturation: every scaled q*k product clamps to the bound, E = 1
    for sign, bound in [(1.0, 5.0), (-1.0, -5.0)]:
        q1 = np.ones_like(v)
        kk = np.full_like(v, 1000.0 * sign)
        got = run_oracle(orc, n, wl.src, wl.dst, q1, kk, v, np.ones_like(e), "clipped", wl.scale)
        s = math.exp(bound)
        np.testing.assert_allclose(got, (deg * s / (deg * s + eps))[:, None, None] * mean, rtol=1e-13, atol=1e-15)


def test_clip_order_worked_example(orc):
    fx = json.load(open(os.path.join(GOLDEN, "clip_order_example.json")))
    q, k, v = (np.array(fx[x], np.float64) for x in ("q", "k", "v"))
    e = np.array(fx["e_by_edge"], np.float64)
    src, dst = np.array(fx["edges_src"]), np.array(fx["edges_dst"])
    out, alpha = run_oracle(orc, fx["num_nodes"], src, dst, q, k, v, e, "clipped", fx["scale"],
                            clip=tuple(fx["clip"]), eps=fx["eps"], want_alpha=True)
    eps = fx["eps"]
    zc = math.exp(0.5) + 1 + eps
    a_code = [math.exp(0.5) / zc, 1 / zc]
    assert alpha[:2, 0] == pytest.approx(a_code, rel=1e-15)
    assert out[0, 0] == pytest.approx(a_code, rel=1e-15)      # v_a = e_x, v_b = e_y
    assert a_code[0] == pytest.approx(0.6224590962, abs=1e-10)
    zp = math.exp(5) + 1 + eps
    assert abs(alpha[0, 0] - math.exp(5) / zp) > 0.3            # the single-clip reading differs
    assert np.all(out[1:] == 0.0)                               # nodes without in-edges


def test_isolated_and_single_edge_exact(orc):
    n = 4
    src, dst = np.array([2, 0, 1], np.int32), np.array([1, 3, 3], np.int32)   # node 0, 2 isolated
    q, k, v, e = feats(7, n, 3, 2, 8, True)
    for mode in ("standard", "clipped"):
        out = run_oracle(orc, n, src, dst, q, k, v, e, mode, 0.35)
        assert np.all(out[0] == 0.0) and np.all(out[2] == 0.0)
        if mode == "standard":
            assert np.array_equal(out[1], v[2])                  # alpha = exp(0)/1 = 1 exactly
        else:
            t = np.clip(0.35 * q[1] * k[2], -5, 5) * e[0]
            s = np.exp(np.clip(t.sum(-1), -5, 5))
            np.testing.assert_allclose(out[1], (s / (s + 1e-6))[:, None] * v[2], rtol=1e-14)
    # eps = 0 keeps isolated nodes at exactly zero
    out = run_oracle(orc, n, src, dst, q, k, v, None, "clipped", 0.35, eps=0.0)
    assert np.all(out[0] == 0.0)


def test_modes_agree_without_clip_and_eps(orc):
    wl = W.make(1)
    q, k, v = (x.astype(np.float64) for x in (wl.q(), wl.k(), wl.v()))
    a = run_oracle(orc, wl.num_nodes, wl.src, wl.dst, q, k, v, None, "standard", wl.scale)
    b = run_oracle(orc, wl.num_nodes, wl.src, wl.dst, q, k, v, None, "clipped", wl.scale,
                   clip=(-math.inf, math.inf), eps=0.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_weights_sum(orc, mode):
    wl = W.make(1)
    q, k, v = (x.astype(np.float64) for x in (wl.q(), wl.k(), wl.v()))
    if mode == "clipped":
        q = np.zeros_like(q)
    rp, ci, pe = orc.build_csr(wl.num_nodes, wl.src, wl.dst)
    _, alpha = orc.forward(rp, ci, q, k, v, None, mode=mode, scale=wl.scale, want_alpha=True)
    for i in range(wl.num_nodes):
        s = alpha[rp[i]:rp[i + 1]].sum(axis=0)
        deg = rp[i + 1] - rp[i]
        target = 1.0 if mode == "standard" else deg / (deg + 1e-6)
        np.testing.assert_allclose(s, target, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_invariants(orc, mode):
    n, h, d = 60, 3, 16
    src, dst = W.random_graph(902, 3, n, 12)
    q, k, v, e = feats(11, n, src.shape[0], h, d, True)
    scale = 0.25
    base = run_oracle(orc, n, src, dst, q, k, v, e, mode, scale)
    # 1. edge order: the COO order, hence the order inside each destination, is free
    perm = np.random.default_rng(1).permutation(src.shape[0])
    rp, ci, pe = orc.build_csr(n, src[perm], dst[perm])
    np.testing.assert_allclose(run_oracle(orc, n, src[perm], dst[perm], q, k, v, e[perm], mode, scale),
                               base, rtol=0, atol=1e-13)
    rp, ci, pe = orc.build_csr(n, src, dst)
    g = np.random.default_rng(2)
    pos = np.arange(ci.shape[0])
    for i in range(n):
        g.shuffle(pos[rp[i]:rp[i + 1]])
    shuffled = orc.forward(rp, ci[pos], q, k, v, e[pe][pos], mode=mode, scale=scale)
    np.testing.assert_allclose(shuffled, base, rtol=0, atol=1e-13)
    # 2. node relabelling permutes the output rows
    pi = np.random.default_rng(3).permutation(n)
    qp, kp, vp = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    qp[pi], kp[pi], vp[pi] = q, k, v
    relab = run_oracle(orc, n, pi[src], pi[dst], qp, kp, vp, e, mode, scale)
    np.testing.assert_allclose(relab[pi], base, rtol=0, atol=1e-13)
    # 3. heads are independent
    for hh in range(h):
        one = run_oracle(orc, n, src, dst, q[:, hh:hh + 1], k[:, hh:hh + 1], v[:, hh:hh + 1],
                         e[:, hh:hh + 1], mode, scale)
        assert np.array_equal(one[:, 0], base[:, hh])
    # 4. linear in V
    v2 = np.random.default_rng(4).standard_normal(v.shape)
    lin = run_oracle(orc, n, src, dst, q, k, 2.0 * v - 3.0 * v2, e, mode, scale)
    o2 = run_oracle(orc, n, src, dst, q, k, v2, e, mode, scale)
    np.testing.assert_allclose(lin, 2.0 * base - 3.0 * o2, rtol=0, atol=1e-12)


def test_rows_subset_and_threads(orc):
    wl = W.make(1)
    q, k, v = (x.astype(np.float64) for x in (wl.q(), wl.k(), wl.v()))
    rp, ci, pe = orc.build_csr(wl.num_nodes, wl.src, wl.dst)
    full = orc.forward(rp, ci, q, k, v, scale=wl.scale, threads=1)
    par = orc.forward(rp, ci, q, k, v, scale=wl.scale, threads=4)
    assert np.array_equal(full, par)
    rows = np.array([5, 0, 319, 5], np.int32)
    sub = orc.forward(rp, ci, q, k, v, scale=wl.scale, rows=rows)
    assert np.array_equal(sub, full[rows])


# ---- edge update output, edge-id indirection, weighted aggregation ---------------

def test_e_out_is_the_elementwise_update(orc):
    """The edge update (the article's per-edge store before the feature sum)
    restated as a vectorised edge-list expression."""
    n, h, d = 50, 3, 8
    src, dst = W.random_graph(910, 1, n, 12)
    q, k, v, e = feats(21, n, src.shape[0], h, d, True)
    q *= 3.0
    scale = 0.3
    rp, ci, pe = orc.build_csr(n, src, dst)
    out, e_out = orc.forward(rp, ci, q, k, v, e, mode="clipped", scale=scale, edge_ids=pe, want_e_out=True)
    ref = np.clip(scale * q[dst] * k[src], -5.0, 5.0) * e            # rows in the caller's edge order
    np.testing.assert_allclose(e_out, ref, rtol=0, atol=1e-13)
    assert np.any(np.abs(scale * q[dst] * k[src]) > 5.0)             # the clamp is exercised
    with pytest.raises(orc.OracleError):
        orc.forward(rp, ci, q, k, v, e, mode="standard", scale=scale, edge_ids=pe, want_e_out=True)


@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_edge_ids_indirection(orc, mode):
    n, h, d = 70, 2, 16
    src, dst = W.random_graph(911, 2, n, 10)
    q, k, v, e = feats(22, n, src.shape[0], h, d, True)
    rp, ci, pe = orc.build_csr(n, src, dst)
    by_position = orc.forward(rp, ci, q, k, v, e[pe], mode=mode, scale=0.25)
    by_edge_id = orc.forward(rp, ci, q, k, v, e, mode=mode, scale=0.25, edge_ids=pe)
    assert np.array_equal(by_position, by_edge_id)


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("multi", [False, True])
def test_aggregate_matches_scipy(orc, normalize, multi):
    n, h, d = 90, 3, 8
    src, dst = W.random_graph(912, 3, n, 14, multi=multi)
    g = np.random.default_rng(5)
    x = g.standard_normal((n, h, d))
    w = g.random((src.shape[0], h)) + 0.1
    rp, ci, pe = orc.build_csr(n, src, dst)
    out = orc.aggregate(rp, ci, x, w, normalize=normalize, eps=1e-6, edge_ids=pe)
    for hh in range(h):
        A = sp.csr_matrix((w[:, hh], (dst, src)), shape=(n, n))          # repeated pairs add up
        ref = A @ x[:, hh, :]
        if normalize:
            z = np.asarray(A.sum(axis=1)).ravel()
            deg = np.bincount(dst, minlength=n)
            ref = np.where(deg[:, None] > 0, ref / (z[:, None] + 1e-6), 0.0)
        np.testing.assert_allclose(out[:, hh, :], ref, rtol=1e-13, atol=1e-13)


def test_aggregate_closed_form(orc):
    wl = W.make(1)
    x = wl.v().astype(np.float64)
    rp, ci, pe = orc.build_csr(wl.num_nodes, wl.src, wl.dst)
    ones = np.ones((wl.nnz, wl.heads))
    mean, deg = neighbour_mean(wl.num_nodes, wl.src, wl.dst, x)
    out = orc.aggregate(rp, ci, x, ones, normalize=True, eps=1e-6)
    np.testing.assert_allclose(out, (deg / (deg + 1e-6))[:, None, None] * mean, rtol=1e-13, atol=1e-15)
    out = orc.aggregate(rp, ci, x, ones, normalize=False)
    np.testing.assert_allclose(out, deg[:, None, None] * mean, rtol=1e-13, atol=1e-13)
