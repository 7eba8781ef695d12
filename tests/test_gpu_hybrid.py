"""GPU: the per-window hybrid dispatch (dense row windows on the MFMA path,
the other rows gathered) against the oracle, the plan's coverage of the rows,
its two extremes, and its argument checks."""
import ctypes
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


def mixed_inputs(num_pairs, h, d, dtype, seed):
    wl = W.gen_mixed(seed=seed, num_pairs=num_pairs)
    rp, ci, _ = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
    g = np.random.default_rng(seed + 100)
    mk = lambda: W.cast(g.standard_normal((wl.num_nodes, h, d), dtype=np.float32), dtype)
    return wl.num_nodes, rp, ci, mk(), mk(), mk()


def plan_rows(hy, n):
    """Rows of the dense windows and of the gather ranges, from the device lists."""
    dense = hy.dense_windows[:hy.num_dense].cpu().numpy()
    rng = hy.ranges[:2 * hy.num_ranges].cpu().numpy().reshape(-1, 2)
    rows_mfma = np.concatenate([np.arange(16 * w, min(16 * w + 16, n)) for w in dense]) if dense.size else np.zeros(0, int)
    rows_gather = np.concatenate([np.arange(s, s + c) for s, c in rng]) if rng.size else np.zeros(0, int)
    return dense, rng, rows_mfma, rows_gather


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [(8, 64), (2, 32), (3, 128)])
def test_hybrid_matches_oracle(gsa, dtype, hd):
    h, d = hd
    n, rp, ci, q, k, v = mixed_inputs(20, h, d, dtype, 3 + h)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), scale=scale, want_mag=True,
                              threads=8)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    hy = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc, min_density=0.25)
    assert hy.num_dense > 0 and hy.num_ranges > 0
    # every row exactly once: dense windows' rows and the ranges' rows
    dense, rng, rows_mfma, rows_gather = plan_rows(hy, n)
    assert np.all(np.diff(dense) > 0)
    assert np.all(rng[:, 1] >= 1) and np.all(rng[:, 1] <= hy.range_rows)
    both = np.concatenate([rows_mfma, rows_gather])
    assert both.size == n and np.array_equal(np.sort(both), np.arange(n))
    # the dense windows are those at or above the density
    deg = np.diff(rp)
    wcp = rw.win_col_ptr.cpu().numpy()
    for w in range((n + 15) // 16):
        e = int(deg[16 * w:16 * w + 16].sum())
        cols = int(wcp[w + 1] - wcp[w])
        assert (w in set(dense.tolist())) == (cols > 0 and e >= 0.25 * 16 * cols)
    assert gsa.gattn_forward_path(rp_t, ci_t, qc, kc, vc, rw=rw, hybrid=hy) == "hybrid"
    out = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, scale=scale, path="hybrid", rw=rw, hybrid=hy)
    err = check_forward(out, ref, mag, dtype)
    again = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, scale=scale, rw=rw, hybrid=hy)   # AUTO takes the plan
    assert torch.equal(out, again)
    print(f"hybrid {dtype} H={h} D={d}: {hy.num_dense} dense windows, {hy.num_ranges} ranges, error {err:.3e}")


def test_hybrid_extremes(gsa):
    n, rp, ci, q, k, v = mixed_inputs(12, 8, 64, "f16", 5)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    # density 0: every window with columns on the MFMA path -> the MFMA path's bits
    hy0 = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc, min_density=0.0)
    wcp = rw.win_col_ptr.cpu().numpy()
    assert hy0.num_dense == int((np.diff(wcp) > 0).sum())
    out0 = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw, hybrid=hy0)
    mf = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="mfma", rw=rw)
    assert torch.equal(out0, mf)
    # density above 1: everything gathered
    hy2 = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc, min_density=2.0)
    assert hy2.num_dense == 0
    _, _, _, rows_gather = plan_rows(hy2, n)
    assert np.array_equal(np.sort(rows_gather), np.arange(n))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), want_mag=True, threads=8)
    out2 = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw, hybrid=hy2)
    check_forward(out2, ref, mag, "f16")


def test_hybrid_mixed_workload(gsa):
    # the full mixed-density batch of the benchmark's hybrid variant
    wl = W.make(6)
    rp, ci, _ = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
    q, k, v = (W.cast(x, wl.dtype) for x in (wl.q(), wl.k(), wl.v()))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v), scale=wl.scale,
                              want_mag=True, threads=8)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, wl.num_nodes)
    hy = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc)
    out = gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, scale=wl.scale, path="hybrid", rw=rw, hybrid=hy)
    err = check_forward(out, ref, mag, wl.dtype)
    print(f"mixed workload hybrid: {hy.num_dense} dense windows, {hy.num_ranges} ranges, rel-L2 {err:.3e}")


def test_auto_path_density_rule(gsa):
    # Without a plan, AUTO takes the MFMA path for row windows whose tiles are
    # at least 9% full overall: the mixed batch (about 12%) goes to the matrix
    # cores, the power-law graph (about 6%, with hubs) stays gathered
    for cfg, want in ((6, "mfma"), (3, "gather")):
        wl = W.make(cfg)
        rp, ci, _ = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
        rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
        q = W.cast(wl.q(), wl.dtype).cuda()
        rw = gsa.gattn_build_rowwindows(rp_t, ci_t, wl.num_nodes)
        density = wl.nnz / (16.0 * rw.num_cols)
        print(f"config {cfg}: tile density {density:.3f}", flush=True)
        assert (density >= 0.09) == (want == "mfma")
        assert gsa.gattn_forward_path(rp_t, ci_t, q, q, q, rw=rw) == want


def test_hybrid_errors(gsa):
    n, rp, ci, q, k, v = mixed_inputs(4, 2, 32, "f16", 9)
    rp_t, ci_t = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    rw = gsa.gattn_build_rowwindows(rp_t, ci_t, n)
    with pytest.raises(gsa.GattnError):        # fp32 has no MFMA path, so no hybrid plan
        gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc.float())
    with pytest.raises(gsa.GattnError):        # the hybrid path needs a plan
        gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw)
    hy = gsa.gattn_build_hybrid(rp_t, ci_t, rw, qc, min_density=2.0)
    assert hy.num_ranges > 0
    bad = gsa.Hybrid(hy.num_dense, hy.num_ranges, 100000, hy.dense_windows, hy.ranges)
    with pytest.raises(gsa.GattnError):        # ranges larger than the gather path stages
        gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw, hybrid=bad)
    bad = gsa.Hybrid(n, hy.num_ranges, hy.range_rows, hy.dense_windows, hy.ranges)
    with pytest.raises(gsa.GattnError):        # more dense windows than the graph has
        gsa.gattn_forward(rp_t, ci_t, qc, kc, vc, path="hybrid", rw=rw, hybrid=bad)
