"""GPU: the balanced gather partition with cross-workgroup splitting of heavy
destinations (edge-parallel parts merged in order through the workspace)
against the oracle, and its workspace contract."""
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


def hub_graph(seed, n, hubs, light_rows=0, light_max=6):
    """Destinations `hubs` = [(dst, degree)] with distinct random sources, plus
    `light_rows` destinations of degree 1..light_max; the rest isolated."""
    g = np.random.default_rng(seed)
    srcs, dsts = [], []
    for hub, deg in hubs:
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, hub))
    taken = {h for h, _ in hubs}
    others = [i for i in g.choice(n, min(n, light_rows + len(taken)), replace=False) if i not in taken][:light_rows]
    for i in others:
        deg = int(g.integers(1, light_max + 1))
        srcs.append(g.choice(n, deg, replace=False))
        dsts.append(np.full(deg, i))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    perm = g.permutation(src.shape[0])
    return src[perm], dst[perm]


def run_both(gsa, n, src, dst, h, d, dtype, mode, with_e, seed, workspace=True):
    rp, ci, pe = oracle.build_csr(n, src, dst)
    g = np.random.default_rng(seed)
    mk = lambda *s: W.cast(g.standard_normal(s, dtype=np.float32) * 1.5, dtype)
    q, k, v = mk(n, h, d), mk(n, h, d), mk(n, h, d)
    e = mk(src.shape[0], h, d) if with_e else None
    scale = float(np.float32(1 / math.sqrt(d)))
    ref, mag = oracle.forward(rp, ci, oracle.widen(q), oracle.widen(k), oracle.widen(v),
                              None if e is None else oracle.widen(e), mode=mode, scale=scale, want_mag=True,
                              threads=8)
    args = (torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), q.cuda(), k.cuda(), v.cuda(),
            None if e is None else e.cuda())
    out = gsa.gattn_forward(*args, mode=mode, scale=scale, path="gather", workspace=workspace)
    return out, ref, mag, args, scale


@pytest.mark.parametrize("dtype,hd", [("f32", (4, 32)), ("f16", (1, 64)), ("bf16", (2, 128)), ("f32", (8, 16))])
@pytest.mark.parametrize("mode,with_e", [("standard", False), ("clipped", True)])
def test_one_giant_row(gsa, dtype, hd, mode, with_e):
    # one destination holding every edge: cut into many parts, most of them
    # neither the first nor the last
    h, d = hd
    n = 50000
    src, dst = hub_graph(5, n, [(123, 40000)])
    out, ref, mag, args, scale = run_both(gsa, n, src, dst, h, d, dtype, mode, with_e, 6)
    check_forward(out, ref, mag, dtype)
    again = gsa.gattn_forward(*args, mode=mode, scale=scale, path="gather", workspace=True)
    assert torch.equal(out, again)          # merge order is fixed: identical bits


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_many_hubs_and_light_rows(gsa, dtype):
    # heavy rows of many sizes (some cut in two, some in dozens), light rows
    # on both sides of every cut, isolated rows
    n = 30000
    g = np.random.default_rng(8)
    hubs = [(int(x), int(dg)) for x, dg in zip(g.choice(n, 40, replace=False),
                                             np.geomspace(200, 20000, 40).astype(int))]
    src, dst = hub_graph(9, n, hubs, light_rows=9000)
    for mode, with_e in (("standard", False), ("clipped", True)):
        out, ref, mag, _, _ = run_both(gsa, n, src, dst, 2, 32, dtype, mode, with_e, 10)
        check_forward(out, ref, mag, dtype)


def test_partitions_agree_on_power_law(gsa):
    # both partitions against the oracle on a power-law graph with hubs
    import parity
    c = parity.case(3)
    ref, mag = c.oracle_forward()
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    for workspace in (True, None):
        out = gsa.gattn_forward(rp, ci, c.q, c.k, c.v, scale=c.wl.scale, path="gather", workspace=workspace)
        check_forward(out, ref, mag, c.wl.dtype)


def test_workspace_with_stale_contents(gsa):
    # any contents on entry: garbage, then the flags of other calls and graphs
    n = 20000
    src, dst = hub_graph(12, n, [(7, 9000), (19000, 3000), (500, 700)], light_rows=5000)
    out_fresh, ref, mag, args, scale = run_both(gsa, n, src, dst, 2, 64, "f16", "standard", False, 13)
    nbytes = gsa.gattn_forward_workspace(*args[:5])
    ws = torch.randint(0, 256, (nbytes + 4096,), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        out = gsa.gattn_forward(*args, scale=scale, path="gather", workspace=ws)
        assert torch.equal(out, out_fresh)
    # another graph through the same workspace, then the first one again
    src2, dst2 = hub_graph(14, n, [(11, 12000)], light_rows=3000)
    out2, ref2, mag2, args2, _ = run_both(gsa, n, src2, dst2, 2, 64, "f16", "standard", False, 15, workspace=ws)
    check_forward(out2, ref2, mag2, "f16")
    out = gsa.gattn_forward(*args, scale=scale, path="gather", workspace=ws)
    assert torch.equal(out, out_fresh)
    check_forward(out, ref, mag, "f16")


def test_workspace_too_small(gsa):
    n = 5000
    src, dst = hub_graph(16, n, [(3, 4000)], light_rows=1000)
    _, _, _, args, scale = run_both(gsa, n, src, dst, 1, 64, "f16", "standard", False, 17)
    nbytes = gsa.gattn_forward_workspace(*args[:5])
    assert nbytes > 0
    small = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gsa.gattn_forward(*args, scale=scale, path="gather", workspace=small)
    # through the C ABI directly: the size is checked there too
    a, keep = gsa._forward_args(*args[:5], None, torch.empty_like(args[2]), "standard", scale, (-5.0, 5.0), 1e-6,
                                "gather", None, False)
    a.workspace, a.workspace_bytes = small.data_ptr(), small.numel()
    import ctypes
    st = gsa._lib.gattn_forward(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gsa.GATTN_ERR_BUFFER_TOO_SMALL
    del keep


def test_aggregate_giant_row(gsa):
    n = 40000
    src, dst = hub_graph(18, n, [(321, 30000), (5, 2500)], light_rows=2000)
    rp, ci, pe = oracle.build_csr(n, src, dst)
    g = np.random.default_rng(19)
    x = W.cast(g.standard_normal((n, 4, 32), dtype=np.float32), "f32")
    w = np.exp(g.standard_normal((src.shape[0], 4), dtype=np.float32)).astype(np.float32)
    for normalize in (False, True):
        ref = oracle.aggregate(rp, ci, oracle.widen(x), w.astype(np.float64), normalize=normalize, threads=8)
        mag = oracle.aggregate(rp, ci, np.abs(oracle.widen(x)), w.astype(np.float64), normalize=normalize, threads=8)
        out = gsa.gattn_aggregate(torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), x.cuda(),
                                  torch.from_numpy(w).cuda(), normalize=normalize)
        check_forward(out, ref, mag, "f32")
