"""GPU: gattn_forward_noalloc, the forward for callers that cannot allocate
(the balanced partition with its workspace in the library's fixed scratch
array), against gattn_forward with a workspace of its own: the same kernels
and partition, so identical bits, on two calls in a row, the second with a
smaller input; both also against the oracle."""
import pytest
import torch

from parity import case, check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


def test_noalloc_matches_the_workspace_entry_point(gsa):
    # config 3 (622k edges, hub rows cut across workgroups), then the smaller
    # RTMScore batch (122k edges, edge projection, clipped softmax)
    for cfg in (3, 2):
        c = case(cfg)
        wl = c.wl
        print(f"gattn_forward_noalloc, config {cfg}", flush=True)
        rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
        kw = dict(mode=wl.mode, scale=wl.scale, clip=wl.clip, eps=wl.eps, path="gather")
        assert gsa.gattn_forward_workspace(rp, ci, c.q, c.k, c.v, c.e, wl.mode) <= gsa.GATTN_NOALLOC_SCRATCH_BYTES
        want = gsa.gattn_forward(rp, ci, c.q, c.k, c.v, c.e, workspace=True, **kw)
        out = torch.full_like(c.q, float("nan"))
        got = gsa.gattn_forward_noalloc(rp, ci, c.q, c.k, c.v, out, c.e, **kw)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, want), f"config {cfg}: the no-alloc entry point differs from gattn_forward"
        ref, mag = c.oracle_forward()
        check_forward(out, ref, mag, wl.dtype)


def test_noalloc_refuses_what_it_cannot_do(gsa):
    c = case(2)
    wl = c.wl
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    out = torch.empty_like(c.q)
    with pytest.raises(ValueError):
        gsa.gattn_forward_noalloc(rp, ci, c.q, c.k, c.v, None, c.e, mode=wl.mode)
    with pytest.raises(gsa.GattnError) as ei:
        gsa._check(gsa._lib.gattn_forward_noalloc(None, None), "gattn_forward_noalloc")
    assert ei.value.status == gsa.GATTN_ERR_INVALID_VALUE
    torch.cuda.synchronize()
