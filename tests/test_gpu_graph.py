"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every call of the library is stream-ordered and allocation-free given its
buffers, so a CSR build (both algorithms: the counting build below 2^18
edges, the radix build above) followed by a forward (gather path with either
partition, or the MFMA row-window path) can be captured once and replayed.
Each replay runs after eager work that overwrites the outputs and after a
synchronization, and must reproduce the eager result bit for bit (the
kernels are deterministic); the device status must read OK.
"""
import pytest
import torch

from parity import case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


@pytest.mark.parametrize("cfg,path,ws,kvi", [(2, "gather", None, False), (2, "gather", True, False),
                                             (3, "gather", None, False), (3, "gather", True, False),
                                             (5, "mfma", None, False), (3, "gather", True, True),
                                             (5, "mfma", None, True)],
                         ids=["cfg2-node", "cfg2-balanced", "cfg3-node", "cfg3-balanced", "cfg5-mfma",
                              "cfg3-balanced-kv-interleaved", "cfg5-mfma-kv-interleaved"])
def test_graph_replays_match_eager(gsa, cfg, path, ws, kvi):
    c = case(cfg)
    wl = c.wl
    print(f"graph capture config {cfg} path {path} workspace {ws} kv interleaved {kvi}", flush=True)
    k, v = c.k, c.v
    if kvi:  # K and V as the halves of one [N, 2, H, D] buffer: strided row views
        kv = torch.stack((c.k, c.v), dim=1)
        k, v = kv[:, 0], kv[:, 1]
    b = gsa.CsrBuilder(c.n, wl.nnz, c.src.device)
    rw = None
    if path == "mfma":  # row windows once per graph, outside the graph (they synchronize)
        b(c.src, c.dst)
        torch.cuda.synchronize()
        rw = gsa.gattn_build_rowwindows(b.row_ptr, b.col_idx, c.n)

    def step():
        b(c.src, c.dst)
        return gsa.gattn_forward(b.row_ptr, b.col_idx, c.q, k, v, c.e, mode=wl.mode, scale=wl.scale,
                                 clip=wl.clip, eps=wl.eps, path=path, rw=rw, workspace=ws)

    ref = step().clone()
    torch.cuda.synchronize()
    ref_csr = [t.clone() for t in (b.row_ptr, b.col_idx, b.edge_perm)]
    assert int(b.status.item()) == gsa.GATTN_OK

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for i in range(3):
        for t in (b.row_ptr, b.col_idx, b.edge_perm):
            t.fill_(-7)
        out.fill_(float("nan"))
        b.status.fill_(-1)
        eager = step()  # eager work of the program between replays
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)
        for t in (b.row_ptr, b.col_idx, b.edge_perm):
            t.fill_(-7)
        b.status.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(b.status.item()) == gsa.GATTN_OK, f"replay {i}: device status"
        for name, got, want in zip(("row_ptr", "col_idx", "edge_perm"), (b.row_ptr, b.col_idx, b.edge_perm), ref_csr):
            assert torch.equal(got, want), f"replay {i}: {name} differs"
        assert torch.equal(out, ref), f"replay {i}: forward output differs"


@pytest.mark.parametrize("mode", ["standard", "clipped"])
def test_graph_replays_with_new_inputs_balanced(gsa, mode):
    # The balanced partition cuts config 3's hub rows (up to 2000 in-edges)
    # across workgroups and merges their parts through the workspace.  One
    # workspace serves the captured launch, whose token the graph keeps;
    # q, k, v change before every replay, eager launches on the same
    # workspace run in between, and each replay must equal an eager launch on
    # the same inputs with a workspace of its own.
    c = case(3)
    wl = c.wl
    print(f"graph replay with new inputs, config 3 balanced, {mode}", flush=True)
    rp, ci = torch.from_numpy(c.rp).cuda(), torch.from_numpy(c.ci).cuda()
    deg = torch.diff(rp)
    q, k, v = c.q.clone(), c.k.clone(), c.v.clone()
    ws = torch.empty(gsa.gattn_forward_workspace(rp, ci, q, k, v, mode=mode), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                       # arbitrary contents on entry

    def step(workspace, out=None):
        return gsa.gattn_forward(rp, ci, q, k, v, mode=mode, scale=wl.scale, path="gather", workspace=workspace,
                                 out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(ws)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    hubs = torch.nonzero(deg > 500).flatten()
    assert hubs.numel() > 0
    for i in range(4):
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        want = step(True)
        if i % 2:
            step(ws)                     # eager work on the captured launch's workspace
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[hubs], want[hubs]), f"replay {i}: hub rows differ from the eager launch"
        assert torch.equal(out, want), f"replay {i}: output differs from the eager launch"
