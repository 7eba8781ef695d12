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


@pytest.mark.parametrize("cfg,path,ws", [(2, "gather", None), (2, "gather", True), (3, "gather", None),
                                         (3, "gather", True), (5, "mfma", None)],
                         ids=["cfg2-node", "cfg2-balanced", "cfg3-node", "cfg3-balanced", "cfg5-mfma"])
def test_graph_replays_match_eager(gsa, cfg, path, ws):
    c = case(cfg)
    wl = c.wl
    print(f"graph capture config {cfg} path {path} workspace {ws}", flush=True)
    b = gsa.CsrBuilder(c.n, wl.nnz, c.src.device)
    rw = None
    if path == "mfma":  # row windows once per graph, outside the graph (they synchronize)
        b(c.src, c.dst)
        torch.cuda.synchronize()
        rw = gsa.gattn_build_rowwindows(b.row_ptr, b.col_idx, c.n)

    def step():
        b(c.src, c.dst)
        return gsa.gattn_forward(b.row_ptr, b.col_idx, c.q, c.k, c.v, c.e, mode=wl.mode, scale=wl.scale,
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
