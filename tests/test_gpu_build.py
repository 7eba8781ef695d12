"""GPU: CSR and row-window construction, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    import graph_sparse_attention_amd as g
    return g


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_csr(gsa, n, src, dst):
    s = torch.from_numpy(np.ascontiguousarray(src, np.int32)).cuda()
    d = torch.from_numpy(np.ascontiguousarray(dst, np.int32)).cuda()
    rp, ci, pe = gsa.gattn_build_csr(s, d, n)
    return to_np(rp), to_np(ci), to_np(pe)


def assert_csr_equal(gsa, n, src, dst):
    ref = oracle.build_csr(n, src, dst)
    got = gpu_csr(gsa, n, src, dst)
    for name, a, b in zip(("row_ptr", "col_idx", "edge_perm"), got, ref):
        assert np.array_equal(a, b), f"{name} differs"
    return ref


@pytest.fixture(params=["default", "atomic", "radix"])
def csr_path(request, monkeypatch):
    """Which of the two builds runs: the library's own choice by size (the
    counting build below 2^18 edges, the radix build above), or one forced."""
    if request.param != "default":
        monkeypatch.setenv("GATTN_CSR_PATH", request.param)
    return request.param


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_csr_configs(gsa, cfg, csr_path):
    c = case(cfg)
    print(f"csr config {cfg} path {csr_path}", flush=True)
    got = gpu_csr(gsa, c.n, c.wl.src, c.wl.dst)
    for a, b in zip(got, (c.rp, c.ci, c.pe)):
        assert np.array_equal(a, b)


@pytest.mark.slow
def test_csr_config4_shuffled(gsa):
    # the large graph in a random edge order: the radix build's stable passes
    # leave rows in edge-id order, so the row sort runs on 2.45M rows of up
    # to 5000 keys (chunked ranks above 2048)
    c = case(4)
    perm = np.random.default_rng(4).permutation(c.wl.nnz)
    print("csr config 4 shuffled", flush=True)
    assert_csr_equal(gsa, c.n, c.wl.src[perm], c.wl.dst[perm])


@pytest.mark.parametrize("cfg", [2, 3])
def test_csr_shuffled_order(gsa, cfg, csr_path):
    # the same graphs handed over in a random edge order: the radix build's
    # stable pass then leaves rows in edge-id order and the row sort runs
    c = case(cfg)
    perm = np.random.default_rng(cfg).permutation(c.wl.nnz)
    print(f"csr shuffled config {cfg} path {csr_path}", flush=True)
    assert_csr_equal(gsa, c.n, c.wl.src[perm], c.wl.dst[perm])


@pytest.mark.parametrize("order", ["by_source", "shuffled"])
def test_csr_radix_large_tiles(gsa, order):
    # above 2^23 edges the radix passes take 7168-key tiles
    g = np.random.default_rng(11)
    n, m = 1_500_000, 9_000_000
    dst = (g.lognormal(1.5, 1.0, m) * 1000).astype(np.int64) % n
    src = g.integers(0, n, m)
    if order == "by_source":
        o = np.argsort(src, kind="stable")
        src, dst = src[o], dst[o]
    print(f"csr radix large tiles, {order}", flush=True)
    assert_csr_equal(gsa, n, src.astype(np.int32), dst.astype(np.int32))


@pytest.mark.parametrize("n", [1, 255, 256, 65535, 65536, (1 << 18) - 1, 1 << 18, 1 << 24, (1 << 27) - 1])
def test_csr_radix_digit_counts(gsa, n, monkeypatch):
    # node counts at the edges of 1, 2, 3 and 4 radix passes, with 8-bit digits
    # and with the 9-bit digits (512 buckets) that save a pass for 17, 18 and
    # 25-27-bit keys; rows of every length from 0 up, long runs of empty rows,
    # sorted and unsorted sources
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    g = np.random.default_rng(n)
    m = 20000
    dst = (np.minimum(g.zipf(1.5, m) - 1, n - 1).astype(np.int64) * 7919 % n).astype(np.int32)
    src = g.integers(0, n, m).astype(np.int32)
    print(f"csr radix n={n}", flush=True)
    assert_csr_equal(gsa, n, np.sort(src), dst[np.argsort(src, kind="stable")])
    assert_csr_equal(gsa, n, src, dst)


@pytest.mark.slow
def test_csr_config4(gsa, csr_path):
    c = case(4)
    print(f"csr config 4 path {csr_path}", flush=True)
    rp, ci, pe = gsa.gattn_build_csr(c.src, c.dst, c.n)
    assert np.array_equal(to_np(rp), c.rp)
    assert np.array_equal(to_np(ci), c.ci)
    assert np.array_equal(to_np(pe), c.pe)


@pytest.mark.parametrize("seed", range(8))
def test_csr_fuzz(gsa, seed, csr_path):
    n = [1, 2, 17, 64, 100, 1000, 3, 500][seed]
    src, dst = W.random_graph(500 + seed, seed, n, [5, 70, 40, 66, 130, 20, 1, 90][seed], multi=seed % 2 == 1)
    assert_csr_equal(gsa, n, src, dst)


def test_csr_long_rows(gsa, csr_path):
    # one destination above the LDS sort capacity (chunks ranked by binary search),
    # rows of exactly 64 and 65 in-edges, and isolated nodes
    g = np.random.default_rng(3)
    n = 30000
    src = [g.integers(0, n, 20000), g.integers(0, n, 64), g.integers(0, n, 65), g.integers(0, n, 8192)]
    dst = [np.full(20000, 7), np.full(64, 8), np.full(65, 9), np.full(8192, 10)]
    src, dst = np.concatenate(src).astype(np.int32), np.concatenate(dst).astype(np.int32)
    perm = g.permutation(src.shape[0])
    assert_csr_equal(gsa, n, src[perm], dst[perm])


@pytest.mark.parametrize("kind", ["star", "four_hubs", "runs"])
def test_csr_radix_large_peer_groups(gsa, kind, monkeypatch):
    # many lanes of a wave holding one digit at once: every edge into one node,
    # edges spread over four destinations, and destinations in runs of 64
    # (a whole wave's item on one digit), in source order and shuffled
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    g = np.random.default_rng(11)
    n, m = 70000, 100000
    if kind == "star":
        dst = np.full(m, 12345, np.int64)
    elif kind == "four_hubs":
        dst = g.choice(np.array([3, 259, 40000, 69999]), m)
    else:
        dst = np.repeat(g.integers(0, n, m // 64 + 1), 64)[:m]
    src = g.integers(0, n, m)
    src, dst = src.astype(np.int32), dst.astype(np.int32)
    print(f"csr radix peer groups {kind}", flush=True)
    order = np.argsort(src, kind="stable")
    assert_csr_equal(gsa, n, src[order], dst[order])
    assert_csr_equal(gsa, n, src, dst)


@pytest.mark.parametrize("tiles", [1, 15, 16, 17, 32, 33, 48])
def test_csr_radix_lookback_groups(gsa, tiles, monkeypatch):
    # the look-back of the 4096-key tiles works in groups of 16 tiles: tile
    # counts at and around whole groups (a last tile that ends a group, one
    # that opens a new group alone), with a ragged last tile
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    g = np.random.default_rng(100 + tiles)
    n = 50000
    m = tiles * 4096 - (0 if tiles % 2 else 1000)
    src, dst = g.integers(0, n, m).astype(np.int32), g.integers(0, n, m).astype(np.int32)
    print(f"csr radix look-back groups tiles={tiles} m={m}", flush=True)
    assert_csr_equal(gsa, n, src, dst)


def test_csr_radix_many_groups(gsa, monkeypatch):
    # 3M edges: 733 tiles of 4096 keys in 46 look-back groups, more tiles than
    # are resident at once; a power-law-like destination mix, random order
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    g = np.random.default_rng(21)
    n, m = 400000, 3000000
    dst = (np.minimum(g.zipf(1.7, m) - 1, n - 1).astype(np.int64) * 7919 % n).astype(np.int32)
    src = g.integers(0, n, m).astype(np.int32)
    print("csr radix many groups", flush=True)
    assert_csr_equal(gsa, n, src, dst)


@pytest.mark.parametrize("seed", range(12))
def test_csr_radix_random_sizes(gsa, seed, monkeypatch):
    # random node counts (1 to 2^22: one to three passes of 7- to 9-bit
    # digits) and edge counts (1 to 1.5M: one tile to many look-back groups),
    # uniform or skewed destinations, source-sorted or shuffled
    monkeypatch.setenv("GATTN_CSR_PATH", "radix")
    g = np.random.default_rng(1000 + seed)
    n = int(g.integers(1, 1 << int(g.integers(1, 23)) + 1))
    m = int(g.integers(1, 1500000))
    if seed % 3 == 0:
        dst = g.integers(0, n, m)
    else:
        dst = np.minimum(g.zipf(1.3 + 0.2 * (seed % 4), m) - 1, n - 1) * 7919 % n
    src = g.integers(0, n, m)
    if seed % 2 == 0:
        order = np.argsort(src, kind="stable")
        src, dst = src[order], dst[order]
    src, dst = src.astype(np.int32), dst.astype(np.int32)
    print(f"csr radix random n={n} m={m}", flush=True)
    assert_csr_equal(gsa, n, src, dst)


@pytest.mark.parametrize("path,m", [("atomic", 262143), ("radix", 600000)])
def test_csr_giant_unsorted_row(gsa, path, m, monkeypatch):
    # one destination with every edge, sources in random order: the row is
    # sorted as LDS-sorted chunks merged pairwise (128 / 293 chunks), a few
    # other rows around it
    monkeypatch.setenv("GATTN_CSR_PATH", path)
    g = np.random.default_rng(31)
    n = 5000
    src = g.integers(0, n, m).astype(np.int32)
    dst = np.full(m, 4242, np.int32)
    dst[: m // 50] = g.integers(0, n, m // 50)
    perm = g.permutation(m)
    print(f"csr giant unsorted row {path} m={m}", flush=True)
    assert_csr_equal(gsa, n, src[perm], dst[perm])


@pytest.mark.parametrize("n", [16383, 16384, 16385, 40000, 131073, 300000])
def test_csr_atomic_scan_sizes(gsa, n, monkeypatch):
    # the look-back scan of the degree counts (2048 per tile): one count short
    # of 8 full tiles, exactly 8, a 9th tile holding one count, 20 tiles, and
    # 65 / 147 tiles (look-backs over more than the 64 tiles one poll reads)
    monkeypatch.setenv("GATTN_CSR_PATH", "atomic")
    g = np.random.default_rng(n)
    m = 60000
    src = g.integers(0, n, m).astype(np.int32)
    dst = g.integers(0, n, m).astype(np.int32)
    dst[:50] = n - 1
    assert_csr_equal(gsa, n, src, dst)


def test_csr_empty_and_bad(gsa, csr_path):
    for n in (0, 5):
        rp, ci, pe = gpu_csr(gsa, n, np.zeros(0, np.int32), np.zeros(0, np.int32))
        assert rp.tolist() == [0] * (n + 1) and ci.size == 0
    with pytest.raises(gsa.GattnError) as ei:
        gpu_csr(gsa, 5, np.array([0, 5], np.int32), np.array([1, 2], np.int32))
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    # asynchronous form: status written on the device
    b = gsa.CsrBuilder(5, 2, "cuda")
    b(torch.tensor([0, 1], dtype=torch.int32, device="cuda"), torch.tensor([-1, 2], dtype=torch.int32, device="cuda"))
    assert int(b.status.item()) == gsa.GATTN_ERR_BAD_GRAPH
    b(torch.tensor([0, 1], dtype=torch.int32, device="cuda"), torch.tensor([4, 2], dtype=torch.int32, device="cuda"))
    assert int(b.status.item()) == gsa.GATTN_OK
    assert to_np(b.row_ptr).tolist() == [0, 0, 0, 1, 1, 2]


def test_csr_deterministic(gsa):
    c = case(3)
    a = gsa.gattn_build_csr(c.src, c.dst, c.n)
    b = gsa.gattn_build_csr(c.src, c.dst, c.n)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def gpu_rw(gsa, n, rp, ci):
    rw = gsa.gattn_build_rowwindows(torch.from_numpy(np.ascontiguousarray(rp)).cuda(),
                                    torch.from_numpy(np.ascontiguousarray(ci)).cuda(), n)
    return to_np(rw.win_col_ptr), to_np(rw.win_cols), to_np(rw.tile_mask).view(np.uint16)


def assert_rw_equal(gsa, n, rp, ci):
    ref = oracle.rowwindows(n, rp, ci)
    got = gpu_rw(gsa, n, rp, ci)
    for name, a, b in zip(("win_col_ptr", "win_cols", "tile_mask"), got, ref):
        assert np.array_equal(a, b.reshape(a.shape)), f"{name} differs"


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_rowwindows_configs(gsa, cfg):
    c = case(cfg)
    assert_rw_equal(gsa, c.n, c.rp, c.ci)


@pytest.mark.parametrize("seed", range(6))
def test_rowwindows_fuzz(gsa, seed):
    n = [1, 16, 17, 33, 250, 1000][seed]
    src, dst = W.random_graph(600 + seed, seed, n, [3, 16, 30, 40, 25, 12][seed])
    rp, ci, _ = oracle.build_csr(n, src, dst)
    assert_rw_equal(gsa, n, rp, ci)
    # any order inside a row gives the same windows
    g = np.random.default_rng(seed)
    ci2 = ci.copy()
    for i in range(n):
        g.shuffle(ci2[rp[i]:rp[i + 1]])
    ref = oracle.rowwindows(n, rp, ci)
    got = gpu_rw(gsa, n, rp, ci2)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b.reshape(a.shape))


def test_rowwindows_mixed_spans(gsa):
    # windows whose sources span less than 4096 values (bitmap) next to windows
    # spanning the whole graph (sorted keys), spans right at the threshold, and
    # windows whose masks do not fit the LDS assembly (> 2048 columns)
    g = np.random.default_rng(21)
    n = 40000
    srcs, dsts = [], []
    for r in range(0, 16):            # window 0: sources within 4095 of each other
        s = g.choice(4096, 30, replace=False) + 1000
        srcs.append(s); dsts.append(np.full(30, r))
    srcs.append(np.array([5000, 5000 + 4095])); dsts.append(np.array([16, 17]))   # span 4096 -> sorted keys
    srcs.append(np.array([7000, 7000 + 4094])); dsts.append(np.array([32, 33]))   # span 4095 -> bitmap
    for r in range(48, 64):           # window 3: 16 x 200 random sources, > 2048 columns
        s = g.choice(n, 200, replace=False)
        srcs.append(s); dsts.append(np.full(200, r))
    for r in range(64, 80):           # window 4: narrow again
        s = g.choice(100, 12, replace=False) + 30000
        srcs.append(s); dsts.append(np.full(12, r))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    rp, ci, _ = oracle.build_csr(n, src, dst)
    assert_rw_equal(gsa, n, rp, ci)


def test_rowwindows_long_window(gsa):
    # a window with more than 8192 edges takes the chunked workspace sort
    n = 20000
    g = np.random.default_rng(9)
    srcs, dsts = [], []
    for r in range(16, 32):
        s = g.choice(n, 700, replace=False)
        srcs.append(s)
        dsts.append(np.full(700, r))
    srcs.append(g.choice(n, 50, replace=False))
    dsts.append(np.full(50, 40))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    rp, ci, _ = oracle.build_csr(n, src, dst)
    assert_rw_equal(gsa, n, rp, ci)


def test_rowwindows_giant_window(gsa):
    # 16 rows x 5000 edges in one window: 40 sorted chunks merged over six
    # levels, with sources shared between rows (duplicates across rows) and
    # each row's sources in random order
    n = 200000
    g = np.random.default_rng(21)
    pool = g.choice(n, 30000, replace=False)
    srcs, dsts = [], []
    for r in range(32, 48):
        srcs.append(g.choice(pool, 5000, replace=False))
        dsts.append(np.full(5000, r))
    srcs.append(g.choice(n, 300, replace=False))
    dsts.append(np.full(300, 5))
    src, dst = np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)
    rp, ci, _ = oracle.build_csr(n, src, dst)
    ci2 = ci.copy()
    for i in range(32, 48):
        g.shuffle(ci2[rp[i]:rp[i + 1]])
    ref = oracle.rowwindows(n, rp, ci)
    got = gpu_rw(gsa, n, rp, ci2)
    for name, a, b in zip(("win_col_ptr", "win_cols", "tile_mask"), got, ref):
        assert np.array_equal(a, b.reshape(a.shape)), f"{name} differs"


@pytest.mark.parametrize("n", [16 * 16384 - 1, 16 * 16384, 16 * 16384 + 1])
def test_rowwindows_scan_sizes(gsa, n):
    # 16384 windows (8 full look-back scan tiles of window sizes, the last
    # window full or one row short) and 16385 (a 9th tile with one window)
    g = np.random.default_rng(n)
    m = 50000
    src = g.integers(0, n, m).astype(np.int32)
    dst = g.integers(0, n, m).astype(np.int32)
    dst[:20] = n - 1
    rp, ci, _ = oracle.build_csr(n, src, dst)
    assert_rw_equal(gsa, n, rp, ci)


@pytest.mark.parametrize("n", [40, 50000])
def test_rowwindows_errors(gsa, n):
    # n = 40: every window's sources span < 4096 values (bitmap path); n = 50000:
    # random sources span more (sorted-key path) -- both must find the repeat
    src, dst = W.random_graph(700, 0, 40, 10)
    if n > 40:
        src = (src.astype(np.int64) * 1237 % n).astype(np.int32)
    src, dst = np.append(src, src[0]).astype(np.int32), np.append(dst, dst[0]).astype(np.int32)
    rp, ci, _ = oracle.build_csr(n, src, dst)
    with pytest.raises(gsa.GattnError) as ei:
        gpu_rw(gsa, n, rp, ci)
    assert ei.value.status == gsa.GATTN_ERR_DUPLICATE_EDGE
    ci_bad = ci.copy()
    ci_bad[3] = n
    with pytest.raises(gsa.GattnError) as ei:
        gpu_rw(gsa, n, rp, ci_bad)
    assert ei.value.status == gsa.GATTN_ERR_BAD_GRAPH
    # empty graph
    rp0 = np.zeros(n + 1, np.int32)
    wcp, cols, mask = gpu_rw(gsa, n, rp0, np.zeros(0, np.int32))
    assert np.all(wcp == 0) and cols.size == 0
