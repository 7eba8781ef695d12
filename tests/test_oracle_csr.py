"""Pins of the oracle's CSR and row-window builders (CPU only).

CSR: the canonical order (destination, source, edge id) is exactly what
``np.lexsort`` returns and the pointer vector is a bincount prefix sum.
Row windows: decoding every (window, tile, row, bit) must give back the CSR
edge set; distinct counts match ``np.unique``; padding is -1 with no bits.
"""
import numpy as np
import pytest

import workloads as W


def lexsort_csr(n, src, dst):
    eid = np.arange(src.shape[0])
    order = np.lexsort((eid, src, dst))
    row_ptr = np.zeros(n + 1, np.int64)
    row_ptr[1:] = np.cumsum(np.bincount(dst, minlength=n))
    return row_ptr, src[order], order


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("multi", [False, True])
def test_csr_matches_lexsort(orc, seed, multi):
    n = [1, 7, 16, 33, 100, 257][seed]
    src, dst = W.random_graph(100 + seed, seed, n, 12, multi=multi)
    rp, ci, pe = orc.build_csr(n, src, dst)
    rp2, ci2, pe2 = lexsort_csr(n, src.astype(np.int64), dst.astype(np.int64))
    assert np.array_equal(rp, rp2)
    assert np.array_equal(ci, ci2)
    assert np.array_equal(pe, pe2)
    # edge_perm is a permutation and maps positions back to the COO edges
    assert np.array_equal(np.sort(pe), np.arange(src.shape[0]))
    assert np.array_equal(src[pe], ci)
    for i in range(n):
        assert np.all(dst[pe[rp[i]:rp[i + 1]]] == i)


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_csr_configs(orc, cfg):
    wl = W.make(cfg)
    rp, ci, pe = orc.build_csr(wl.num_nodes, wl.src, wl.dst)
    rp2, ci2, pe2 = lexsort_csr(wl.num_nodes, wl.src.astype(np.int64), wl.dst.astype(np.int64))
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2) and np.array_equal(pe, pe2)


def test_csr_empty_and_errors(orc):
    rp, ci, pe = orc.build_csr(0, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert rp.tolist() == [0] and ci.size == 0
    rp, ci, pe = orc.build_csr(5, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert rp.tolist() == [0] * 6
    for s, d in [([5], [0]), ([0], [5]), ([-1], [0]), ([0], [-2])]:
        with pytest.raises(orc.OracleError) as ei:
            orc.build_csr(5, np.array(s, np.int32), np.array(d, np.int32))
        assert ei.value.code == orc.ORC_BAD_GRAPH


def decode_windows(n, wcp, cols, mask):
    edges = set()
    W_ = (n + 15) // 16
    for w in range(W_):
        base, end = int(wcp[w]), int(wcp[w + 1])
        assert base % 16 == 0 and end % 16 == 0
        for t in range((end - base) // 16):
            tile = base // 16 + t
            for r in range(16):
                bits = int(mask[tile, r])
                if 16 * w + r >= n:
                    assert bits == 0
                for c in range(16):
                    if bits >> c & 1:
                        col = int(cols[base + 16 * t + c])
                        assert col >= 0
                        edges.add((16 * w + r, col))
    return edges


@pytest.mark.parametrize("seed", range(5))
def test_rowwindows_roundtrip(orc, seed):
    n = [5, 16, 31, 64, 200][seed]
    src, dst = W.random_graph(200 + seed, seed, n, 20)
    rp, ci, _ = orc.build_csr(n, src, dst)
    wcp, cols, mask = orc.rowwindows(n, rp, ci)
    csr_edges = {(i, int(ci[p])) for i in range(n) for p in range(rp[i], rp[i + 1])}
    assert decode_windows(n, wcp, cols, mask) == csr_edges
    assert sum(bin(int(x)).count("1") for x in mask.reshape(-1)) == ci.shape[0]
    for w in range((n + 15) // 16):
        r0, r1 = 16 * w, min(16 * w + 16, n)
        u = np.unique(ci[rp[r0]:rp[r1]])
        seg = cols[wcp[w]:wcp[w + 1]]
        assert seg.shape[0] == 16 * ((u.shape[0] + 15) // 16)
        assert np.array_equal(seg[:u.shape[0]], u)
        assert np.all(seg[u.shape[0]:] == -1)
        pad_tiles = mask[wcp[w] // 16:wcp[w + 1] // 16]
        # padding columns carry no bits
        for t in range(pad_tiles.shape[0]):
            for c in range(16):
                if seg[16 * t + c] == -1:
                    assert not any(int(pad_tiles[t, r]) >> c & 1 for r in range(16))


def test_rowwindows_order_free_and_duplicates(orc):
    n = 40
    src, dst = W.random_graph(300, 0, n, 15)
    rp, ci, _ = orc.build_csr(n, src, dst)
    ref = orc.rowwindows(n, rp, ci)
    # any within-row order gives the same windows (they are defined by sets)
    g = np.random.default_rng(0)
    ci2 = ci.copy()
    for i in range(n):
        g.shuffle(ci2[rp[i]:rp[i + 1]])
    got = orc.rowwindows(n, rp, ci2)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    # a repeated (dst, src) pair cannot live in a bit mask
    src_m, dst_m = np.append(src, src[0]), np.append(dst, dst[0])
    rp3, ci3, _ = orc.build_csr(n, src_m, dst_m)
    with pytest.raises(orc.OracleError) as ei:
        orc.rowwindows(n, rp3, ci3)
    assert ei.value.code == orc.ORC_DUPLICATE


def test_rowwindows_config5_density(orc):
    wl = W.make(5)
    rp, ci, _ = orc.build_csr(wl.num_nodes, wl.src, wl.dst)
    wcp, cols, mask = orc.rowwindows(wl.num_nodes, rp, ci)
    tiles = wcp[-1] // 16
    density = ci.shape[0] / (256.0 * tiles)
    assert 0.4 < density < 0.8
    assert sum(bin(int(x)).count("1") for x in mask.reshape(-1)) == ci.shape[0]
