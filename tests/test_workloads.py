"""Seeded generators: reproducible, and their graphs have the stated laws."""
import numpy as np

import workloads as W


def test_reproducible():
    a, b = W.make(1), W.make(1)
    assert np.array_equal(a.src, b.src) and np.array_equal(a.dst, b.dst)
    assert np.array_equal(a.q(), b.q())
    c = W.make(1, seed=1)
    assert not np.array_equal(a.src, c.src)


def test_config_structure():
    w1 = W.make(1)
    deg = np.bincount(w1.dst, minlength=w1.num_nodes)
    assert w1.num_nodes == 320 and abs(deg.mean() - 14) < 1.0
    w2 = W.make(2)
    deg = np.bincount(w2.dst, minlength=w2.num_nodes)
    assert np.all(deg == 10) and not np.any(w2.src == w2.dst)
    assert 64 * 100 <= w2.num_nodes <= 64 * 300
    assert w2.e().shape == (w2.nnz, 8, 16)
    w5 = W.make(5)
    assert 1024 * 20 <= w5.num_nodes <= 1024 * 40
    deg = np.bincount(w5.dst, minlength=w5.num_nodes)
    assert deg.min() >= 20 and deg.max() <= 40 and w5.nnz == int((deg ** 1).dot(np.ones_like(deg)))
    for w in (w1, w2, w5):
        key = w.src.astype(np.int64) * w.num_nodes + w.dst
        assert np.all(np.diff(key) > 0)          # source-grouped, no repeated pair


def test_powerlaw_laws_small():
    w3 = W.gen_config3(n=20000)
    deg = np.bincount(w3.dst, minlength=w3.num_nodes)
    assert deg.min() >= 1 and deg.max() <= 2000 and not np.any(w3.src == w3.dst)
    assert 3.0 < deg.mean() < 4.6                 # truncated Zipf(2.1) mean is about 3.8
    w4 = W.gen_config4(n=20000)
    deg = np.bincount(w4.dst, minlength=w4.num_nodes)
    assert deg.min() >= 1 and deg.max() <= 5000
    assert 36 < deg.mean() < 47                   # rint(lognormal(3, 1.2)) mean is about 41
    for w in (w3, w4):
        key = w.src.astype(np.int64) * w.num_nodes + w.dst
        assert np.all(np.diff(key) > 0)
