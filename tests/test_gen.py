"""The seeded input generator: determinism, independence of streams, distributions."""
import numpy as np
from scipy import stats

import gen


def test_deterministic_and_offset_consistent():
    a = gen.normal(7, 3, 1000)
    assert np.array_equal(a, gen.normal(7, 3, 1000))
    assert np.array_equal(a[100:200], gen.normal(7, 3, 100, start=100))
    assert not np.array_equal(a, gen.normal(7, 4, 1000))
    assert not np.array_equal(a, gen.normal(8, 3, 1000))


def test_normal_distribution():
    x = gen.normal(1, 1, 200000).astype(np.float64)
    assert stats.kstest(x, "norm").pvalue > 1e-3
    w = gen.normal(1, 2, 200000, scale=0.02).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4


def test_student_t_distribution():
    x = gen.student_t(1, 5, 100000, nu=4).astype(np.float64)
    assert stats.kstest(x, stats.t(df=4).cdf).pvalue > 1e-3


def test_uniform_open_interval():
    u = gen.uniform(2, 9, 100000)
    assert u.min() > 0 and u.max() < 1
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_routing_shapes_and_weights():
    ids, w = gen.route_uniform(3, 50, 32, 8)
    assert ids.shape == (50, 8) and w.shape == (50, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(1), 1, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # softmax of scores sorted descending


def test_zipf_routing_skew_and_zero_experts():
    cfg = gen.CONFIGS["c2"]
    ids, w = gen.routing(cfg)
    cnt = np.bincount(ids.ravel(), minlength=cfg.E)
    assert (cnt == 0).sum() == cfg.zipf_zero          # "several experts receive 0 tokens"
    assert (cnt > 1000).sum() >= 3                     # "a few receive more than 1000"
    assert all(len(set(r)) == cfg.k for r in ids[:200].tolist())
