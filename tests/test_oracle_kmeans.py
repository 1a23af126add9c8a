"""Pins of the weighted k-means oracle (CPU): a hand-computed example, the reduction to plain k-means
means, Lloyd's monotone objective, weight-scale invariance, empty clusters, separable clusters."""

import numpy as np

from oracle import kmeans as km
from oracle.loopvq import nearest_codeword


def test_hand_example():
    # three points on a line, two codewords at 0 and 10: points 1 and 3 go to e_0, 12 to e_1
    z = np.array([[1.0], [3.0], [12.0]])
    w = np.array([1.0, 3.0, 2.0])
    E = np.array([[0.0], [10.0]])
    new, a = km.lloyd_step(z, w, E)
    assert list(a) == [0, 0, 1]
    assert new[0, 0] == (1 * 1 + 3 * 3) / 4          # 2.5
    assert new[1, 0] == 12.0


def test_equal_weights_give_cluster_means():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(500, 6))
    E = rng.normal(size=(16, 6))
    a, _ = nearest_codeword(z, E)
    new = km.weighted_update(z, np.ones(500), a, E)
    for r in range(16):
        members = z[a == r]
        expect = members.mean(axis=0) if len(members) else E[r]
        np.testing.assert_allclose(new[r], expect, rtol=0, atol=1e-12)


def test_objective_never_rises():
    rng = np.random.default_rng(4)
    z = rng.normal(size=(800, 8)) * rng.uniform(0.5, 2.0, size=8)
    w = rng.lognormal(0.0, 1.0, size=800)
    E = z[rng.choice(800, 32, replace=False)]
    prev = km.objective(z, w, E)
    for _ in range(6):
        E, _ = km.lloyd_step(z, w, E)
        cur = km.objective(z, w, E)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


def test_weight_scale_invariance_and_zero_weights():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(300, 4))
    w = rng.lognormal(size=300)
    E = z[:12].copy()
    a, _ = nearest_codeword(z, E)
    np.testing.assert_allclose(km.weighted_update(z, w, a, E), km.weighted_update(z, 7.5 * w, a, E),
                               rtol=1e-13, atol=1e-13)
    # zero-weight samples do not move their codeword; a cluster of zero total weight keeps its value
    w0 = w.copy()
    w0[a == 3] = 0.0
    new = km.weighted_update(z, w0, a, E)
    np.testing.assert_array_equal(new[3], E[3])


def test_separable_clusters_reach_weighted_means():
    rng = np.random.default_rng(6)
    centers = np.array([[-10.0, 0.0], [0.0, 10.0], [10.0, 0.0]])
    lab = rng.integers(0, 3, size=600)
    z = centers[lab] + rng.normal(scale=0.5, size=(600, 2))
    w = rng.uniform(0.1, 3.0, size=600)
    E0 = centers + rng.normal(scale=2.0, size=(3, 2))
    E = km.weighted_kmeans(z, w, E0, iters=5)
    for r in range(3):
        expect = (w[lab == r, None] * z[lab == r]).sum(axis=0) / w[lab == r].sum()
        np.testing.assert_allclose(E[r], expect, rtol=0, atol=1e-12)
