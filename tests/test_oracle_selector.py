"""Pins of the oracle's IBCS selector (key-block means, k-means, scores).

Each check ties the oracle to something other than itself: a hand-worked
example, scikit-learn's k-means, scipy's softmax, closed forms and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
from sklearn.cluster import KMeans

import oracle
from oracle import Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ln3(x):
    return math.log(3.0) if x == "ln3" else float(x)


def test_ibcs_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "ibcs_worked_example.json")))
    Q = np.array(g["queries"], dtype=np.float64)[None, None]
    K = np.array([[_ln3(x) for x in row] for row in g["keys"]])[None, None]
    prob = Problem(B=1, H=1, N=Q.shape[2], D=g["D"], q_block=4, kv_block=4,
                   n_clusters=g["n_clusters"], kmeans_iters=g["kmeans_iters"],
                   scale=g["scale"])
    # the query block has 4 tokens but the keys have 8: use separate problems
    probk = Problem(B=1, H=1, N=K.shape[2], D=g["D"], q_block=8, kv_block=4,
                    n_clusters=g["n_clusters"], kmeans_iters=g["kmeans_iters"],
                    scale=g["scale"])
    kbar = oracle.key_block_means(K, probk)[0, 0]
    want_kbar = np.array([[_ln3(x) for x in row] for row in g["expected_key_means"]])
    np.testing.assert_allclose(kbar, want_kbar, rtol=0, atol=1e-15)
    mu, w, counts = oracle.query_clusters(Q, prob)
    np.testing.assert_array_equal(mu[0], np.array(g["expected_centroids"]))
    np.testing.assert_array_equal(w[0], np.array(g["expected_weights"]))
    s = oracle.block_scores(mu[0], w[0], kbar, prob.tau)
    np.testing.assert_allclose(s, g["expected_scores"], rtol=1e-15, atol=0)


def test_key_means_invariants():
    rng = np.random.default_rng(3)
    prob = Problem(B=2, H=3, N=64, D=8)
    K = rng.standard_normal((2, 3, 64, 8))
    kbar = oracle.key_block_means(K, prob)
    assert kbar.shape == (2, 3, 16, 8)
    # the block means carry the total of the keys (each block has 4 tokens)
    np.testing.assert_allclose(4.0 * kbar.sum(axis=2), K.sum(axis=2), rtol=1e-12)
    # blocks made of one repeated row average to that row; order inside a
    # block does not matter
    Kc = np.repeat(rng.standard_normal((1, 1, 16, 8)), 4, axis=2)
    np.testing.assert_array_equal(oracle.key_block_means(Kc, Problem(1, 1, 64, 8))[0, 0],
                                  Kc[0, 0, ::4])
    Kp = K.copy()
    Kp[:, :, 0:4] = K[:, :, [3, 1, 0, 2]]
    np.testing.assert_allclose(oracle.key_block_means(Kp, prob), kbar, rtol=1e-15)
    # forced tail tokens are not part of any scored block
    probf = Problem(B=2, H=3, N=64, D=8, n_forced_tail=8)
    assert oracle.key_block_means(K, probf).shape == (2, 3, 14, 8)
    np.testing.assert_array_equal(oracle.key_block_means(K, probf), kbar[:, :, :14])


# seeds whose clustering never empties a cluster (scikit-learn relocates an
# empty cluster; the method keeps its centroid, which the fixed-point and
# edge-case tests below cover)
@pytest.mark.parametrize("seed", range(1, 7))
def test_kmeans_matches_sklearn(seed):
    rng = np.random.default_rng(seed)
    n, d, C, it = 128, 16, 8, 10
    X = rng.standard_normal((n, d)) + 3.0 * rng.standard_normal((8, d))[rng.integers(0, 8, n)]
    mu, counts = oracle.kmeans(X, C, it)
    init = X[[(c * n) // C for c in range(C)]]
    km = KMeans(n_clusters=C, init=init, n_init=1, max_iter=it, tol=0.0,
                algorithm="lloyd").fit(X)
    assert np.all(np.bincount(km.labels_, minlength=C) > 0) and np.all(counts > 0)
    np.testing.assert_allclose(mu, km.cluster_centers_, rtol=1e-10, atol=1e-12)
    assert counts.sum() == n


def test_kmeans_separated_clusters_closed_form():
    # eight tight, far-apart groups laid out so that the evenly spaced init
    # picks one member of each: one step reaches the exact group means.
    rng = np.random.default_rng(7)
    n, d, C = 128, 32, 8
    centers = 50.0 * rng.standard_normal((C, d))
    sizes = [16] * C
    X = np.concatenate([centers[c] + 0.01 * rng.standard_normal((sizes[c], d))
                        for c in range(C)])
    mu, counts = oracle.kmeans(X, C, 10)
    for c in range(C):
        np.testing.assert_allclose(mu[c], X[16 * c:16 * (c + 1)].mean(axis=0), rtol=1e-12)
    np.testing.assert_array_equal(counts, sizes)


def test_kmeans_fixed_point_and_edge_cases():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((40, 5))
    mu, counts = oracle.kmeans(X, 4, 50)
    # converged: one more iteration from the result changes nothing
    dist = ((X[:, None, :] - mu[None]) ** 2).sum(-1)
    a = np.argmin(dist, 1)
    for c in range(4):
        if np.any(a == c):
            np.testing.assert_allclose(mu[c], X[a == c].mean(0), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.bincount(a, minlength=4), counts)
    # fewer points than clusters: duplicates lose ties and stay empty
    Y = rng.standard_normal((3, 5))
    mu, counts = oracle.kmeans(Y, 8, 10)
    assert counts.sum() == 3 and (counts > 0).sum() == 3
    # identical points: everything joins cluster 0 (lowest index on ties)
    Z = np.ones((16, 4))
    mu, counts = oracle.kmeans(Z, 8, 10)
    assert counts[0] == 16 and counts[1:].sum() == 0


def test_block_scores_single_centroid_is_softmax():
    rng = np.random.default_rng(5)
    mu = rng.standard_normal((1, 16))
    kbar = rng.standard_normal((300, 16))
    s = oracle.block_scores(mu, np.array([1.0]), kbar, 0.25)
    np.testing.assert_allclose(s, scipy.special.softmax(0.25 * kbar @ mu[0]), rtol=1e-13)


def test_block_scores_invariants():
    rng = np.random.default_rng(9)
    C, n, d = 8, 500, 32
    mu = 2.0 * rng.standard_normal((C, d))
    w = rng.random(C)
    w /= w.sum()
    kbar = rng.standard_normal((n, d))
    s = oracle.block_scores(mu, w, kbar, 1 / math.sqrt(d))
    assert np.all(s > 0)
    assert abs(s.sum() - 1.0) < 1e-12
    # linear in the weights: each centroid contributes its own softmax
    parts = [scipy.special.softmax(kbar @ mu[c] / math.sqrt(d)) for c in range(C)]
    np.testing.assert_allclose(s, sum(w[c] * parts[c] for c in range(C)), rtol=1e-12)
    # a zero-weight centroid contributes nothing
    w0 = w.copy()
    w0[3] = 0.0
    mu2 = mu.copy()
    mu2[3] = 1e3
    np.testing.assert_allclose(oracle.block_scores(mu2, w0, kbar, 1 / math.sqrt(d)),
                               oracle.block_scores(mu, w0, kbar, 1 / math.sqrt(d)), rtol=1e-13)


def test_ibcs_scores_shapes_and_partial_block():
    rng = np.random.default_rng(2)
    prob = Problem(B=1, H=2, N=300, D=16, n_clusters=4)
    Q = rng.standard_normal((1, 2, 300, 16))
    K = rng.standard_normal((1, 2, 300, 16))
    sc = oracle.ibcs_scores(Q, K, prob)
    assert prob.n_qb == 3 and sc["S"].shape == (6, 75)
    np.testing.assert_allclose(sc["S"].sum(1), 1.0, rtol=1e-12)
    # the last query block has 300-256 = 44 queries
    assert sc["counts"][2].sum() == 44 and sc["counts"][0].sum() == 128
    assert sc["S32"].dtype == np.float32
    np.testing.assert_array_equal(sc["S32"], sc["S"].astype(np.float32))
