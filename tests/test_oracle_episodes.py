"""Pins of the oracle's episode clustering, medoids and matching (EpiCache
review, "방법: 3단계" (1) and (3), Fig. 3(a) and (c)): Lloyd's K-means from
given centroids, the medoid of each episode, and the nearest episode of a
query."""
import numpy as np
import pytest
from scipy.spatial.distance import cdist
from sklearn.cluster import KMeans

from oracle import oracle as O


def blobs(rng, n, d, e, spread=0.3):
    centers = rng.standard_normal((e, d)) * 3
    lab = rng.integers(0, e, size=n)
    return centers[lab] + spread * rng.standard_normal((n, d)), lab


def test_nearest_centroid_is_cdist_argmin():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((200, 7))
    c = rng.standard_normal((5, 7))
    assert np.array_equal(O.nearest_centroid(x, c), np.argmin(cdist(x, c, "sqeuclidean"), 1))
    # an exact tie goes to the lower centroid
    c2 = np.array([[1.0, 0.0], [-1.0, 0.0]])
    assert O.nearest_centroid(np.array([[0.0, 5.0]]), c2).tolist() == [0]


@pytest.mark.parametrize("seed", range(4))
def test_kmeans_matches_sklearn_lloyd(seed):
    rng = np.random.default_rng(seed)
    x, _ = blobs(rng, 300, 6, 4, spread=1.0)
    init = x[rng.choice(300, 4, replace=False)]
    rounds = 8
    c, a = O.kmeans(x, init, rounds)
    km = KMeans(4, init=init, n_init=1, max_iter=rounds, tol=0.0, algorithm="lloyd").fit(x)
    # sklearn stops early once assignments no longer change; Lloyd's fixed
    # point is unaffected by further rounds
    assert np.allclose(c, km.cluster_centers_, rtol=0, atol=1e-10)
    assert np.array_equal(a, km.labels_)


def test_kmeans_fixed_point_properties():
    rng = np.random.default_rng(5)
    x, lab = blobs(rng, 400, 16, 4, spread=0.2)
    init = np.stack([x[lab == e][0] for e in range(4)])
    c, a = O.kmeans(x, init, 10)
    assert np.array_equal(a, lab)                    # well separated: the true labels
    for e in range(4):
        assert np.allclose(c[e], x[a == e].mean(0), atol=1e-12)
    assert np.array_equal(a, O.nearest_centroid(x, c))


def test_kmeans_empty_cluster_keeps_its_centroid():
    x = np.array([[0.0], [0.1], [10.0], [10.2]])
    init = np.array([[0.0], [10.0], [1000.0]])
    c, a = O.kmeans(x, init, 3)
    assert c[2, 0] == 1000.0 and a.tolist() == [0, 0, 1, 1]
    assert c[0, 0] == pytest.approx(0.05) and c[1, 0] == pytest.approx(10.1)


def test_kmeans_zero_rounds_is_plain_assignment():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 3))
    init = rng.standard_normal((3, 3))
    c, a = O.kmeans(x, init, 0)
    assert np.array_equal(c, init) and np.array_equal(a, O.nearest_centroid(x, init))


def test_medoid_by_brute_force_and_one_dimension():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((60, 5))
    a = rng.integers(0, 3, size=60)
    got = O.medoids(x, a, 4)
    assert got[3] == -1                              # empty cluster
    for e in range(3):
        idx = np.nonzero(a == e)[0]
        tot = cdist(x[idx], x[idx]).sum(1)
        assert got[e] == idx[np.argmin(tot)]
        assert np.allclose(O.medoid_totals(x, a)[idx], tot, rtol=0, atol=1e-12)
    # on a line with an odd count the medoid is the median point
    line = np.array([[5.0], [1.0], [9.0], [2.0], [100.0]])
    assert O.medoids(line, np.zeros(5, int), 1).tolist() == [0]     # the median, 5.0


def test_medoid_ties_go_to_the_lower_index():
    x = np.array([[0.0], [1.0], [2.0], [3.0]])       # points 1 and 2 tie
    assert O.medoids(x, np.zeros(4, int), 1).tolist() == [1]
