"""Pins of the oracle's layer sensitivity (EpiCache review, "+α: 레이어별 예산
배분" and Fig. 4(a): per-layer similarity of the keys computed under block
prefill to the full-prefill keys; sensitivity = 1 - similarity)."""
import numpy as np
import pytest
from scipy.spatial import distance

from oracle import oracle as O


def test_identical_and_scaled_keys_have_similarity_one():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((3, 2, 50, 16))
    assert np.allclose(O.key_similarity(k, k), 1.0, rtol=0, atol=1e-15)
    scale = rng.uniform(0.1, 10.0, size=(3, 2, 50, 1))
    assert np.allclose(O.key_similarity(k, k * scale), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(O.sensitivity(O.key_similarity(k, k)), 0.0, atol=1e-15)


def test_opposite_and_orthogonal_keys():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 1, 30, 8))
    assert np.allclose(O.key_similarity(k, -k), -1.0, atol=1e-15)
    # rows built orthogonal by Gram-Schmidt against each key row
    r = rng.standard_normal(k.shape)
    orth = r - np.sum(r * k, -1, keepdims=True) / np.sum(k * k, -1, keepdims=True) * k
    assert np.allclose(O.key_similarity(k, orth), 0.0, atol=1e-14)
    assert np.allclose(O.sensitivity(O.key_similarity(k, -k)), 2.0)


def test_matches_scipy_cosine_distance_by_brute_force():
    rng = np.random.default_rng(2)
    L, H, N, d = 3, 2, 7, 5
    a = rng.standard_normal((L, H, N, d))
    b = a + 0.7 * rng.standard_normal((L, H, N, d)) * np.arange(1, L + 1)[:, None, None, None]
    want = [np.mean([1.0 - distance.cosine(a[l, h, i], b[l, h, i])
                     for h in range(H) for i in range(N)]) for l in range(L)]
    assert np.allclose(O.key_similarity(a, b), want, rtol=0, atol=1e-14)
    # the mean is taken per layer and symmetric in its arguments
    assert np.allclose(O.key_similarity(b, a), want, rtol=0, atol=1e-14)


def test_zero_rows_count_as_cosine_zero():
    a = np.ones((1, 1, 4, 3))
    b = np.ones((1, 1, 4, 3))
    b[0, 0, 1] = 0.0
    assert O.key_similarity(a, b)[0] == pytest.approx(0.75, abs=1e-15)


def test_more_perturbed_layers_are_more_sensitive():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((4, 2, 200, 32))
    noise = rng.standard_normal(k.shape)
    sig = np.array([0.05, 0.2, 0.5, 1.0])
    kb = k + sig[:, None, None, None] * noise
    s = O.sensitivity(O.key_similarity(k, kb))
    assert np.all(np.diff(s) > 0) and np.all(s > 0)
    # the budget split then gives the more sensitive layers more positions
    kl = O.layer_budgets(4000, 4, s, 2.0)
    assert np.all(np.diff(kl) > 0) and kl.sum() == 4000
