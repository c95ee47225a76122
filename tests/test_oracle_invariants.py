"""Properties the scores, selection and budgets must satisfy at any size.

Each test states a fact that follows from the definitions on the pages (or
from mathematics) without re-deriving the oracle's own formulas:
probabilities sum to one, scores lie in [0, 1], the order of the queries does
not matter, a constant key offset cancels in the softmax, duplicate queries or
heads change nothing, extra queries never lower a max, chunks are scored only
by their own queries, and the one-chunk case is the plain column max.
"""
import math

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

from oracle import oracle as O


def problem(seed, G=2, Hkv=2, L=1, d=8, S=2, chunk=5, nq=3, extra=3, scale=2.0):
    rng = np.random.default_rng(seed)
    N = S + 2 * chunk + extra
    R = len(O.chunk_bounds(N, S, chunk))
    q = rng.normal(size=(L, Hkv * G, R * nq, d)) * scale
    k = rng.normal(size=(L, Hkv, N, d)) * scale
    return q, k, dict(n_sinks=S, chunk_size=chunk, q_per_chunk=nq)


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 10_000), st.floats(0.1, 6.0))
def test_rows_sum_to_one(seed, scale):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(5, 16)) * scale
    k = rng.normal(size=(40, 16)) * scale
    p = O.attention_probs(q, k)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 10_000))
def test_scores_in_unit_interval_and_sinks_one(seed):
    q, k, kw = problem(seed)
    s = O.scores(q, k, **kw)
    assert np.all(s >= 0) and np.all(s <= 1)
    assert np.all(s[..., : kw["n_sinks"]] == 1.0)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 10_000))
def test_query_order_within_a_chunk_does_not_matter(seed):
    q, k, kw = problem(seed)
    rng = np.random.default_rng(seed + 1)
    nq = kw["q_per_chunk"]
    q2 = q.copy()
    for r in range(q.shape[2] // nq):
        perm = rng.permutation(nq) + r * nq
        q2[:, :, r * nq:(r + 1) * nq] = q[:, :, perm]
    np.testing.assert_allclose(O.scores(q2, k, **kw), O.scores(q, k, **kw), rtol=1e-14, atol=0)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 10_000))
def test_constant_key_offset_cancels(seed):
    q, k, kw = problem(seed)
    b = np.random.default_rng(seed + 2).normal(size=k.shape[-1]) * 8.0
    np.testing.assert_allclose(O.scores(q, k + b, **kw), O.scores(q, k, **kw), rtol=1e-11, atol=1e-300)


def test_duplicate_query_and_duplicate_head_change_nothing():
    q, k, kw = problem(7, G=2, Hkv=1)
    base = O.scores(q, k, **kw)
    nq = kw["q_per_chunk"]
    # one more query per chunk, equal to that chunk's first query
    R = q.shape[2] // nq
    rows = []
    for r in range(R):
        blk = q[:, :, r * nq:(r + 1) * nq]
        rows.append(np.concatenate([blk, blk[:, :, :1]], axis=2))
    q_more = np.concatenate(rows, axis=2)
    kw2 = dict(kw, q_per_chunk=nq + 1)
    np.testing.assert_allclose(O.scores(q_more, k, **kw2), base, rtol=1e-14, atol=0)
    # a third head equal to head 0 of the group (G: 2 -> 3)
    q_head = np.concatenate([q, q[:, :1]], axis=1)
    np.testing.assert_allclose(O.scores(q_head, k, **kw), base, rtol=1e-14, atol=0)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 10_000))
def test_more_queries_never_lower_a_score(seed):
    q, k, kw = problem(seed)
    nq = kw["q_per_chunk"]
    R = q.shape[2] // nq
    extra = np.random.default_rng(seed + 3).normal(size=q.shape[:2] + (R, q.shape[3])) * 2
    rows = []
    for r in range(R):
        rows.append(np.concatenate([q[:, :, r * nq:(r + 1) * nq], extra[:, :, r:r + 1]], axis=2))
    q_more = np.concatenate(rows, axis=2)
    base = O.scores(q, k, **kw)
    more = O.scores(q_more, k, **dict(kw, q_per_chunk=nq + 1))
    assert np.all(more >= base)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 10_000))
def test_chunk_locality(seed):
    q, k, kw = problem(seed)
    nq = kw["q_per_chunk"]
    bounds = O.chunk_bounds(k.shape[2], kw["n_sinks"], kw["chunk_size"])
    base = O.scores(q, k, **kw)
    q2 = q.copy()
    q2[:, :, nq:2 * nq] += 3.0                      # disturb chunk 1's queries only
    moved = O.scores(q2, k, **kw)
    for r, (a, b) in enumerate(bounds):
        if r != 1:
            assert np.array_equal(moved[..., a:b], base[..., a:b])


def test_single_chunk_is_plain_column_max_and_single_query_is_scipy_softmax():
    rng = np.random.default_rng(5)
    d, N, S = 8, 19, 3
    k = rng.normal(size=(N, d)) * 2
    q = rng.normal(size=(1, 1, d)) * 2
    s = O.unit_scores(q, k, S, chunk_size=N, q_per_chunk=1)
    ref = scipy.special.softmax(q[0, 0] @ k.T / math.sqrt(d))
    np.testing.assert_allclose(s[S:], ref[S:], rtol=1e-13)
    # several heads and queries, one chunk: max over all rows of the probabilities
    q = rng.normal(size=(3, 4, d)) * 2
    s = O.unit_scores(q, k, S, chunk_size=N, q_per_chunk=4)
    allp = np.concatenate([scipy.special.softmax(q[h] @ k.T / math.sqrt(d), axis=1) for h in range(3)])
    np.testing.assert_allclose(s[S:], allp.max(axis=0)[S:], rtol=1e-13)


# --- selection properties -----------------------------------------------------

@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10_000), st.integers(1, 300), st.integers(0, 6))
def test_select_count_sinks_order_validity(seed, n, S):
    rng = np.random.default_rng(seed)
    S = min(S, n)
    k = int(rng.integers(S, n + 1))
    s = rng.integers(0, 5, size=n) / 4.0
    s[:S] = 1.0
    kept = O.select_unit(s, k, S)
    assert len(kept) == k
    assert kept[:S].tolist() == list(range(S))
    assert np.all(np.diff(kept) > 0)
    inside = np.zeros(n, bool)
    inside[kept] = True
    ins = [i for i in range(S, n) if inside[i]]
    outs = [i for i in range(S, n) if not inside[i]]
    if ins and outs:
        worst_in = min(ins, key=lambda i: (s[i], -i))
        best_out = max(outs, key=lambda i: (s[i], -i))
        assert (s[worst_in] > s[best_out]) or (s[worst_in] == s[best_out] and worst_in < best_out)


def test_select_rejects_budget_outside_range():
    s = np.array([1.0, 0.3, 0.2])
    with pytest.raises(O.BudgetError):
        O.select_unit(s, 0, 1)
    with pytest.raises(O.BudgetError):
        O.select_unit(s, 4, 1)


# --- budget properties --------------------------------------------------------

@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10_000), st.integers(1, 40), st.integers(0, 100_000), st.floats(0, 6))
def test_budget_sum_and_rounding(seed, L, T, alpha):
    s = np.random.default_rng(seed).uniform(0.5, 1.5, size=L)
    k = O.layer_budgets(T, L, s, alpha)
    assert int(k.sum()) == T
    w = s ** alpha
    t = T * w / w.sum()
    assert np.all(np.abs(k - t) < 1.0 + 1e-9)
    order = np.argsort(s, kind="stable")
    # non-decreasing in s, up to the one-unit rounding
    assert np.all(np.diff(k[order]) >= -1)


@pytest.mark.parametrize("L,T", [(1, 5), (3, 10), (28, 229376), (7, 3)])
def test_budget_uniform_when_flat(L, T):
    a = O.layer_budgets(T, L, None, 0.0)
    b = O.layer_budgets(T, L, np.full(L, 0.7), 3.0)
    c = O.layer_budgets(T, L, np.random.default_rng(0).uniform(0.5, 1.5, L), 0.0)
    for k in (a, b, c):
        assert k.max() - k.min() <= 1 and int(k.sum()) == T
        assert list(k) == sorted(k, reverse=True)   # leftovers to the lower layers


def test_budget_errors():
    with pytest.raises(O.BudgetError):
        O.layer_budgets(10, 2, [1.0, -1.0], 1.0)
    with pytest.raises(O.BudgetError):
        O.layer_budgets(10, 2, [1.0, float("nan")], 1.0)
    with pytest.raises(O.BudgetError):
        O.layer_budgets(10, 2, [1.0, 2.0], -1.0)
    with pytest.raises(O.BudgetError):
        O.layer_budgets(10, 2, None, 0.0, n_cache=4, n_sinks=0)    # 5 > N
    with pytest.raises(O.BudgetError):
        O.layer_budgets(4, 2, None, 0.0, n_cache=100, n_sinks=4)   # 2 < S


# --- compaction -------------------------------------------------------------------

def test_compact_copies_the_listed_rows():
    rng = np.random.default_rng(0)
    L, Hkv, N, d = 2, 3, 11, 4
    k = rng.normal(size=(L, Hkv, N, d))
    v = rng.normal(size=(L, Hkv, N, d))
    kept = [np.array([[0, 2, 5], [0, 1, 10], [0, 7, 8]]), np.array([[0, 1], [0, 3], [0, 4]])]
    out = O.compact(k, v, kept)
    for l in range(L):
        for g in range(Hkv):
            for t, i in enumerate(kept[l][g]):
                for c in range(d):
                    assert out[l][0][g, t, c] == k[l, g, i, c]
                    assert out[l][1][g, t, c] == v[l, g, i, c]
    flat = O.pack_kept(kept)
    assert flat.tolist() == [0, 2, 5, 0, 1, 10, 0, 7, 8, 0, 1, 0, 3, 0, 4]
