"""Pins of the oracle's stage-1 query selection (KV² summary, "어떻게 동작하나":
token score = mean over layers and KV heads; per chunk the top
n_q = max(floor(rho |C_r|), 1) positions; "무엇과 다른가": stage-2 scores may
serve as that score in a refinement pass).

Each test checks the oracle against something other than itself: closed forms,
a hand-worked float32 rounding case, brute force over every subset of tiny
chunks, and invariants."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O


def test_query_counts_closed_forms():
    # 8 chunks of 4096 after 4 sinks, the last 4092 long: floor(0.1 * 4096) = 409
    assert O.query_counts(32768, 4, 4096, 0.1) == [409] * 8
    # a ragged last chunk of 100 positions
    assert O.query_counts(4 + 4096 + 100, 4, 4096, 0.1) == [409, 10]
    # tiny rho: at least one query per chunk
    assert O.query_counts(1000, 0, 100, 1e-9) == [1] * 10
    # rho = 1: every position
    assert O.query_counts(250, 2, 100, 1.0) == [100, 100, 48]
    # the product is formed in IEEE double: 0.29 * 100 = 28.999999999999996
    assert O.query_counts(100, 0, 100, 0.29) == [28]
    # no chunk when every position is a sink
    assert O.query_counts(4, 4, 4096, 0.5) == []
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            O.query_counts(100, 0, 10, bad)


def test_token_scores_closed_form():
    L, H, N = 3, 4, 7
    l, g, i = np.meshgrid(np.arange(L), np.arange(H), np.arange(N), indexing="ij")
    s = l + 10.0 * g + 100.0 * i
    want = (L - 1) / 2 + 10.0 * (H - 1) / 2 + 100.0 * np.arange(N)
    assert np.array_equal(O.token_scores(s), want)


def dominates(p, i, j):
    return p[i] > p[j] or (p[i] == p[j] and i < j)


@pytest.mark.parametrize("seed", range(12))
def test_select_queries_brute_force(seed):
    rng = np.random.default_rng(seed)
    S, m = int(rng.integers(0, 3)), int(rng.integers(3, 8))
    N = S + int(rng.integers(1, 3 * m))
    rho = float(rng.choice([0.2, 0.34, 0.5, 0.9]))
    p = rng.integers(0, 4, size=N).astype(np.float64)   # few values: many ties
    got = O.select_queries(p, N, S, m, rho)
    bounds = O.chunk_bounds(N, S, m)
    assert len(got) == len(bounds)
    for (a, b), sel in zip(bounds, got):
        nq = max(math.floor(rho * (b - a)), 1)
        # exactly one subset of size nq has every member dominating every non-member
        good = [set(c) for c in itertools.combinations(range(a, b), nq)
                if all(dominates(p, i, j) for i in c for j in range(a, b) if j not in c)]
        assert len(good) == 1
        assert set(sel.tolist()) == good[0]
        assert list(sel) == sorted(sel)


def test_select_queries_invariants():
    rng = np.random.default_rng(7)
    L, H, N, S, m, rho = 4, 3, 1000, 4, 128, 0.1
    s = rng.integers(0, 1000, size=(L, H, N)).astype(np.float64)
    p = O.token_scores(s)
    sel = O.select_queries(p, N, S, m, rho)
    counts = O.query_counts(N, S, m, rho)
    for (a, b), x, nq in zip(O.chunk_bounds(N, S, m), sel, counts):
        assert len(x) == nq and x.min() >= a and x.max() < b
        assert np.all(np.diff(x) > 0)
        chosen = np.zeros(b - a, bool)
        chosen[x - a] = True
        assert p[a:b][chosen].min() >= p[a:b][~chosen].max()
    assert all(x.min() >= S for x in sel)        # sinks never become queries
    # permuting the (layer, KV head) units does not change the mean (integers:
    # exact), hence not the selection
    perm = rng.permutation(L * H)
    s2 = s.reshape(L * H, N)[perm].reshape(L, H, N)
    sel2 = O.select_queries(O.token_scores(s2), N, S, m, rho)
    assert all(np.array_equal(x, y) for x, y in zip(sel, sel2))


def test_refinement_takes_stage_two_scores():
    """Stage-2 scores (the oracle's own unit scores) have token granularity and
    drive a second selection: the pass keeps the chunk structure and counts."""
    rng = np.random.default_rng(11)
    L, Hq, Hkv, d, N, S, m, nq = 2, 4, 2, 16, 300, 4, 100, 5
    R = len(O.chunk_bounds(N, S, m))
    q = rng.standard_normal((L, Hq, R * nq, d))
    k = rng.standard_normal((L, Hkv, N, d))
    sc = O.scores(q, k, S, m, nq)
    sel = O.select_queries(O.token_scores(sc), N, S, m, 0.05)
    assert [len(x) for x in sel] == O.query_counts(N, S, m, 0.05) == [5, 5, 4]
