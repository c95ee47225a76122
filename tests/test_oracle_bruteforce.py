"""The oracle against an independent 50-digit brute force on tiny inputs.

The brute force walks the definition element by element in mpmath (no max
shift, no vectorisation, no row blocking): for each chunk position it takes
every query of the owning chunk and every query head of the group, forms the
exact softmax over the whole cache and keeps the largest value.
"""
import itertools

import mpmath
import numpy as np
import pytest

from oracle import oracle as O

mpmath.mp.dps = 50


def brute_scores(q, k, n_sinks, chunk, nq):
    L, Hq, Nq, d = q.shape
    _, Hkv, N, _ = k.shape
    G = Hq // Hkv
    inv = 1 / mpmath.sqrt(d)
    out = np.zeros((L, Hkv, N))
    for l in range(L):
        for g in range(Hkv):
            for i in range(N):
                if i < n_sinks:
                    out[l, g, i] = 1.0
                    continue
                r = (i - n_sinks) // chunk
                best = mpmath.mpf(0)
                for h in range(g * G, (g + 1) * G):
                    for j in range(r * nq, (r + 1) * nq):
                        z = [sum(mpmath.mpf(float(q[l, h, j, t])) * mpmath.mpf(float(k[l, g, ii, t]))
                                 for t in range(d)) * inv for ii in range(N)]
                        den = sum(mpmath.exp(x) for x in z)
                        p = mpmath.exp(z[i]) / den
                        if p > best:
                            best = p
                out[l, g, i] = float(best)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_scores_match_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    L = 1 + seed % 2
    Hkv = 1 + seed % 2
    G = [1, 2, 3][seed % 3]
    d = [2, 4, 8][seed % 3]
    S = seed % 3
    chunk = 3 + seed % 4
    N = S + 2 * chunk + 1 + seed % 3        # two full chunks and a ragged one
    R = len(O.chunk_bounds(N, S, chunk))
    nq = 1 + seed % 2
    q = rng.normal(size=(L, Hkv * G, R * nq, d)) * 1.5
    k = rng.normal(size=(L, Hkv, N, d)) * 1.5
    got = O.scores(q, k, S, chunk, nq)
    want = brute_scores(q, k, S, chunk, nq)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def brute_select(s, k, n_sinks):
    """Exhaustive: the unique subset whose every member beats every non-member."""
    n = len(s)
    cand = range(n_sinks, n)
    found = []
    for sub in itertools.combinations(cand, k - n_sinks):
        inside = set(sub)
        out = [b for b in cand if b not in inside]
        ok = all((s[a] > s[b]) or (s[a] == s[b] and a < b) for a in sub for b in out)
        if ok:
            found.append(sorted(list(range(n_sinks)) + list(sub)))
    return found


@pytest.mark.parametrize("seed", range(40))
def test_select_matches_exhaustive(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    S = int(rng.integers(0, min(3, n) + 1))
    k = int(rng.integers(S, n + 1))
    levels = int(rng.integers(1, 5))        # few levels: ties are common
    s = rng.integers(0, levels, size=n) / 4.0
    s[:S] = 1.0
    found = brute_select(s, k, S)
    assert len(found) == 1, "the order (score desc, position asc) must give a unique answer"
    assert O.select_unit(s, k, S).tolist() == found[0]
