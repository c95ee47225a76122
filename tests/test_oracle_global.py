"""Pins of the oracle's global eviction with ragged heads and of decode attention
over the ragged compacted cache (KV² summary, "무엇과 다른가": gather the local
scores into one global tensor, pin sinks, evict the lowest to the budget;
"전제와 한계": a headwise-compacted cache with a different length per head needs
an attention kernel that accepts it)."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O


def key(s, u, i):
    return (-s[u, i], u, i)


@pytest.mark.parametrize("seed", range(10))
def test_select_global_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N, S = int(rng.integers(2, 6)), int(rng.integers(0, 2))
    U = L * H
    s = rng.integers(0, 3, size=(L, H, N)).astype(np.float64) / 2   # many ties
    cands = [(u, i) for u in range(U) for i in range(S, N)]
    need = int(rng.integers(0, len(cands) + 1))
    got = O.select_global(s, U * S + need, S)
    flat = s.reshape(U, N)
    good = []
    for c in itertools.combinations(cands, need):
        cs = set(c)
        if all(key(flat, *a) < key(flat, *b) for a in cs for b in cands if b not in cs):
            good.append(cs)
    assert len(good) == 1
    chosen = {(u, i) for u in range(U) for i in got[u] if i >= S}
    assert chosen == good[0]
    for u in range(U):
        assert list(got[u][:S]) == list(range(S)) and list(got[u]) == sorted(got[u])


def test_select_global_one_unit_is_the_per_head_select():
    rng = np.random.default_rng(5)
    s = rng.random(50)
    for k in (4, 10, 50):
        assert np.array_equal(O.select_global(s[None, None], k, 4)[0], O.select_unit(s, k, 4))


def test_select_global_invariants_and_errors():
    rng = np.random.default_rng(6)
    L, H, N, S = 3, 4, 200, 4
    s = rng.random((L, H, N))
    s[:, :, :S] = 1.0
    total = L * H * 20
    kept = O.select_global(s, total, S)
    assert sum(len(x) for x in kept) == total
    assert len({len(x) for x in kept}) > 1                     # ragged
    # every kept non-sink entry scores at least as high as every evicted one
    flat = s.reshape(L * H, N)
    inside = np.zeros_like(flat, bool)
    for u, x in enumerate(kept):
        inside[u, x] = True
    assert flat[:, S:][inside[:, S:]].min() >= flat[:, S:][~inside[:, S:]].max()
    for bad in (L * H * S - 1, L * H * N + 1):
        with pytest.raises(O.BudgetError):
            O.select_global(s, bad, S)
    assert all(len(x) == N for x in O.select_global(s, L * H * N, S))


def test_pack_and_compact_ragged_by_hand():
    kept = [np.array([0, 2]), np.array([1]), np.array([0, 1, 3])]
    flat, off = O.pack_ragged(kept)
    assert flat.tolist() == [0, 2, 1, 0, 1, 3] and off.tolist() == [0, 2, 3, 6]
    k = np.arange(1 * 3 * 4 * 2, dtype=np.float64).reshape(1, 3, 4, 2)
    ko, vo = O.compact_ragged(k, -k, kept)
    assert ko.tolist() == [[0, 1], [4, 5], [10, 11], [16, 17], [18, 19], [22, 23]]
    assert np.array_equal(vo, -ko)


def test_decode_attention_closed_forms():
    d = 4
    q = np.zeros((1, 2, d))
    q[0, :, 0] = 2.0                  # q . k / sqrt(4) = k[0]
    # unit 0: two rows with logits ln 3 and 0 -> weights 3/4 and 1/4
    k0 = np.array([[math.log(3.0), 0, 0, 0], [0, 0, 0, 0]])
    v0 = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    # unit 1: three identical keys -> the mean of the values
    k1 = np.ones((3, d))
    v1 = np.array([[3.0, 0, 0, 0], [0, 6.0, 0, 0], [0, 0, 9.0, 0]])
    ko, vo = np.concatenate([k0, k1]), np.concatenate([v0, v1])
    off = np.array([0, 2, 5])
    o = O.decode_attention(q, ko, vo, off, kv_heads=2)      # G = 1: head h reads unit h
    assert np.allclose(o[0, 0], [0.75, 0.25, 0, 0], rtol=0, atol=1e-15)
    assert np.allclose(o[0, 1], [1.0, 2.0, 3.0, 0], rtol=0, atol=1e-14)


def test_decode_attention_gqa_mapping_single_and_empty_rows():
    d = 2
    q = np.ones((1, 4, d))
    ko = np.zeros((1, d))
    vo = np.array([[5.0, 7.0]])
    off = np.array([0, 1, 1])         # unit 0 has one row, unit 1 none
    o = O.decode_attention(q, ko, vo, off, kv_heads=2)      # G = 2
    assert o[0, 0].tolist() == [5.0, 7.0] and o[0, 1].tolist() == [5.0, 7.0]
    assert o[0, 2].tolist() == [0.0, 0.0] and o[0, 3].tolist() == [0.0, 0.0]


def test_decode_attention_row_order_does_not_matter():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 4, 8))
    ko = rng.standard_normal((30, 8))
    vo = rng.standard_normal((30, 8))
    off = np.array([0, 7, 19, 25, 30])
    a = O.decode_attention(q, ko, vo, off, kv_heads=2)
    perm = np.concatenate([off[u] + rng.permutation(off[u + 1] - off[u]) for u in range(4)])
    b = O.decode_attention(q, ko[perm], vo[perm], off, kv_heads=2)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
