"""The oracle's block-prefill loop and episodic driver on small hand-checkable cases."""
import numpy as np

from oracle import oracle as O


def tokens(L, Hkv, T, d, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(L, Hkv, T, d)), rng.normal(size=(L, Hkv, T, d))


def test_zero_queries_keep_the_oldest_positions():
    # q = 0 makes every probability 1/N, so all non-sinks tie and the lowest
    # positions win: the kept positions are always 0..M-1.
    L, Hkv, G, d, B, M, S, nb, nq = 2, 2, 2, 4, 3, 5, 1, 4, 2
    k, v = tokens(L, Hkv, B * nb, d)
    q = np.zeros((nb, L, Hkv * G, nq, d))
    recs = O.block_loop(k, v, q, B, M, S)
    scored = [r for r in recs if "kept" in r]
    assert [r["block"] for r in scored] == [1, 2, 3]
    for r in scored:
        n = r["n_cache"]
        np.testing.assert_allclose(r["scores"][..., S:], 1.0 / n, rtol=1e-14)
        for kl in r["kept"]:
            assert (kl == np.arange(M)).all()


def test_attended_token_survives_and_positions_track_rows():
    L, Hkv, G, d, B, M, S, nb, nq = 1, 1, 1, 8, 4, 6, 2, 4, 1
    k, v = tokens(L, Hkv, B * nb, d, seed=1)
    target = 13                                  # in block 3
    q = np.zeros((nb, L, G, nq, d))
    q[:, 0, 0, 0] = 6.0 * k[0, 0, target] / np.linalg.norm(k[0, 0, target])
    recs = O.block_loop(k, v, q, B, M, S)
    last = recs[-1]
    assert "kept" in last
    kept_pos = last["pos"][0, 0][last["kept"][0][0]]
    assert target in kept_pos.tolist()
    for r in recs:                               # every cache row is the token it claims to be
        for i, p in enumerate(r["pos"][0, 0]):
            assert np.array_equal(r["k"][0, 0, i], k[0, 0, p])
            assert np.array_equal(r["v"][0, 0, i], v[0, 0, p])


def test_block_step_equals_single_compress_and_teacher_forcing():
    L, Hkv, G, d, B, M, S, nb, nq = 1, 2, 3, 8, 5, 7, 2, 3, 4
    k, v = tokens(L, Hkv, B * nb, d, seed=2)
    q = np.random.default_rng(3).normal(size=(nb, L, Hkv * G, nq, d)) * 2
    recs = O.block_loop(k, v, q, B, M, S)
    r = recs[2]
    n = r["n_cache"]
    one = O.compress(q[2], r["k"], r["v"], S, n - S, nq, [M] * L)
    np.testing.assert_array_equal(one["scores"], r["scores"])
    for a, b in zip(one["kept"], r["kept"]):
        np.testing.assert_array_equal(a, b)
    # teacher forcing from the cache recorded before block 2 reproduces step 2
    prev = recs[1]
    kk = np.stack(prev["kept"])
    start = (np.take_along_axis(prev["k"], kk[..., None], axis=2),
             np.take_along_axis(prev["v"], kk[..., None], axis=2),
             np.take_along_axis(prev["pos"], kk, axis=2))
    forced = O.block_loop(k, v, q, B, M, S, teacher={2: start})
    np.testing.assert_array_equal(forced[2]["scores"], r["scores"])


def test_episodic_budgets_and_counts():
    rng = np.random.default_rng(4)
    L, Hkv, G, d, N, S, E, nq = 3, 2, 2, 8, 40, 2, 4, 3
    k = rng.normal(size=(L, Hkv, N, d))
    v = rng.normal(size=(L, Hkv, N, d))
    q = rng.normal(size=(E, L, Hkv * G, nq, d))
    sens = [0.6, 1.4, 1.0]
    kl, outs = O.episodic(k, v, q, sens, 3.0, 45, S, N, nq)
    assert int(kl.sum()) == 45 and kl[1] == kl.max() and kl[0] == kl.min()
    assert len(outs) == E
    for o in outs:
        for l in range(L):
            assert o["kept"][l].shape == (Hkv, kl[l])
            assert o["out"][l][0].shape == (Hkv, kl[l], d)
