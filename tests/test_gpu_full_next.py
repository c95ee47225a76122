"""GPU parity at full workload sizes for the rows next to the main path: global
eviction with ragged per-head lengths and decode over the ragged cache (KV²
summary, "무엇과 다른가" and "전제와 한계"), the layer-sensitivity calibration
(EpiCache review, "+α: 레이어별 예산 배분", Fig. 4(a)) and episode clustering
(EpiCache review, "방법: 3단계" (1) and (3)).

As in test_gpu_full.py, inputs are generated in HBM and the oracle checks
sampled outputs it can compute alone, while properties that hold at any size
are checked everywhere.  For the global selection those properties fix the
kept set uniquely: the kept count, every unit's sinks, ascending lists, every
kept non-sink entry scoring at least every evicted one, and on the tie value
every kept entry preceding every evicted one in (unit, position) order.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from workloads import FULL, ScoreShape, gen

from gpu_util import assert_scores_close, f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def K():
    import kv_cache_compression_kvs_amd as pkg
    return pkg


def check_global_selection(scores, kept, offsets, total, S, what):
    """The properties above, vectorised on the GPU.  scores [U, N]."""
    U, N = scores.shape
    S = min(S, N)
    off = offsets.long()
    assert int(off[0]) == 0 and int(off[-1]) == total, what
    counts = off[1:] - off[:-1]
    assert torch.all(counts >= S), f"{what}: a unit lost its sinks"
    unit_of = torch.repeat_interleave(torch.arange(U, device=scores.device), counts)
    kk = kept.long()
    pos_in_unit = torch.arange(total, device=scores.device) - off[:-1][unit_of]
    sink = pos_in_unit < S
    assert torch.equal(kk[sink], pos_in_unit[sink]), f"{what}: sinks"
    same = unit_of[1:] == unit_of[:-1]
    assert torch.all(kk[1:][same] > kk[:-1][same]), f"{what}: not ascending"
    inside = torch.zeros(U, N, dtype=torch.bool, device=scores.device)
    inside[unit_of, kk] = True
    inside[:, :S] = False
    out = ~inside
    out[:, :S] = False
    if not inside.any() or not out.any():
        return
    s = scores.float()
    worst_in = s[inside].min()
    best_out = s[out].max()
    assert worst_in >= best_out, f"{what}: a kept score below an evicted one"
    if worst_in == best_out:
        flat = torch.arange(U * N, device=scores.device).view(U, N)
        last_in = flat[inside & (s == worst_in)].max()
        first_out = flat[out & (s == best_out)].min()
        assert last_in < first_out, f"{what}: tie order"


def global_full(K, w, q, k, v, total):
    s = w.shape
    U = s.layers * s.kv_heads
    p = K.make_problem(s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache, s.n_sinks,
                       s.chunk_size, s.q_per_chunk, k.dtype)
    scores = torch.full((s.layers, s.kv_heads, s.n_cache), float("nan"), device="cuda")
    kept = torch.full((total,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((U + 1,), -1, dtype=torch.int64, device="cuda")
    ko = torch.empty(total, s.head_dim, dtype=k.dtype, device="cuda")
    vo = torch.empty(total, s.head_dim, dtype=k.dtype, device="cuda")
    K.kvs_compress_global(p, q, k, v, total, scores, kept, offsets, ko, vo)
    torch.cuda.synchronize()
    return p, scores, kept, offsets, ko, vo


def check_rows_and_decode(K, p, w, k, v, scores, kept, offsets, ko, vo, total, what):
    s = w.shape
    U = s.layers * s.kv_heads
    off = offsets.cpu().numpy()
    for u in range(U):          # gathered rows are the kept rows, bit for bit
        a, b = int(off[u]), int(off[u + 1])
        idx = kept[a:b].long()
        assert torch.equal(ko[a:b], k[u // s.kv_heads, u % s.kv_heads, idx]), f"{what} K u={u}"
        assert torch.equal(vo[a:b], v[u // s.kv_heads, u % s.kv_heads, idx]), f"{what} V u={u}"
    q1 = torch.randn(s.layers, s.q_heads, s.head_dim,
                     generator=torch.Generator().manual_seed(4)).to(k.dtype)
    out = torch.full((s.layers, s.q_heads, s.head_dim), float("nan"), device="cuda")
    K.kvs_decode_ragged(p, q1.cuda(), ko, vo, offsets, total, out)
    torch.cuda.synchronize()
    G = s.group
    for (l, h) in [(0, 0), (s.layers - 1, s.q_heads - 1), (s.layers // 2, s.q_heads // 2 + 1)]:
        u = l * s.kv_heads + h // G
        a, b = int(off[u]), int(off[u + 1])
        # one head at a time: the rows of its unit alone
        qh = f64(q1[l, h])[None, None]
        want = O.decode_attention(qh, f64(ko[a:b]), f64(vo[a:b]), np.array([0, b - a]), 1)[0, 0]
        got = out[l, h].cpu().double().numpy()
        scale = float(np.abs(f64(vo[a:b])).max())
        assert np.abs(got - want).max() <= 1e-3 * scale, f"{what}: decode (l={l}, h={h})"


@pytest.mark.parametrize("name", ["kv2_131k", "episodic"])
def test_global_eviction_full(K, name):
    w = FULL[name]
    s = w.shape
    if w.kind == "episodic":
        x = gen.episodic_inputs(w, device="cuda")
        q, total = x["q_episodes"][0], w.total_budget * s.kv_heads
    else:
        x = gen.single_inputs(w, device="cuda")
        q, total = x["q"], w.keep_per_layer() * s.layers * s.kv_heads
    p, scores, kept, offsets, ko, vo = global_full(K, w, q, x["k"], x["v"], total)
    U = s.layers * s.kv_heads
    check_global_selection(scores.view(U, s.n_cache), kept, offsets, total, s.n_sinks, name)
    counts = (offsets[1:] - offsets[:-1]).cpu()
    print(f"{name}: per-head kept rows from {int(counts.min())} to {int(counts.max())}")
    # the oracle's global selection on the GPU's scores, restricted to two
    # units: their lists are what the whole-tensor threshold leaves in them
    sc = scores.view(U, s.n_cache)
    need = total - U * s.n_sinks
    flat = sc[:, s.n_sinks:].reshape(-1)
    tau = torch.topk(flat, need).values[-1].item()
    for u in (0, U - 1):
        row = sc[u].double().cpu().numpy()
        mine = O.select_global(row[None, None], int(counts[u]), s.n_sinks)[0]
        a = int(offsets[u])
        assert np.array_equal(kept[a:a + int(counts[u])].cpu().numpy().astype(np.int64), mine)
        assert row[mine[s.n_sinks:]].min() >= tau if len(mine) > s.n_sinks else True
    check_rows_and_decode(K, p, w, x["k"], x["v"], scores, kept, offsets, ko, vo, total, name)


def test_similarity_full(K):
    """Key similarity at the episodic shape (28 layers x 8 KV heads x 92,160
    tokens); the oracle recomputes two whole layers."""
    w = FULL["episodic"]
    s = w.shape
    shape = ScoreShape(s.layers, s.kv_heads, s.kv_heads, s.head_dim, s.n_cache, 0, s.n_cache, 1,
                       s.dtype)
    x = gen.calibration_keys(shape, s.n_cache, seed=3, device="cuda")
    p = K.make_problem(s.layers, s.kv_heads, s.kv_heads, s.head_dim, s.n_cache, 0, s.n_cache, 1,
                       x["k_full"].dtype)
    sim = torch.empty(s.layers, dtype=torch.float64, device="cuda")
    K.kvs_key_similarity(p, x["k_full"], x["k_block"], sim)
    torch.cuda.synchronize()
    got = sim.cpu().numpy()
    for l in (0, s.layers - 1):
        want = O.key_similarity(f64(x["k_full"][l:l + 1]), f64(x["k_block"][l:l + 1]))[0]
        assert abs(got[l] - want) <= 2e-5, (l, got[l], want)
    sens = K.kvs_sensitivity(got.tolist())
    assert np.all(sens > 0) and np.all(sens < 1)


def test_episode_clustering_full(K):
    """2,048 unit-norm segment embeddings of width 1,024 into 4 episodes, 10
    rounds, medoids and 64 questions (the bench's configuration)."""
    emb = gen.episode_embeddings(2048, 1024, 4, seed=0)
    x = emb["x"].cuda()
    init = emb["x"][emb["init_index"]].contiguous()
    cent = torch.empty(4, 1024, device="cuda")
    assign = torch.empty(2048, dtype=torch.int32, device="cuda")
    K.kvs_kmeans(x, init.cuda(), 10, cent, assign)
    med = torch.empty(4, dtype=torch.int32, device="cuda")
    totals = torch.empty(2048, device="cuda")
    K.kvs_medoids(x, assign, 4, med, totals)
    ep = torch.empty(64, dtype=torch.int32, device="cuda")
    K.kvs_match_episodes(emb["q"].cuda(), cent, ep)
    torch.cuda.synchronize()
    x64 = emb["x"].double().numpy()
    oc, oa = O.kmeans(x64, init.double().numpy(), 10)
    assert np.array_equal(assign.cpu().numpy(), oa)
    assert np.abs(cent.cpu().double().numpy() - oc).max() <= 1e-5
    want_t = O.medoid_totals(x64, oa)
    assert np.all(np.abs(totals.cpu().double().numpy() - want_t) <= 1e-5 * want_t + 1e-6)
    got_m = med.cpu().numpy()
    for e, want_m in enumerate(O.medoids(x64, oa, 4)):       # up to fp32 near-ties
        assert oa[got_m[e]] == e
        assert want_t[got_m[e]] - want_t[want_m] <= 1e-5 * want_t[want_m]
    assert np.array_equal(ep.cpu().numpy(), O.nearest_centroid(emb["q"].double().numpy(), oc))
