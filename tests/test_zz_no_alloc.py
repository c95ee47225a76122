"""kvs_compress_block_noalloc (the library's own per-GPU scratch) against
kvs_compress_block (a caller workspace): identical scores, kept positions,
budgets and compacted rows, bit for bit, on two calls in a row, the second on
a smaller problem, so that whatever the first call left in the shared scratch
is shown not to leak into the second.  The scoring plan depends on the
workspace a call is given (a large one lets pass 1 split long caches' keys
further), so where the two could differ the workspace call gets a workspace
of the scratch's size."""
import numpy as np
import pytest
import torch

from workloads import SMALL, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import kv_cache_compression_kvs_amd as pkg
    return pkg


def outputs(K, s, kl, dt):
    rows = s.kv_heads * int(sum(kl))
    return (torch.full((s.layers, s.kv_heads, s.n_cache), float("nan"), device="cuda"),
            torch.full((rows,), -1, dtype=torch.int32, device="cuda"),
            torch.zeros(rows, s.head_dim, dtype=dt, device="cuda"),
            torch.zeros(rows, s.head_dim, dtype=dt, device="cuda"))


NOALLOC_BYTES = 64 * 1024 * 1024  # KVS_NOALLOC_SCRATCH_BYTES


def compare_one(K, w, sens=None, alpha=0.0, total=None, q_key="q", ws_bytes=None):
    s = w.shape
    x = gen.episodic_inputs(w, device="cuda") if w.kind == "episodic" else \
        gen.single_inputs(w, device="cuda")
    q = x["q_episodes"][0] if w.kind == "episodic" else x["q"]
    if w.kind == "episodic":
        sens, alpha, total = x["sens"], w.alpha, w.total_budget
    elif total is None:
        total = w.keep_per_layer() * s.layers
    p = K.make_problem(s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache, s.n_sinks,
                       s.chunk_size, s.q_per_chunk, x["k"].dtype)
    kl = K.kvs_layer_budgets(s.layers, total, sens, alpha, s.n_cache, s.n_sinks)
    a = outputs(K, s, kl, x["k"].dtype)
    b = outputs(K, s, kl, x["k"].dtype)
    ws = K.workspace(p) if ws_bytes is None else \
        torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ka = K.kvs_compress_block(p, q, x["k"], x["v"], total, sens, alpha, *a, 0, ws=ws)
    kb = K.kvs_compress_block_noalloc(p, q, x["k"], x["v"], total, sens, alpha, *b, 0)
    torch.cuda.synchronize()
    assert np.array_equal(ka, kb), "budgets"
    names = ("scores", "kept", "k_out", "v_out")
    for n, ta, tb in zip(names, a, b):
        same = torch.equal(ta, tb) if n != "scores" else \
            torch.equal(ta.view(torch.int32), tb.view(torch.int32))
        assert same, f"{w.name}: {n} differs"
    assert not torch.isnan(b[0]).any()
    return s


def test_noalloc_matches_workspace_call_twice(K):
    """First call: several chunks and a ragged tail (the kv2 small shape);
    second call: a smaller problem (one layer, a shorter cache in one chunk,
    pass-1 keys split across workgroups), which reads scratch the first one
    wrote."""
    import dataclasses
    w1 = SMALL["kv2_32k"]
    w2 = dataclasses.replace(w1, name="kv2_smaller",
                             shape=dataclasses.replace(w1.shape, layers=1, n_cache=2100,
                                                       chunk_size=2096, q_per_chunk=60))
    s1 = compare_one(K, w1)
    s2 = compare_one(K, w2)

    def need(s):
        return K.kvs_workspace_bytes(K.make_problem(s.layers, s.q_heads, s.kv_heads, s.head_dim,
                                                    s.n_cache, s.n_sinks, s.chunk_size,
                                                    s.q_per_chunk, torch.bfloat16))
    assert s2.layers * s2.kv_heads * s2.n_cache < s1.layers * s1.kv_heads * s1.n_cache
    assert need(s2) < need(s1)


def test_noalloc_one_chunk_workload(K):
    """The episodic shape (one chunk, sensitivity-split budgets) through both
    entry points."""
    compare_one(K, SMALL["episodic"])


def test_noalloc_full_size_then_small(K):
    """The largest single-GPU workload's scratch (about 60 MB with pass 1's
    keys unsplit), then a small one: both equal to the workspace call given
    the same amount of workspace."""
    from workloads import FULL
    compare_one(K, FULL["kv2_131k"], ws_bytes=NOALLOC_BYTES)
    torch.cuda.empty_cache()
    compare_one(K, SMALL["kv2_131k"])


def test_noalloc_rejects_oversize(K):
    """A problem that needs more than KVS_NOALLOC_SCRATCH_BYTES fails with
    KVS_E_SCRATCH before anything is enqueued; the outputs stay untouched."""
    # 128 layers x 32 query heads x 20 chunks x 410 rows of fp32 row
    # statistics is 134 MB of scratch
    p = K.make_problem(128, 32, 8, 128, 4 + 20 * 4096, 4, 4096, 410, torch.bfloat16)
    assert K.kvs_workspace_bytes(p) > 64 * 1024 * 1024
    t = torch.full((64,), 7.0, device="cuda")
    with pytest.raises(K.KvsError, match="KVS_E_SCRATCH"):
        K.kvs_compress_block_noalloc(p, t, t, t, 2621 * 128, None, 0.0, t, t, t, t, 0)
    torch.cuda.synchronize()
    assert bool((t == 7.0).all())
