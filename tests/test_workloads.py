"""The seeded generators: determinism, unit independence and the stated sizes."""
import torch

from workloads import FULL, SMALL, gen


def test_single_inputs_are_deterministic_and_unit_regenerable():
    w = SMALL["kv2_32k"]
    a = gen.single_inputs(w)
    b = gen.single_inputs(w)
    for key in ("q", "k", "v"):
        assert torch.equal(a[key], b[key])
    one = gen.single_inputs(w, layers=[1])
    assert torch.equal(one["k"][1], a["k"][1]) and torch.equal(one["q"][1], a["q"][1])
    assert a["k"].dtype == torch.bfloat16


def test_shapes_of_full_workloads():
    s = FULL["kv2_32k"].shape
    assert (s.n_chunks, s.n_queries) == (8, 3280)
    assert FULL["kv2_32k"].keep_per_layer() == 1638
    s = FULL["kv2_131k"].shape
    assert (s.n_chunks, s.n_queries) == (32, 13120)
    assert FULL["kv2_131k"].keep_per_layer() == 2621
    assert FULL["episodic"].total_budget == 229376
    assert FULL["epicache_block_loop"].shape.n_queries == 256
    assert gen.needle_positions(131072, 4).numel() == 1310


def test_tiny_recipe_needles_and_aligned_queries():
    x = gen.single_inputs(SMALL["tiny"])
    assert x["q"].dtype == torch.float32 and x["q"].shape == (1, 4, 128, 64)
    # 32 of 128 queries per head have norm sqrt(d) exactly (aligned to a needle)
    nrm = x["q"][0, 0].norm(dim=-1)
    assert torch.allclose(nrm[:32], torch.full((32,), 8.0), atol=1e-4)


def test_score_and_kept_generators():
    s = gen.score_tensor(3, 50, 4, "coarse")
    assert s.shape == (3, 50) and torch.all(s[:, :4] == 1.0)
    kept = gen.kept_lists(2, 30, 4, [10, 7])
    assert kept.numel() == 2 * 10 + 2 * 7
    assert kept[:4].tolist() == [0, 1, 2, 3]
