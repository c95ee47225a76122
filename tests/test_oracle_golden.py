"""The oracle against hand-derived worked examples and closed forms.

The pages print no numeric example, so each fixture under tests/golden/ is a
small case whose answer follows from the definition by hand (ratios of chosen
weights); the derivation and the passage it rests on sit in the fixture.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def frac(s):
    return float(Fraction(s))


def test_chunked_scores_scale_and_whole_cache_softmax():
    g = load("chunked_scores.json")
    w0 = g["key_log_weights"]["dim0"]
    w1 = g["key_log_weights"]["dim1"]
    n = len(w0)
    keys = np.zeros((n, g["d"]))
    keys[:, 0] = [math.log(x) for x in w0]
    keys[:, 1] = [math.log(x) for x in w1]
    q = np.array(g["queries"], float)[None]          # [G=1, Nq, d]
    s = O.unit_scores(q, keys, g["n_sinks"], g["chunk_size"], g["q_per_chunk"])
    np.testing.assert_allclose(s, [frac(x) for x in g["expected_scores"]], rtol=1e-14, atol=0)
    kept = O.select_unit(s, g["keep"], g["n_sinks"])
    assert kept.tolist() == g["expected_kept"]


def test_gqa_max_over_queries_and_heads():
    g = load("gqa_max.json")
    kw = g["key_weights"]
    keys = np.log(np.array([kw["a"], kw["b"], kw["c"], kw["e"]], float).T)   # [3, 4]
    q = np.array([g["queries_head0"], g["queries_head1"]], float)           # [2, 2, 4]
    s = O.unit_scores(q, keys, g["n_sinks"], g["chunk_size"], g["q_per_chunk"])
    np.testing.assert_allclose(s, [frac(x) for x in g["expected_scores"]], rtol=1e-14, atol=0)


def test_gqa_consecutive_head_mapping():
    g = load("gqa_mapping.json")
    d = g["d"]
    k = np.zeros((1, 2, 2, d))
    k[0, 0, :, 0] = np.log(g["kv0_log_weights_dim0"])
    k[0, 1, :, 0] = np.log(g["kv1_log_weights_dim0"])
    q = np.array(g["queries"], float)[None, :, None, :]                     # [1, 4, 1, d]
    s = O.scores(q, k, n_sinks=0, chunk_size=2, q_per_chunk=1)
    want = np.array([[frac(x) for x in row] for row in g["expected_scores"]])
    np.testing.assert_allclose(s[0], want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("case", load("budgets.json")["cases"])
def test_budget_examples(case):
    L = case.get("n_layers", len(case["sens"]) if case["sens"] else None)
    got = O.layer_budgets(case["total"], L, case["sens"], case["alpha"])
    assert got.tolist() == case["expected"]


@pytest.mark.parametrize("case", load("select_ties.json")["cases"])
def test_select_examples(case):
    got = O.select_unit(np.array(case["scores"]), case["keep"], case["n_sinks"])
    assert got.tolist() == case["expected"]


# --- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 7, 64])
def test_equal_keys_give_uniform_attention(n):
    rng = np.random.default_rng(n)
    key = rng.normal(size=8)
    keys = np.tile(key, (n, 1))
    q = rng.normal(size=(3, 8))
    p = O.attention_probs(q, keys)
    np.testing.assert_allclose(p, 1.0 / n, rtol=1e-15)


def test_zero_query_gives_uniform_attention():
    rng = np.random.default_rng(1)
    keys = rng.normal(size=(37, 16)) * 5
    p = O.attention_probs(np.zeros((2, 16)), keys)
    np.testing.assert_allclose(p, 1.0 / 37, rtol=1e-15)


def test_single_position_cache_scores_one():
    s = O.unit_scores(np.ones((1, 1, 4)), np.ones((1, 4)), n_sinks=0, chunk_size=1, q_per_chunk=1)
    assert s.tolist() == [1.0]


def test_all_sinks():
    s = O.unit_scores(np.ones((2, 0, 4)), np.ones((3, 4)), n_sinks=5, chunk_size=4, q_per_chunk=3)
    assert s.tolist() == [1.0, 1.0, 1.0]
    assert O.chunk_bounds(3, 5, 4) == []


def test_two_key_logistic_closed_form():
    # p(key 1) = 1 / (1 + exp(-(q.k1 - q.k0)/sqrt(d))): the logistic of the logit gap.
    d = 16
    rng = np.random.default_rng(3)
    keys = rng.normal(size=(2, d))
    q = rng.normal(size=(1, d))
    gap = float(q[0] @ (keys[1] - keys[0])) / math.sqrt(d)
    p = O.attention_probs(q, keys)
    assert p[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(-gap)), rel=1e-14)


def test_chunk_partition_examples():
    assert O.chunk_bounds(10, 2, 4) == [(2, 6), (6, 10)]
    assert O.chunk_bounds(11, 2, 4) == [(2, 6), (6, 10), (10, 11)]
    # 131,072 positions after 4 sinks in chunks of 4096: 31 full chunks and one of 4092
    b = O.chunk_bounds(131072, 4, 4096)
    assert len(b) == 32 and b[-1] == (4 + 31 * 4096, 131072) and b[-1][1] - b[-1][0] == 4092
    assert O.query_rows(3, 410) == (1230, 1640)
