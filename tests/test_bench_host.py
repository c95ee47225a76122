"""bench.py's host-side contract: one GPU only, a clear failure without one,
and the counted work of the headline workload (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import FULL  # noqa: E402


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run_bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_default_workload_is_the_131k_shape():
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.workload == "kv2_131k" and args.gpus == 1


def test_counted_work_of_the_headline_workload():
    """Scored tokens per step and pass-1 flops per launch, as the bench counts them."""
    s = FULL["kv2_131k"].shape
    assert s.scored_tokens() == 36 * 8 * 131072 == 37_748_736
    assert 2 * s.head_dim * s.pass1_pairs() == 2 * 128 * 36 * 32 * 13120 * 131072
    assert 2 * s.head_dim * s.pass1_pairs() == 507_149_738_311_680


def test_profiled_traffic_needs_a_matching_summary(tmp_path, monkeypatch):
    assert bench.profiled_traffic("no_such_workload", "score_pass1_bf16") is None
    # a summary whose recorded source hash does not match is ignored
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_x.md").write_text(
        "kernel=score_pass1_bf16 traffic_bytes_per_launch=123 "
        "source=kv_cache_compression_kvs_amd/csrc/score_bf16.hip sha256_16=0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("x", "score_pass1_bf16") is None


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_fails_loudly():
    r = run_bench("--no-others", "--no-cpu-baseline")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr and r.stdout == ""
