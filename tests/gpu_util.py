"""Shared helpers for the GPU parity tests (comparison rules and plumbing).

Tolerances:
  scores   relative error <= 2e-3 wherever the oracle value is >= 1e-36 (bf16
           inputs, fp32 accumulation and exp2); below that (fp32 underflow and
           flush-to-zero territory) the GPU value must itself be <= 1e-36.
  kept     exact, except positions whose oracle score lies within 2e-3 (relative)
           of the oracle's threshold tau, the (k - S)-th best non-sink score:
           there the float64 and fp32 orders may legitimately differ.
  queries  (stage-1 selection from a score tensor) the float64 mean of the
           oracle decides; the GPU ranks by a float32 sum over the L * Hkv
           units, whose error is at most (U - 1) 2^-24 of the sum (recursive
           summation of non-negative terms), so a position may differ from the
           oracle's set only if its mean lies within 2 U 2^-24 of the chunk's
           cut-off, relative.
"""
from __future__ import annotations

import multiprocessing
import os

import numpy as np
import torch

from oracle import oracle as O

RTOL = 2e-3
FLOOR = 1e-36


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def score_errors(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    big = o >= FLOOR
    rel = np.abs(g[big] - o[big]) / o[big] if big.any() else np.zeros(1)
    return float(rel.max()), int(np.sum(g[~big] > FLOOR))


def assert_scores_close(g, o, what=""):
    worst, bad_small = score_errors(g, o)
    assert worst <= RTOL, f"{what}: max relative error {worst:.3e} > {RTOL}"
    assert bad_small == 0, f"{what}: {bad_small} values above {FLOOR} where the oracle underflows"
    return worst


def threshold(o_scores: np.ndarray, k: int, S: int) -> float:
    rest = np.sort(o_scores[S:])[::-1]
    if k - S <= 0 or rest.size == 0:
        return float("inf")
    return float(rest[k - S - 1])


def assert_kept_match(g_kept, o_scores, k, S, what=""):
    """GPU kept list vs the oracle's selection on the oracle's scores."""
    g = np.asarray(g_kept, np.int64)
    n = o_scores.shape[0]
    s_eff = min(S, n)
    assert g.shape == (k,), f"{what}: kept count {g.shape} != {k}"
    assert np.all(np.diff(g) > 0), f"{what}: kept not ascending"
    assert g[:s_eff].tolist() == list(range(s_eff)), f"{what}: sinks missing"
    o = O.select_unit(o_scores, k, s_eff)
    diff = set(g.tolist()) ^ set(o.tolist())
    if diff:
        tau = threshold(o_scores, k, s_eff)
        far = [i for i in diff if abs(o_scores[i] - tau) > RTOL * tau]
        assert not far, f"{what}: {len(far)} kept positions differ outside the tie band"
    return len(diff)


def assert_valid_selection(scores_row: torch.Tensor, kept_row: torch.Tensor, k: int, S: int, what=""):
    """Property check at any size: count, sinks, order, and every kept
    non-sink beats every evicted position (score, then lower position)."""
    n = scores_row.numel()
    s_eff = min(S, n)
    kept = kept_row.long()
    assert kept.numel() == k
    assert torch.all(kept[1:] > kept[:-1]), f"{what}: not ascending"
    assert torch.equal(kept[:s_eff].cpu(), torch.arange(s_eff)), f"{what}: sinks"
    mask = torch.zeros(n, dtype=torch.bool, device=scores_row.device)
    mask[kept] = True
    mask[:s_eff] = False
    out = ~mask
    out[:s_eff] = False
    if mask.any() and out.any():
        s = scores_row.float()
        idx = torch.arange(n, device=s.device)
        worst_in = s[mask].min()
        best_out = s[out].max()
        assert worst_in >= best_out, f"{what}: a kept score is below an evicted one"
        if worst_in == best_out:   # on the tie value, kept positions must precede evicted ones
            tie_in = idx[mask & (s == worst_in)].max()
            tie_out = idx[out & (s == best_out)].min()
            assert tie_in < tie_out, f"{what}: tie broken toward a higher position"


def assert_queries_match_f64(got, score64, n_cache, n_sinks, chunk_size, rho, what=""):
    """GPU per-chunk query positions vs the oracle's selection on the float64
    mean over (layer, KV head) of score64 [L, Hkv, N].  Counts, order and range
    are exact; membership may differ only inside the float32 rounding band of
    the chunk's cut-off.  Returns the number of positions that differ."""
    s = np.asarray(score64, np.float64)
    U = int(np.prod(s.shape[:-1]))
    mean = O.token_scores(s)
    want = O.select_queries(mean, n_cache, n_sinks, chunk_size, rho)
    bounds = O.chunk_bounds(n_cache, n_sinks, chunk_size)
    assert len(got) == len(want) == len(bounds), f"{what}: chunk count"
    ndiff = 0
    for r, ((a, b), x, y) in enumerate(zip(bounds, got, want)):
        x = np.asarray(x, np.int64)
        assert x.shape == y.shape, f"{what} chunk {r}: {x.shape[0]} positions, want {y.shape[0]}"
        assert np.all(np.diff(x) > 0), f"{what} chunk {r}: not ascending"
        assert x.size == 0 or (x[0] >= a and x[-1] < b), f"{what} chunk {r}: outside the chunk"
        diff = set(x.tolist()) ^ set(y.tolist())
        if not diff:
            continue
        cut = float(np.sort(mean[a:b])[::-1][len(y) - 1])
        band = 2.05 * U * 2.0 ** -24 * abs(cut)
        for i in diff:
            assert abs(mean[i] - cut) <= band, f"{what} chunk {r}: position {i} mean {mean[i]!r} cut {cut!r}"
        ndiff += len(diff)
    return ndiff


_TASK = None


def _run_task(i):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return _TASK(i)


def fork_map(f, items, procs: int = 8):
    """list(map(f, items)) over a pool of forked worker processes.

    Test plumbing for the oracle's independent pieces (for example the chunks
    of one unit): f is handed to the workers through the fork, so its large
    arguments are never pickled.  The workers run numpy only and never touch
    the GPU; they leave through os._exit, so no exit handler of the parent's
    GPU runtime runs in them."""
    global _TASK
    items = list(items)
    procs = max(1, min(procs, len(items), os.cpu_count() or 1))
    if procs == 1:
        return [f(i) for i in items]
    _TASK = f
    try:
        with multiprocessing.get_context("fork").Pool(procs) as pool:
            return pool.map(_run_task, items)
    finally:
        _TASK = None
