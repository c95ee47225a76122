"""Seeded synthetic inputs for the eviction workloads.

This module builds tensors only: keys, values, scoring queries, sensitivities
and, for the selection and compaction tests, score tensors and kept-index
lists.  It holds none of the method's arithmetic (no attention, no softmax,
no selection), so both the float64 oracle and the GPU path may consume what
it makes without sharing any computation.

Every tensor slice that belongs to one (layer, KV head) unit is drawn from
its own generator whose seed is a hash of (seed, workload, tensor, layer,
head, ...).  A unit can therefore be regenerated alone, and generation order
does not matter.  Values are drawn in float32 and rounded once to the storage
type (bf16 by round-to-nearest-even) so that every consumer reads the same
bits.

Recipes (shapes from the EpiCache review and the KV² summary; the value
distributions are synthetic stand-ins for their conversation and long-document
benchmarks, whose items are not reproduced):
  tiny                 Gaussian keys with two +8 outlier channels, 16 planted
                       needle keys per KV head, 32 of 128 queries aligned to
                       needles (cosine 0.8).
  topics               keys clustered around 4 per-unit topic centroids
                       (256-token segments, seeded topic per segment) plus
                       4 outlier channels; episode queries are centroid+noise.
  reconstruct          Gaussian keys plus 4 outlier channels; each chunk's
                       queries re-encode sorted source positions drawn from
                       that chunk (cosine 0.6 to the source key).
  reconstruct_needles  as reconstruct, plus 10 needle spans covering 1% of
                       the cache; needle positions are used as sources first.
"""
from __future__ import annotations

import hashlib
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from .configs import ScoreShape, Workload

GENERATOR_VERSION = 1


def _seed(*parts) -> int:
    h = hashlib.blake2b(repr((GENERATOR_VERSION,) + parts).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(*parts))
    return g


def storage_dtype(shape: ScoreShape) -> torch.dtype:
    return torch.float32 if shape.dtype == "f32" else torch.bfloat16


def _unit(v: torch.Tensor) -> torch.Tensor:
    return v / v.norm(dim=-1, keepdim=True)


def _orth_unit(n: torch.Tensor, r: torch.Tensor) -> torch.Tensor:
    """Unit vectors orthogonal to the unit rows of ``n`` (Gram-Schmidt of r)."""
    r = r - (r * n).sum(-1, keepdim=True) * n
    return _unit(r)


def _outliers(d: int, n_ch: int, g: torch.Generator, device, lo=4.0, hi=8.0,
              fixed: Optional[float] = None) -> torch.Tensor:
    """A per-unit offset vector with ``n_ch`` large channels."""
    off = torch.zeros(d, device=device)
    ch = torch.randperm(d, generator=g, device=device)[:n_ch]
    if fixed is not None:
        off[ch] = fixed
    else:
        mag = lo + (hi - lo) * torch.rand(n_ch, generator=g, device=device)
        sign = torch.where(torch.rand(n_ch, generator=g, device=device) < 0.5, -1.0, 1.0)
        off[ch] = mag * sign
    return off


def _topics(n_tokens: int, n_topics: int, seed: int, name: str, seg: int = 256) -> torch.Tensor:
    """Seeded topic id for every token (constant over 256-token segments)."""
    g = _gen("cpu", seed, name, "topics")
    n_seg = -(-n_tokens // seg)
    t = torch.randint(0, n_topics, (n_seg,), generator=g)
    return t.repeat_interleave(seg)[:n_tokens]


def _chunk_bounds(shape: ScoreShape):
    out = []
    a = shape.n_sinks
    while a < shape.n_cache:
        b = min(a + shape.chunk_size, shape.n_cache)
        out.append((a, b))
        a = b
    return out


def needle_positions(n_cache: int, n_sinks: int, spans: int = 10, frac: float = 0.01) -> torch.Tensor:
    """1% of the cache as ``spans`` equal spans centred at depths (t+0.5)/spans."""
    per = int(math.floor(frac * n_cache)) // spans
    pos = []
    for t in range(spans):
        c = n_sinks + int(math.floor((t + 0.5) * (n_cache - n_sinks) / spans))
        a = max(n_sinks, c - per // 2)
        b = min(n_cache, a + per)
        pos.append(torch.arange(a, b))
    return torch.unique(torch.cat(pos))


def _sources(shape: ScoreShape, seed: int, name: str, needles: Optional[torch.Tensor]) -> torch.Tensor:
    """Per-chunk sorted source positions [R, nq] shared by every unit.

    Stand-in for the stage-1 token-level selection, which is averaged over
    layers and heads and is therefore the same for all of them.
    """
    g = _gen("cpu", seed, name, "sources")
    rows = []
    for (a, b) in _chunk_bounds(shape):
        span = b - a
        nq = shape.q_per_chunk
        if needles is not None:
            inside = needles[(needles >= a) & (needles < b)]
        else:
            inside = torch.empty(0, dtype=torch.long)
        inside = inside[:nq]
        rest_pool = torch.ones(span, dtype=torch.bool)
        rest_pool[(inside - a)] = False
        pool = torch.nonzero(rest_pool).flatten() + a
        need = nq - inside.numel()
        if need > pool.numel():  # tiny chunk: sample with replacement
            pick = pool[torch.randint(0, pool.numel(), (need,), generator=g)]
        else:
            pick = pool[torch.randperm(pool.numel(), generator=g)[:need]]
        src, _ = torch.sort(torch.cat([inside, pick]))
        rows.append(src)
    if not rows:
        return torch.empty(0, shape.q_per_chunk, dtype=torch.long)
    return torch.stack(rows)


def _store(x: torch.Tensor, dt: torch.dtype) -> torch.Tensor:
    return x.to(dt)


# --------------------------------------------------------------------------
# single-shot workloads: tiny, reconstruct, reconstruct_needles
# --------------------------------------------------------------------------

def single_inputs(w: Workload, device="cpu", layers: Optional[Sequence[int]] = None,
                  seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """q [L,Hq,Nq,d], k and v [L,Hkv,N,d] for a single-shot workload.

    ``layers`` restricts generation to a subset of layers (the others are left
    as zeros), which lets a test rebuild a sampled unit cheaply.
    """
    s = w.shape
    seed = w.seed if seed is None else seed
    dt = storage_dtype(s)
    L, Hq, Hkv, d, N = s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache
    G = s.group
    Nq = s.n_queries
    q = torch.zeros(L, Hq, Nq, d, dtype=dt, device=device)
    k = torch.zeros(L, Hkv, N, d, dtype=dt, device=device)
    v = torch.zeros(L, Hkv, N, d, dtype=dt, device=device)
    layer_ids = range(L) if layers is None else layers
    sqd = math.sqrt(d)

    if w.recipe == "tiny":
        for l in layer_ids:
            for gi in range(Hkv):
                g = _gen(device, seed, w.name, "k", l, gi)
                off = _outliers(d, 2, g, device, fixed=8.0)
                kk = torch.randn(N, d, generator=g, device=device) + off
                pos = s.n_sinks + torch.randperm(N - s.n_sinks, generator=g, device=device)[:16]
                nh = _unit(torch.randn(16, d, generator=g, device=device))
                kk[pos] = sqd * nh + off
                k[l, gi] = _store(kk, dt)
                gv = _gen(device, seed, w.name, "v", l, gi)
                v[l, gi] = _store(torch.randn(N, d, generator=gv, device=device), dt)
                for t in range(G):
                    h = gi * G + t
                    gq = _gen(device, seed, w.name, "q", l, h)
                    qq = torch.randn(Nq, d, generator=gq, device=device)
                    n_al = min(32, Nq)
                    base = nh[torch.arange(n_al, device=device) % 16]
                    u = _orth_unit(base, torch.randn(n_al, d, generator=gq, device=device))
                    qq[:n_al] = sqd * (0.8 * base + 0.6 * u)
                    q[l, h] = _store(qq, dt)
        return {"q": q, "k": k, "v": v}

    if w.recipe in ("reconstruct", "reconstruct_needles"):
        needles = needle_positions(N, s.n_sinks) if w.recipe == "reconstruct_needles" else None
        src = _sources(s, seed, w.name, needles).to(device)      # [R, nq]
        src_flat = src.reshape(-1)                                 # [Nq]
        for l in layer_ids:
            for gi in range(Hkv):
                g = _gen(device, seed, w.name, "k", l, gi)
                off = _outliers(d, 4, g, device)
                kk = torch.randn(N, d, generator=g, device=device) + off
                if needles is not None:
                    nd = needles.to(device)
                    centres = _unit(torch.randn(10, d, generator=g, device=device))
                    span_id = torch.div(torch.arange(nd.numel(), device=device) * 10,
                                        nd.numel(), rounding_mode="floor")
                    kk[nd] = (sqd * centres[span_id]
                              + 0.3 * torch.randn(nd.numel(), d, generator=g, device=device) + off)
                kq = _store(kk, dt)
                k[l, gi] = kq
                gv = _gen(device, seed, w.name, "v", l, gi)
                v[l, gi] = _store(torch.randn(N, d, generator=gv, device=device), dt)
                ksrc = _unit(kq[src_flat].float())
                for t in range(G):
                    h = gi * G + t
                    gq = _gen(device, seed, w.name, "q", l, h)
                    u = _orth_unit(ksrc, torch.randn(Nq, d, generator=gq, device=device))
                    q[l, h] = _store(sqd * (0.6 * ksrc + 0.8 * u), dt)
        return {"q": q, "k": k, "v": v, "sources": src}

    raise ValueError(f"recipe {w.recipe!r} is not a single-shot recipe")


# --------------------------------------------------------------------------
# topic-clustered caches: the block loop and the episodic workload
# --------------------------------------------------------------------------

def _topic_keys(w: Workload, l: int, gi: int, n_tokens: int, topics: torch.Tensor,
                device, seed: int):
    s = w.shape
    d = s.head_dim
    g = _gen(device, seed, w.name, "k", l, gi)
    mu = 0.5 * torch.randn(4, d, generator=g, device=device)
    off = _outliers(d, 4, g, device)
    kk = mu[topics.to(device)] + torch.randn(n_tokens, d, generator=g, device=device) + off
    return kk, mu


def block_loop_inputs(w: Workload, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Token stream and per-step patched-prompt queries for the block loop.

    k_tokens, v_tokens: [L, Hkv, n_blocks*block_len, d]; block b is rows
    [b*block_len, (b+1)*block_len).
    q_steps: [n_blocks, L, Hq, nq, d]; the queries appended after block b.
    """
    s = w.shape
    seed = w.seed if seed is None else seed
    dt = storage_dtype(s)
    L, Hq, Hkv, d = s.layers, s.q_heads, s.kv_heads, s.head_dim
    G = s.group
    T = w.n_blocks * w.block_len
    nq = s.q_per_chunk
    topics = _topics(T, 4, seed, w.name)
    k = torch.empty(L, Hkv, T, d, dtype=dt, device=device)
    v = torch.empty(L, Hkv, T, d, dtype=dt, device=device)
    q = torch.empty(w.n_blocks, L, Hq, nq, d, dtype=dt, device=device)
    for l in range(L):
        for gi in range(Hkv):
            kk, mu = _topic_keys(w, l, gi, T, topics, device, seed)
            k[l, gi] = _store(kk, dt)
            gv = _gen(device, seed, w.name, "v", l, gi)
            v[l, gi] = _store(torch.randn(T, d, generator=gv, device=device), dt)
            for t in range(G):
                h = gi * G + t
                for b in range(w.n_blocks):
                    gq = _gen(device, seed, w.name, "q", l, h, b)
                    q[b, l, h] = _store(mu[0] + torch.randn(nq, d, generator=gq, device=device), dt)
    return {"k_tokens": k, "v_tokens": v, "q_steps": q, "topics": topics}


def episodic_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                    layers: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Cache k, v [L,Hkv,N,d], per-episode queries [E,L,Hq,Nq,d], sensitivities [L]."""
    s = w.shape
    seed = w.seed if seed is None else seed
    dt = storage_dtype(s)
    L, Hq, Hkv, d, N = s.layers, s.q_heads, s.kv_heads, s.head_dim, s.n_cache
    G = s.group
    Nq = s.n_queries
    E = w.episodes
    topics = _topics(N, E, seed, w.name)
    k = torch.zeros(L, Hkv, N, d, dtype=dt, device=device)
    v = torch.zeros(L, Hkv, N, d, dtype=dt, device=device)
    q = torch.zeros(E, L, Hq, Nq, d, dtype=dt, device=device)
    layer_ids = range(L) if layers is None else layers
    for l in layer_ids:
        for gi in range(Hkv):
            kk, mu = _topic_keys(w, l, gi, N, topics, device, seed)
            k[l, gi] = _store(kk, dt)
            gv = _gen(device, seed, w.name, "v", l, gi)
            v[l, gi] = _store(torch.randn(N, d, generator=gv, device=device), dt)
            for t in range(G):
                h = gi * G + t
                for e in range(E):
                    gq = _gen(device, seed, w.name, "q", l, h, e)
                    q[e, l, h] = _store(mu[e] + torch.randn(Nq, d, generator=gq, device=device), dt)
    return {"k": k, "v": v, "q_episodes": q, "sens": sensitivities(w, seed), "topics": topics}


def sensitivities(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Per-layer sensitivities s_l ~ U[0.5, 1.5], float64 [L]."""
    seed = w.seed if seed is None else seed
    rs = np.random.Generator(np.random.Philox(_seed(seed, w.name, "sens")))
    return rs.uniform(0.5, 1.5, size=w.shape.layers)


# --------------------------------------------------------------------------
# layer-sensitivity calibration: keys of one sample from a full prefill and
# from a block-wise prefill
# --------------------------------------------------------------------------

def calibration_keys(shape: ScoreShape, n_tokens: int, seed: int = 0, device="cpu",
                     kv_row_stride: int = 0) -> Dict[str, torch.Tensor]:
    """k_full, k_block [L, Hkv, kv_row_stride or n_tokens, d] and drift [L].

    Full-prefill keys are Gaussian plus 4 outlier channels per (layer, KV
    head); the block-prefill keys of the same tokens add noise of a seeded
    per-layer size drift[l] ~ U[0.05, 0.8] (a fixed property of each layer).
    Rows past n_tokens (when a row stride is given) are zero.
    """
    dt = storage_dtype(shape)
    L, Hkv, d = shape.layers, shape.kv_heads, shape.head_dim
    rows = kv_row_stride or n_tokens
    rs = np.random.Generator(np.random.Philox(_seed(seed, "calib", "drift", L)))
    drift = rs.uniform(0.05, 0.8, size=L)
    kf = torch.zeros(L, Hkv, rows, d, dtype=dt, device=device)
    kb = torch.zeros(L, Hkv, rows, d, dtype=dt, device=device)
    for l in range(L):
        for gi in range(Hkv):
            g = _gen(device, seed, "calib", "k", l, gi, n_tokens, d)
            base = torch.randn(n_tokens, d, generator=g, device=device) + _outliers(d, 4, g, device)
            noise = torch.randn(n_tokens, d, generator=g, device=device)
            kf[l, gi, :n_tokens] = _store(base, dt)
            kb[l, gi, :n_tokens] = _store(base + float(drift[l]) * noise, dt)
    return {"k_full": kf, "k_block": kb, "drift": drift}


# --------------------------------------------------------------------------
# episode clustering: segment and question embeddings
# --------------------------------------------------------------------------

def episode_embeddings(n_segments: int, dim: int, episodes: int, seed: int = 0,
                       n_questions: int = 64, noise: float = 0.9) -> Dict[str, torch.Tensor]:
    """Unit-norm fp32 segment embeddings [n_segments, dim] of a conversation
    that drifts between `episodes` topics in runs of 2-12 segments, questions
    [n_questions, dim] about seeded topics, the true labels of both, and the
    initial centroids' row indices (the first segment of each topic's first
    run, so every cluster starts inside its topic)."""
    g = _gen("cpu", seed, "episodes", n_segments, dim, episodes)
    topics = _unit(torch.randn(episodes, dim, generator=g)) * math.sqrt(dim) / 8
    labels = torch.empty(n_segments, dtype=torch.int64)
    i = 0
    while i < n_segments:
        run = int(torch.randint(2, 13, (1,), generator=g))
        labels[i:i + run] = int(torch.randint(0, episodes, (1,), generator=g))
        i += run
    labels[:episodes] = torch.arange(episodes)     # every topic appears early
    x = _unit(topics[labels] + noise * torch.randn(n_segments, dim, generator=g) / 8)
    qlab = torch.randint(0, episodes, (n_questions,), generator=g)
    q = _unit(topics[qlab] + noise * torch.randn(n_questions, dim, generator=g) / 8)
    init = torch.tensor([int(torch.nonzero(labels == e)[0]) for e in range(episodes)])
    return {"x": x.float().contiguous(), "labels": labels, "q": q.float().contiguous(),
            "q_labels": qlab, "init_index": init}


# --------------------------------------------------------------------------
# inputs for the selection and compaction kernels in isolation
# --------------------------------------------------------------------------

def score_tensor(units: int, n: int, n_sinks: int, kind: str = "uniform", seed: int = 0,
                 device="cpu") -> torch.Tensor:
    """fp32 scores [units, n] in [0, 1] with a chosen tie structure.

    kind: "uniform" (continuous, ties improbable), "coarse" (values on a grid of
    17 levels, so ties are everywhere), "equal" (all identical), "narrow"
    (every value within a relative 2^-12 of 0.3: a few thousand distinct
    values, each repeated, all sharing their top 20 bits), "sparse"
    (mostly exact zeros with a few positives), "tiny" (values down to 1e-38,
    including denormals and zero).
    """
    g = _gen("cpu", seed, "scores", kind, units, n)
    if kind == "uniform":
        s = torch.rand(units, n, generator=g)
    elif kind == "coarse":
        s = torch.randint(0, 17, (units, n), generator=g).float() / 16.0
    elif kind == "equal":
        s = torch.full((units, n), 0.375)
    elif kind == "narrow":
        s = 0.3 * (1.0 + torch.rand(units, n, generator=g) * 2.0 ** -12)
    elif kind == "sparse":
        s = torch.rand(units, n, generator=g)
        s = torch.where(torch.rand(units, n, generator=g) < 0.97, torch.zeros_like(s), s)
    elif kind == "tiny":
        e = torch.randint(-149, 0, (units, n), generator=g).float()
        s = torch.pow(2.0, e) * (1 + torch.rand(units, n, generator=g))
        s = torch.where(torch.rand(units, n, generator=g) < 0.05, torch.zeros_like(s), s)
        s = s.clamp(max=1.0)
    else:
        raise ValueError(kind)
    s[:, :min(n_sinks, n)] = 1.0
    return s.to(device)


def kept_lists(units_per_layer: int, n: int, n_sinks: int, k_per_layer: Sequence[int],
               seed: int = 0, device="cpu") -> torch.Tensor:
    """Random ascending kept-index lists, packed layer after layer.

    Layer l contributes units_per_layer lists of k_per_layer[l] ascending
    positions, each starting with the sinks [0, n_sinks).
    """
    g = _gen("cpu", seed, "kept", units_per_layer, n, tuple(k_per_layer))
    out = []
    for kl in k_per_layer:
        for _ in range(units_per_layer):
            s0 = min(n_sinks, n)
            rest = torch.randperm(n - s0, generator=g)[: kl - s0] + s0
            idx, _ = torch.sort(torch.cat([torch.arange(s0), rest]))
            out.append(idx.to(torch.int32))
    if not out:
        return torch.empty(0, dtype=torch.int32, device=device)
    return torch.cat(out).to(device)
