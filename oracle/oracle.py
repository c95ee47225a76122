"""Float64 CPU oracle for query-agnostic KV-cache eviction.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
GPU path is checked against.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the library and its Python
binding never do, and it imports nothing from them.

What it computes, step by step, with the passage each step follows:

  partition   KV² summary ("KV²가 전체 문맥 재계산 없이 KV 캐시를 압축한다"),
              section "어떻게 동작하나": the first few prompt tokens are sinks
              kept as they are; the rest of the cache is cut into consecutive
              chunks C_1..C_M of size m (the last one may be shorter).  Each
              chunk owns its own set of reconstruction queries.
  attention   same page, section "무엇과 다른가": the reconstruction queries are
              appended after the prefilled cache and attend the whole cache.
              The probability a query pays to cache position i is the softmax
              over all cached positions of q.k_i scaled by 1/sqrt(d) (the
              usual scaled dot product; the page names no scale).
  score       same section: a position i in chunk C_r is scored by the largest
              attention any of C_r's queries pays to it, so one query leaning
              on a token is enough to keep it.  With grouped-query attention
              the query heads sharing a KV head are pooled the same way (max).
  sinks       same section: after all chunks are scored the sink positions get
              the largest possible score (1.0, the top of a probability).
  budgets     EpiCache review ("[26'ICML] EpiCache"), section "+α: 레이어별 예산
              배분": more sensitive layers get a larger share of the cache
              budget, with sharpness alpha.  Read as k_l proportional to
              s_l^alpha with the integer total kept exact by largest remainder.
  select      KV² summary, "무엇과 다른가": the lowest-scoring entries are
              evicted down to the budget.  Ties go to the lower position, and
              the kept positions are listed in ascending order.
  compact     KV² summary, "전제와 한계": serving needs the cache physically
              compacted per head; the kept rows of K and V are copied out.
  block loop  EpiCache review, "방법: 3단계" (2) and Fig. 1(b): the history is
              read block by block and the cache is compressed back to the
              budget after every block, which bounds peak memory.
  episodes    EpiCache review, "방법: 3단계" (2) and Fig. 3(b): one compressed
              cache is built per episode from that episode's prompt queries.
  queries     KV² summary, "어떻게 동작하나" (stage 1, query selection): the
              per-(layer, KV head) scores of a token are averaged into one
              token score p_i (the page found the mean better than the max),
              and each chunk takes its n_q = max(floor(rho |C_r|), 1)
              best-scoring positions as its reconstruction queries; they need
              not be contiguous.  Section "무엇과 다른가": stage 2's scores
              have the same token granularity and can replace the stage-1
              proxy for another pass (refinement); this is that selection.
              Ties go to the lower position; each chunk's list is ascending.
  global      KV² summary, "무엇과 다른가": the chunks' local scores are gathered
              into one global tensor, the sinks pinned to the top, and the
              lowest entries evicted down to the target budget, so each head
              keeps its own number of positions ("전제와 한계": a headwise
              compacted cache with a different length per head).  Read as one
              budget over every (layer, KV head, position); ties by (score
              descending, unit l*Hkv + g ascending, position ascending).
  decode      KV² summary, "전제와 한계": serving needs an attention kernel
              that accepts a different compressed length per head.  One new
              query token per query head attends its KV head's kept rows with
              the usual scaled dot product; a head with no kept row yields 0.

  sensitivity EpiCache review, "+α: 레이어별 예산 배분" and Fig. 4(a): the keys
              a layer computes under block prefill differ from its full-prefill
              keys by a layer-specific amount, a property of the model that one
              calibration sample measures; the more a layer's keys move, the
              more sensitive it is.  Read as: similarity of layer l = mean over
              (KV head, position) of the cosine between the full-prefill and
              block-prefill key rows (a zero row has cosine 0), and sensitivity
              s_l = 1 - similarity_l (the page gives no formula).

  episodes    EpiCache review, "방법: 3단계" (1) and (3), Fig. 3(a) and (c): the
              history's segments are embedded and clustered by K-means into E
              episodes; each episode's medoid segment is its representative;
              a new question's embedding is matched to the closest episode.
              Read as Lloyd's algorithm with squared Euclidean distance from
              given initial centroids (ties to the lower cluster, an empty
              cluster keeps its centroid), a fixed number of rounds of
              (assign, update) followed by a final assignment; the medoid is
              the member with the least sum of Euclidean distances to the
              other members of its cluster (ties to the lower index); matching
              is the nearest centroid.

Every pin of these functions lives in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from functools import partial
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# partition (KV² summary, "어떻게 동작하나")
# ---------------------------------------------------------------------------

def chunk_bounds(n_cache: int, n_sinks: int, chunk_size: int) -> List[Tuple[int, int]]:
    """Half-open position ranges of the chunks that follow the sinks."""
    if chunk_size < 1:
        raise ValueError("chunk_size must be positive")
    bounds = []
    a = n_sinks
    while a < n_cache:
        b = min(a + chunk_size, n_cache)
        bounds.append((a, b))
        a = b
    return bounds


def query_rows(r: int, q_per_chunk: int) -> Tuple[int, int]:
    """Rows of the scoring-query tensor that belong to chunk r."""
    return r * q_per_chunk, (r + 1) * q_per_chunk


# ---------------------------------------------------------------------------
# attention of the appended queries over the whole cache ("무엇과 다른가")
# ---------------------------------------------------------------------------

def logits(q_rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Scaled dot products q.k / sqrt(d): [n_rows, N]."""
    d = keys.shape[-1]
    return (np.asarray(q_rows, np.float64) @ np.asarray(keys, np.float64).T) / math.sqrt(d)


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax, max-shifted for range only."""
    z = np.asarray(z, np.float64)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    return e / e.sum(axis=1, keepdims=True)


def attention_probs(q_rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Probability each query row pays to every cached key: [n_rows, N]."""
    return softmax_rows(logits(q_rows, keys))


# ---------------------------------------------------------------------------
# per-position score: chunk-restricted max over queries and grouped heads
# ---------------------------------------------------------------------------

def chunk_scores(q_group: np.ndarray, keys: np.ndarray, r: int, n_sinks: int,
                 chunk_size: int, q_per_chunk: int, row_block: int = 64) -> np.ndarray:
    """Scores of the positions of chunk r for one (layer, KV head).

    q_group: [G, Nq, d] the queries of the G heads that share this KV head.
    keys:    [N, d].
    Returns  [|C_r|]: max over heads and over chunk r's queries of the
    probability paid to each position of C_r (probabilities normalised over
    the whole cache).
    """
    n_cache = keys.shape[0]
    a, b = chunk_bounds(n_cache, n_sinks, chunk_size)[r]
    r0, r1 = query_rows(r, q_per_chunk)
    best = np.zeros(b - a, np.float64)
    for h in range(q_group.shape[0]):
        rows = q_group[h, r0:r1]
        for s0 in range(0, rows.shape[0], row_block):
            p = attention_probs(rows[s0:s0 + row_block], keys)
            best = np.maximum(best, p[:, a:b].max(axis=0))
    return best


def unit_scores(q_group: np.ndarray, keys: np.ndarray, n_sinks: int, chunk_size: int,
                q_per_chunk: int, row_block: int = 64, chunk_map=map) -> np.ndarray:
    """Scores of every position of one (layer, KV head): [N], sinks = 1.

    The chunks are independent; ``chunk_map(f, chunk_indices)`` evaluates f on
    each of them (the builtin map by default; a test may pass a parallel map,
    which changes nothing in what is computed)."""
    n_cache = keys.shape[0]
    bounds = chunk_bounds(n_cache, n_sinks, chunk_size)
    parts = list(chunk_map(partial(chunk_scores, q_group, keys, n_sinks=n_sinks,
                                   chunk_size=chunk_size, q_per_chunk=q_per_chunk,
                                   row_block=row_block), range(len(bounds))))
    s = np.zeros(n_cache, np.float64)
    for (a, b), part in zip(bounds, parts):
        s[a:b] = part
    s[:min(n_sinks, n_cache)] = 1.0
    return s


def kv_head_of(h: int, group: int) -> int:
    """Query head h reads KV head h // G (consecutive grouping)."""
    return h // group


def scores(q: np.ndarray, k: np.ndarray, n_sinks: int, chunk_size: int,
           q_per_chunk: int, units: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Scores [L, Hkv, N] for queries q [L, Hq, Nq, d] over keys k [L, Hkv, N, d].

    ``units`` restricts the work to a list of (layer, kv_head) pairs; the
    remaining entries are left at NaN.
    """
    L, Hq, _, _ = q.shape
    _, Hkv, N, _ = k.shape
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    G = Hq // Hkv
    out = np.full((L, Hkv, N), np.nan)
    todo = [(l, g) for l in range(L) for g in range(Hkv)] if units is None else units
    for (l, g) in todo:
        heads = [h for h in range(Hq) if kv_head_of(h, G) == g]
        qg = np.asarray(q[l, heads], np.float64)
        out[l, g] = unit_scores(qg, np.asarray(k[l, g], np.float64), n_sinks,
                                chunk_size, q_per_chunk)
    return out


# ---------------------------------------------------------------------------
# per-layer budgets (EpiCache review, "+α: 레이어별 예산 배분")
# ---------------------------------------------------------------------------

class BudgetError(ValueError):
    pass


def layer_budgets(total: int, n_layers: int, sens: Optional[Sequence[float]] = None,
                  alpha: float = 0.0, n_cache: Optional[int] = None,
                  n_sinks: int = 0) -> np.ndarray:
    """Kept positions per (layer, KV head) for each layer: int64 [L].

    Target shares t_l = T * s_l^alpha / sum_j s_j^alpha (uniform when sens is
    None).  Each layer gets floor(t_l); the T - sum floor(t) leftover units go
    one each to the layers with the largest fractional parts, lower layer
    first on equal parts.  A result outside [n_sinks, n_cache] is an error.
    """
    if n_layers < 1:
        raise BudgetError("need at least one layer")
    if total < 0:
        raise BudgetError("negative total budget")
    if sens is None:
        w = np.ones(n_layers, np.float64)
    else:
        s = np.asarray(sens, np.float64)
        if s.shape != (n_layers,) or not np.all(np.isfinite(s)) or np.any(s <= 0):
            raise BudgetError("sensitivities must be finite and positive, one per layer")
        if not (math.isfinite(alpha) and alpha >= 0):
            raise BudgetError("alpha must be finite and non-negative")
        w = np.array([float(x) ** float(alpha) for x in s])
    share = total * w / w.sum()
    base = np.floor(share).astype(np.int64)
    left = int(total - base.sum())
    frac = share - base
    order = sorted(range(n_layers), key=lambda l: (-frac[l], l))
    for l in order[:left]:
        base[l] += 1
    if n_cache is not None and (np.any(base < n_sinks) or np.any(base > n_cache)):
        raise BudgetError("a layer budget falls outside [n_sinks, n_cache]")
    return base


# ---------------------------------------------------------------------------
# selection (KV² summary, "무엇과 다른가": evict the lowest to the budget)
# ---------------------------------------------------------------------------

def select_unit(s: np.ndarray, k: int, n_sinks: int) -> np.ndarray:
    """Ascending kept positions: the sinks plus the k - S best of the rest.

    "Best" orders by score descending, then position ascending.
    """
    s = np.asarray(s, np.float64)
    n = s.shape[0]
    s0 = min(n_sinks, n)
    if not (s0 <= k <= n):
        raise BudgetError("budget must lie in [n_sinks, n_cache]")
    cand = np.arange(s0, n)
    order = np.lexsort((cand, -s[s0:]))          # primary: -score, then position
    chosen = cand[order[: k - s0]]
    return np.sort(np.concatenate([np.arange(s0), chosen])).astype(np.int64)


def select(score: np.ndarray, k_per_layer: Sequence[int], n_sinks: int) -> List[np.ndarray]:
    """Per layer an int64 array [Hkv, k_l] of kept positions."""
    L, Hkv, _ = score.shape
    return [np.stack([select_unit(score[l, g], int(k_per_layer[l]), n_sinks)
                      for g in range(Hkv)]) for l in range(L)]


def pack_kept(kept: List[np.ndarray]) -> np.ndarray:
    """Layer after layer, head after head: the flat kept-index layout."""
    return np.concatenate([x.reshape(-1) for x in kept]) if kept else np.zeros(0, np.int64)


# ---------------------------------------------------------------------------
# headwise compaction (KV² summary, "전제와 한계")
# ---------------------------------------------------------------------------

def compact(k: np.ndarray, v: np.ndarray, kept: List[np.ndarray]):
    """Per layer (K_out [Hkv, k_l, d], V_out [Hkv, k_l, d]): rows K[l, g, kept]."""
    outs = []
    for l, kl in enumerate(kept):
        ko = np.stack([np.take(k[l, g], kl[g], axis=0) for g in range(kl.shape[0])])
        vo = np.stack([np.take(v[l, g], kl[g], axis=0) for g in range(kl.shape[0])])
        outs.append((ko, vo))
    return outs


# ---------------------------------------------------------------------------
# one compression call and the two drivers
# ---------------------------------------------------------------------------

def compress(q, k, v, n_sinks: int, chunk_size: int, q_per_chunk: int,
             k_per_layer: Sequence[int]) -> Dict[str, object]:
    """Score, select and compact one cache."""
    sc = scores(q, k, n_sinks, chunk_size, q_per_chunk)
    kept = select(sc, k_per_layer, n_sinks)
    return {"scores": sc, "kept": kept, "out": compact(k, v, kept)}


def block_loop(k_tokens: np.ndarray, v_tokens: np.ndarray, q_steps: np.ndarray,
               block_len: int, budget_m: int, n_sinks: int,
               teacher: Optional[Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]]] = None):
    """EpiCache-style block prefill with compression after every block.

    k_tokens, v_tokens: [L, Hkv, T, d]; q_steps: [n_blocks, L, Hq, nq, d].
    After appending block b the cache holds n rows; if n exceeds the budget M
    it is scored with block b's queries (one chunk covering every non-sink
    position) and compacted back to M rows per (layer, KV head).

    Returns a list with one record per block: the cache it started from,
    the original token positions of each row, and (for scoring steps) the
    scores and kept positions.  ``teacher`` maps a block index to a cache
    (k, v, positions) that replaces the running cache before that block's
    append, so each step can be checked from a common starting point.
    """
    L, Hkv, T, d = k_tokens.shape
    n_blocks = q_steps.shape[0]
    ck = np.zeros((L, Hkv, 0, d), k_tokens.dtype)
    cv = np.zeros((L, Hkv, 0, d), v_tokens.dtype)
    pos = np.zeros((L, Hkv, 0), np.int64)
    recs = []
    for b in range(n_blocks):
        if teacher is not None and b in teacher:
            ck, cv, pos = teacher[b]
        a0, a1 = b * block_len, min((b + 1) * block_len, T)
        ck = np.concatenate([ck, k_tokens[:, :, a0:a1]], axis=2)
        cv = np.concatenate([cv, v_tokens[:, :, a0:a1]], axis=2)
        pos = np.concatenate([pos, np.broadcast_to(np.arange(a0, a1), (L, Hkv, a1 - a0))], axis=2)
        n = ck.shape[2]
        rec = {"block": b, "n_cache": n, "k": ck, "v": cv, "pos": pos}
        if n > budget_m:
            chunk = max(n - n_sinks, 1)
            sc = scores(q_steps[b], ck, n_sinks, chunk, q_steps.shape[3])
            kept = select(sc, [budget_m] * L, n_sinks)
            kk = np.stack(kept)                         # [L, Hkv, M]
            ck = np.take_along_axis(ck, kk[..., None], axis=2)
            cv = np.take_along_axis(cv, kk[..., None], axis=2)
            pos = np.take_along_axis(pos, kk, axis=2)
            rec.update(scores=sc, kept=kept)
        recs.append(rec)
    return recs


def episodic(k, v, q_episodes, sens, alpha: float, total: int, n_sinks: int,
             chunk_size: int, q_per_chunk: int):
    """One compressed cache per episode, each with sensitivity-split budgets."""
    L, _, N, _ = k.shape
    kl = layer_budgets(total, L, sens, alpha, n_cache=N, n_sinks=n_sinks)
    return kl, [compress(q_episodes[e], k, v, n_sinks, chunk_size, q_per_chunk, kl)
                for e in range(q_episodes.shape[0])]


# ---------------------------------------------------------------------------
# stage-1 query selection (KV² summary, "어떻게 동작하나"; the refinement pass
# of "무엇과 다른가" feeds it stage-2 scores)
# ---------------------------------------------------------------------------

def query_counts(n_cache: int, n_sinks: int, chunk_size: int, rho: float) -> List[int]:
    """n_q of every chunk: max(floor(rho * |C_r|), 1), the product in IEEE double."""
    if not (0.0 < rho <= 1.0):
        raise ValueError("rho must lie in (0, 1]")
    return [max(int(math.floor(rho * (b - a))), 1)
            for a, b in chunk_bounds(n_cache, n_sinks, chunk_size)]


def token_scores(score: np.ndarray) -> np.ndarray:
    """p_i: the mean over layers and KV heads of score[l, g, i]  ([L, Hkv, N] -> [N])."""
    s = np.asarray(score, np.float64)
    return s.reshape(-1, s.shape[-1]).mean(axis=0)


def select_queries(p: np.ndarray, n_cache: int, n_sinks: int, chunk_size: int,
                   rho: float) -> List[np.ndarray]:
    """Per chunk, ascending: the n_q positions of C_r with the largest p, ties to
    the lower position."""
    p = np.asarray(p)
    out = []
    for (a, b), nq in zip(chunk_bounds(n_cache, n_sinks, chunk_size),
                          query_counts(n_cache, n_sinks, chunk_size, rho)):
        cand = np.arange(a, b)
        order = np.lexsort((cand, -p[a:b].astype(np.float64)))
        out.append(np.sort(cand[order[:nq]]).astype(np.int64))
    return out


# ---------------------------------------------------------------------------
# global eviction with ragged heads (KV² summary, "무엇과 다른가" and
# "전제와 한계") and decode attention over the result
# ---------------------------------------------------------------------------

def select_global(score: np.ndarray, total: int, n_sinks: int) -> List[np.ndarray]:
    """Per unit u = l * Hkv + g, the ascending kept positions: every sink, plus the
    total - U*S best non-sink entries of the whole tensor by (score desc, u, i)."""
    s = np.asarray(score, np.float64)
    L, H, N = s.shape
    U = L * H
    s0 = min(n_sinks, N)
    need = total - U * s0
    if not (0 <= need <= U * (N - s0)):
        raise BudgetError("total must lie in [units * n_sinks, units * n_cache]")
    flat = s.reshape(U, N)[:, s0:]
    uu, ii = np.meshgrid(np.arange(U), np.arange(s0, N), indexing="ij")
    order = np.lexsort((ii.ravel(), uu.ravel(), -flat.ravel()))[:need]
    chosen = np.zeros((U, N - s0), bool)
    chosen.ravel()[order] = True
    return [np.concatenate([np.arange(s0), s0 + np.nonzero(chosen[u])[0]]).astype(np.int64)
            for u in range(U)]


def pack_ragged(kept: List[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """The lists end to end, and offsets [U + 1] (unit u's list at offsets[u])."""
    counts = np.array([len(x) for x in kept], np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    flat = np.concatenate(kept).astype(np.int64) if kept else np.zeros(0, np.int64)
    return flat, offsets


def compact_ragged(k: np.ndarray, v: np.ndarray, kept: List[np.ndarray]):
    """K_out, V_out [sum k_u, d]: unit u's kept rows, unit after unit."""
    L, H, N, d = k.shape
    ks = [k[u // H, u % H][kept[u]] for u in range(L * H)]
    vs = [v[u // H, u % H][kept[u]] for u in range(L * H)]
    return (np.concatenate(ks) if ks else np.zeros((0, d)),
            np.concatenate(vs) if vs else np.zeros((0, d)))


def decode_attention(q: np.ndarray, k_out: np.ndarray, v_out: np.ndarray, offsets: np.ndarray,
                     kv_heads: int) -> np.ndarray:
    """o[l, h] = softmax_j(q[l, h] . k_j / sqrt(d)) v_j over the rows of KV head
    h // G of layer l in the ragged compacted cache ([L, Hq, d] -> [L, Hq, d])."""
    q = np.asarray(q, np.float64)
    L, Hq, d = q.shape
    G = Hq // kv_heads
    out = np.zeros((L, Hq, d))
    for l in range(L):
        for h in range(Hq):
            u = l * kv_heads + h // G
            a, b = int(offsets[u]), int(offsets[u + 1])
            if b == a:
                continue
            kr = np.asarray(k_out[a:b], np.float64)
            vr = np.asarray(v_out[a:b], np.float64)
            out[l, h] = softmax_rows((kr @ q[l, h] / math.sqrt(d))[None])[0] @ vr
    return out



# ---------------------------------------------------------------------------
# layer sensitivity from key similarity (EpiCache review, "+α: 레이어별 예산
# 배분" and Fig. 4(a))
# ---------------------------------------------------------------------------

def key_similarity(k_full: np.ndarray, k_block: np.ndarray) -> np.ndarray:
    """[L]: mean over (KV head, position) of cos(k_full row, k_block row); a
    pair with a zero row counts as cosine 0.  Inputs [L, Hkv, N, d]."""
    a = np.asarray(k_full, np.float64)
    b = np.asarray(k_block, np.float64)
    L = a.shape[0]
    out = np.zeros(L)
    for l in range(L):
        dot = np.sum(a[l] * b[l], axis=-1)
        na = np.sqrt(np.sum(a[l] * a[l], axis=-1))
        nb = np.sqrt(np.sum(b[l] * b[l], axis=-1))
        den = na * nb
        cos = np.where(den > 0, dot / np.where(den > 0, den, 1.0), 0.0)
        out[l] = cos.mean() if cos.size else 0.0
    return out


def sensitivity(similarity: np.ndarray) -> np.ndarray:
    """s_l = 1 - similarity_l: layers whose keys move more under block prefill
    are more sensitive to compression."""
    return 1.0 - np.asarray(similarity, np.float64)


# ---------------------------------------------------------------------------
# episode clustering and matching (EpiCache review, "방법: 3단계" (1) and (3))
# ---------------------------------------------------------------------------

def nearest_centroid(x: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Index of the centroid at the least squared Euclidean distance from each
    row of x, ties to the lower index."""
    x = np.asarray(x, np.float64)
    c = np.asarray(centroids, np.float64)
    d2 = ((x[:, None, :] - c[None, :, :]) ** 2).sum(-1)
    return np.argmin(d2, axis=1).astype(np.int64)


def kmeans(x: np.ndarray, init: np.ndarray, rounds: int) -> Tuple[np.ndarray, np.ndarray]:
    """Lloyd's algorithm: `rounds` times assign every point to its nearest
    centroid and move each centroid to the mean of its points (an empty
    cluster keeps its centroid); then assign once more.  Returns (centroids,
    assignment)."""
    x = np.asarray(x, np.float64)
    c = np.array(init, np.float64)
    for _ in range(rounds):
        a = nearest_centroid(x, c)
        for e in range(c.shape[0]):
            members = x[a == e]
            if len(members):
                c[e] = members.mean(axis=0)
    return c, nearest_centroid(x, c)


def medoids(x: np.ndarray, assign: np.ndarray, clusters: int) -> np.ndarray:
    """Per cluster, the member whose summed Euclidean distance to the
    cluster's members is least (ties to the lower index); -1 for an empty
    cluster."""
    x = np.asarray(x, np.float64)
    assign = np.asarray(assign)
    out = np.full(clusters, -1, np.int64)
    for e in range(clusters):
        idx = np.nonzero(assign == e)[0]
        if len(idx) == 0:
            continue
        pts = x[idx]
        total = np.sqrt(((pts[:, None, :] - pts[None, :, :]) ** 2).sum(-1)).sum(1)
        out[e] = idx[int(np.argmin(total))]
    return out


def medoid_totals(x: np.ndarray, assign: np.ndarray) -> np.ndarray:
    """Each point's summed Euclidean distance to the members of its cluster."""
    x = np.asarray(x, np.float64)
    assign = np.asarray(assign)
    out = np.zeros(len(x))
    for i in range(len(x)):
        same = x[assign == assign[i]]
        out[i] = np.sqrt(((same - x[i]) ** 2).sum(-1)).sum()
    return out
