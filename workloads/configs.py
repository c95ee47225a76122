"""Workload shapes for query-agnostic KV-cache eviction.

Each configuration names a model shape (layers, query heads, KV heads, head
dimension), a cache length, the scoring-query layout (chunk size, queries per
chunk) and the budget rule.  Nothing here computes any part of the method; the
classes only hold sizes and derive the obvious counts (number of chunks,
total scoring queries) so that generators, tests and the benchmark agree on
them.

Sources of the shapes:
  * EpiCache review ("[26'ICML] EpiCache"), sections "방법: 3단계" (2) and
    "+α: 레이어별 예산 배분": block-wise prefill of 128-2048-token blocks with a
    fixed cache budget M, E=4 episodes, sensitivity^alpha layer budgets.
  * KV² summary ("KV²가 전체 문맥 재계산 없이 KV 캐시를 압축한다"), section
    "어떻게 동작하나": sinks, chunks of size m (4K by default), rho-fraction
    reconstruction queries per chunk.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class ScoreShape:
    """One scoring problem: a prefilled cache and the queries appended to it."""

    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    n_cache: int
    n_sinks: int
    chunk_size: int
    q_per_chunk: int
    dtype: str = "bf16"  # "bf16" or "f32"

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def n_chunks(self) -> int:
        if self.n_cache <= self.n_sinks:
            return 0
        return -(-(self.n_cache - self.n_sinks) // self.chunk_size)

    @property
    def n_queries(self) -> int:
        return self.n_chunks * self.q_per_chunk

    @property
    def units(self) -> int:
        return self.layers * self.kv_heads

    def scored_tokens(self) -> int:
        """Cache positions scored: layers x kv_heads x N."""
        return self.layers * self.kv_heads * self.n_cache

    def pass1_pairs(self) -> int:
        """(query head, query, key) triples of the full-cache normaliser pass."""
        return self.layers * self.q_heads * self.n_queries * self.n_cache

    def pass2_pairs(self) -> int:
        """(query head, query, key) triples restricted to each query's chunk."""
        total = 0
        for r in range(self.n_chunks):
            a = self.n_sinks + r * self.chunk_size
            b = min(a + self.chunk_size, self.n_cache)
            total += self.q_per_chunk * (b - a)
        return self.layers * self.q_heads * total

    def counted_flops(self) -> int:
        """2*d per (query, key) product, both passes, no tile padding."""
        return 2 * self.head_dim * (self.pass1_pairs() + self.pass2_pairs())

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named workload: a scoring shape plus the driver around it."""

    name: str
    kind: str                      # "single" | "block_loop" | "episodic"
    shape: ScoreShape              # for block_loop: the shape of one scoring step
    keep: Optional[int] = None     # kept positions per (layer, kv head), uniform budget
    keep_frac: Optional[float] = None
    # block loop
    block_len: int = 0
    n_blocks: int = 0
    budget_m: int = 0
    # episodic
    episodes: int = 0
    alpha: float = 0.0
    total_budget: int = 0
    # generator recipe knobs
    recipe: str = "gauss"
    seed: int = 0

    def keep_per_layer(self) -> int:
        if self.keep is not None:
            return self.keep
        if self.keep_frac is not None:
            return int(math.floor(self.keep_frac * self.shape.n_cache))
        return self.budget_m


# --- the five workloads at full size ----------------------------------------

TINY = Workload(
    name="tiny", kind="single",
    shape=ScoreShape(layers=1, q_heads=4, kv_heads=2, head_dim=64, n_cache=2048,
                     n_sinks=4, chunk_size=2048, q_per_chunk=128, dtype="f32"),
    keep=256, recipe="tiny")

# EpiCache-style block prefill, Llama-3.2-3B shape.  Each scoring step sees the
# kept cache (M rows) plus one new block and evicts back to M.
EPI_BLOCK = Workload(
    name="epicache_block_loop", kind="block_loop",
    shape=ScoreShape(layers=28, q_heads=24, kv_heads=8, head_dim=128,
                     n_cache=4096 + 2048, n_sinks=4, chunk_size=4096 + 2048,
                     q_per_chunk=256),
    block_len=2048, n_blocks=8, budget_m=4096, recipe="topics")

KV2_32K = Workload(
    name="kv2_32k", kind="single",
    shape=ScoreShape(layers=32, q_heads=32, kv_heads=8, head_dim=128, n_cache=32768,
                     n_sinks=4, chunk_size=4096, q_per_chunk=410),
    keep_frac=0.05, recipe="reconstruct")

KV2_131K = Workload(
    name="kv2_131k", kind="single",
    shape=ScoreShape(layers=36, q_heads=32, kv_heads=8, head_dim=128, n_cache=131072,
                     n_sinks=4, chunk_size=4096, q_per_chunk=410),
    keep_frac=0.02, recipe="reconstruct_needles")

# 90K tokens read as 90 x 1024 = 92,160 positions, one chunk covering the cache.
EPISODIC = Workload(
    name="episodic", kind="episodic",
    shape=ScoreShape(layers=28, q_heads=24, kv_heads=8, head_dim=128, n_cache=92160,
                     n_sinks=4, chunk_size=92160, q_per_chunk=512),
    episodes=4, alpha=3.0, total_budget=8192 * 28, recipe="topics")

FULL = {w.name: w for w in (TINY, EPI_BLOCK, KV2_32K, KV2_131K, EPISODIC)}


# --- reduced variants: same recipes, sizes the float64 oracle finishes in ----
# seconds, still spanning several kernel tiles and a ragged tail.

SMALL = {
    "tiny": TINY,
    "epicache_block_loop": Workload(
        name="epicache_block_loop_small", kind="block_loop",
        shape=ScoreShape(layers=2, q_heads=6, kv_heads=2, head_dim=128,
                         n_cache=1000 + 520, n_sinks=4, chunk_size=1000 + 520,
                         q_per_chunk=96),
        block_len=520, n_blocks=5, budget_m=1000, recipe="topics"),
    "kv2_32k": Workload(
        name="kv2_small", kind="single",
        shape=ScoreShape(layers=2, q_heads=8, kv_heads=2, head_dim=128, n_cache=4300,
                         n_sinks=4, chunk_size=1024, q_per_chunk=41),
        keep_frac=0.05, recipe="reconstruct"),
    "kv2_131k": Workload(
        name="kv2_needles_small", kind="single",
        shape=ScoreShape(layers=1, q_heads=8, kv_heads=2, head_dim=128, n_cache=9001,
                         n_sinks=4, chunk_size=2048, q_per_chunk=70),
        keep_frac=0.02, recipe="reconstruct_needles"),
    "episodic": Workload(
        name="episodic_small", kind="episodic",
        shape=ScoreShape(layers=4, q_heads=6, kv_heads=2, head_dim=128, n_cache=3333,
                         n_sinks=4, chunk_size=3333, q_per_chunk=80),
        episodes=4, alpha=3.0, total_budget=4 * 600, recipe="topics"),
}
