"""The two drivers of the eviction path, as sequences of C ABI calls.

BlockLoop   EpiCache review ("[26'ICML] EpiCache"), "방법: 3단계" (2) and
            Fig. 1(b): the history arrives block by block; each block is
            appended behind the kept cache and, once the cache exceeds the
            budget M, the episode prompt's queries score it and it is
            compressed back to M rows per (layer, KV head).  Two cache buffers
            of M + block rows alternate (ping-pong), so peak memory is fixed.
            A block that triggers a compression is read in place rather than
            copied behind the cache first, and so are the blocks before the
            first compression: until then the cache is the leading rows of
            the token buffer, copied into a cache buffer only if it is asked
            for before any compression.
episodic    EpiCache review, "방법: 3단계" (2) and Fig. 3(b), with the
            "+α: 레이어별 예산 배분" budget split: one compressed cache per
            episode, built from that episode's prompt queries.

Control flow only: every byte is moved and every score computed by libkvs.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

from . import api


class BlockLoop:
    """Ping-pong buffers and workspace for one block-prefill run."""

    def __init__(self, layers: int, q_heads: int, kv_heads: int, head_dim: int,
                 dtype: torch.dtype, block_len: int, budget_m: int, n_sinks: int,
                 q_per_step: int, device="cuda"):
        self.L, self.Hq, self.Hkv, self.d = layers, q_heads, kv_heads, head_dim
        self.dtype = dtype
        self.B, self.M, self.S, self.nq = block_len, budget_m, n_sinks, q_per_step
        self.cap = budget_m + block_len
        shape = (layers, kv_heads, self.cap, head_dim)
        self.k = [torch.empty(shape, dtype=dtype, device=device) for _ in range(2)]
        self.v = [torch.empty(shape, dtype=dtype, device=device) for _ in range(2)]
        self.scores = torch.empty(layers * kv_heads * self.cap, dtype=torch.float32, device=device)
        self.kept = torch.empty(layers * kv_heads * budget_m, dtype=torch.int32, device=device)
        self.ws = api.workspace(self.problem(self.cap), device)
        self.reset()

    def problem(self, n: int, row_stride: Optional[int] = None) -> api.KvsProblem:
        """The problem of one compression of an n-row cache whose rows lie
        row_stride apart per slab (None: the cache buffers' stride; 0: the
        cache is given in segments)."""
        chunk = max(n - self.S, 1)   # one chunk over every non-sink position
        stride = self.cap if row_stride is None else row_stride
        return api.make_problem(self.L, self.Hq, self.Hkv, self.d, n, self.S, chunk, self.nq,
                                self.dtype, kv_row_stride=stride)

    def reset(self) -> None:
        self.cur = 0
        self.n = 0
        self._tok = None   # (k_tokens, v_tokens) while the cache is their rows [0, n)

    def _materialize(self) -> None:
        """Copies a cache still held as token rows [0, n) into the cache buffer."""
        if self._tok is None:
            return
        kt, vt = self._tok
        self._tok = None
        if self.n:
            slabs, T = self.L * self.Hkv, kt.shape[2]
            api.kvs_append_rows(slabs, self.d, self.dtype, kt, T, 0, self.n, self.k[self.cur],
                                self.cap, 0)
            api.kvs_append_rows(slabs, self.d, self.dtype, vt, T, 0, self.n, self.v[self.cur],
                                self.cap, 0)

    def load_cache(self, k: torch.Tensor, v: torch.Tensor, n: int) -> None:
        """Sets the cache to the first n rows of k, v [L, Hkv, >= n, d]."""
        self._tok = None
        self.cur = 0
        self.n = n
        if n:
            self.k[0][:, :, :n] = k[:, :, :n]
            self.v[0][:, :, :n] = v[:, :, :n]

    def step(self, b: int, k_tokens: torch.Tensor, v_tokens: torch.Tensor,
             q_step: torch.Tensor) -> bool:
        """Append block b; compress if the cache exceeds M.  Returns True if scored.

        A block that fills the cache past M is not copied in: the compression
        reads the kept cache and the block where they lie (two segments) and
        gathers the kept rows of both into the other buffer.  Before the first
        compression the cache is rows [0, n) of the token buffer itself, so
        that compression reads one strided segment and nothing is copied."""
        T = k_tokens.shape[2]
        r0 = b * self.B
        nb = min(self.B, T - r0)
        slabs = self.L * self.Hkv
        nxt = 1 - self.cur
        if self._tok is not None and (self._tok[0] is not k_tokens or self._tok[1] is not v_tokens
                                      or r0 != self.n):
            self._materialize()
        if self._tok is None and self.n == 0 and r0 == 0:
            self._tok = (k_tokens, v_tokens)
        if self._tok is not None:
            if self.n + nb <= self.M:
                self.n += nb
                return False
            p = self.problem(self.n + nb, row_stride=T)
            api.kvs_compress_block(p, q_step, k_tokens, v_tokens, self.M * self.L, None, 0.0,
                                   self.scores, self.kept, self.k[nxt], self.v[nxt],
                                   out_row_stride=self.cap, ws=self.ws)
            self._tok = None
            self.cur = nxt
            self.n = self.M
            return True
        if self.n + nb > self.M and self.n % 8 == 0:
            p = self.problem(self.n + nb, row_stride=0)
            api.kvs_compress_block_seg(p, q_step, self.k[self.cur], self.v[self.cur], self.n,
                                       self.cap, k_tokens, v_tokens, r0, T, self.M * self.L,
                                       None, 0.0, self.scores, self.kept, self.k[nxt],
                                       self.v[nxt], out_row_stride=self.cap, ws=self.ws)
            self.cur = nxt
            self.n = self.M
            return True
        api.kvs_append_rows(slabs, self.d, self.dtype, k_tokens, T, r0, nb,
                            self.k[self.cur], self.cap, self.n)
        api.kvs_append_rows(slabs, self.d, self.dtype, v_tokens, T, r0, nb,
                            self.v[self.cur], self.cap, self.n)
        self.n += nb
        if self.n <= self.M:
            return False
        p = self.problem(self.n)
        api.kvs_compress_block(p, q_step, self.k[self.cur], self.v[self.cur],
                               self.M * self.L, None, 0.0, self.scores, self.kept,
                               self.k[nxt], self.v[nxt], out_row_stride=self.cap, ws=self.ws)
        self.cur = nxt
        self.n = self.M
        return True

    def run(self, k_tokens: torch.Tensor, v_tokens: torch.Tensor, q_steps: torch.Tensor,
            on_step: Optional[Callable[[int, "BlockLoop", bool], None]] = None) -> int:
        """All blocks; returns the number of scoring steps."""
        self.reset()
        scored = 0
        for b in range(q_steps.shape[0]):
            did = self.step(b, k_tokens, v_tokens, q_steps[b])
            scored += int(did)
            if on_step is not None:
                on_step(b, self, did)
        return scored

    def cache_view(self):
        """The current cache (k, v) [L, Hkv, n, d] where it lies: the cache
        buffer, or the token buffer's leading rows before any compression."""
        if self._tok is not None:
            return self._tok[0][:, :, :self.n], self._tok[1][:, :, :self.n]
        return self.k[self.cur][:, :, :self.n], self.v[self.cur][:, :, :self.n]

    def cache(self):
        """Views of the current cache in the cache buffer: (k, v) [L, Hkv, n, d]."""
        self._materialize()
        return self.k[self.cur][:, :, :self.n], self.v[self.cur][:, :, :self.n]


def episodic(k: torch.Tensor, v: torch.Tensor, q_episodes: torch.Tensor, sens: Sequence[float],
             alpha: float, total: int, n_sinks: int, chunk_size: int, q_per_chunk: int,
             outputs: Optional[List[dict]] = None) -> List[dict]:
    """One compressed cache per episode; returns dicts of output tensors."""
    L, Hkv, N, d = k.shape
    Hq = q_episodes.shape[2]
    p = api.make_problem(L, Hq, Hkv, d, N, n_sinks, chunk_size, q_per_chunk, k.dtype)
    kl = api.kvs_layer_budgets(L, total, sens, alpha, N, n_sinks)
    rows = int(Hkv * kl.sum())
    if outputs is None:
        ws = api.workspace(p, k.device)
        outputs = []
        for _ in range(q_episodes.shape[0]):
            outputs.append({
                "scores": torch.empty(L * Hkv * N, dtype=torch.float32, device=k.device),
                "kept": torch.empty(rows, dtype=torch.int32, device=k.device),
                "k": torch.empty(rows, d, dtype=k.dtype, device=k.device),
                "v": torch.empty(rows, d, dtype=k.dtype, device=k.device),
                "ws": ws,
            })
    for e, o in enumerate(outputs):
        got = api.kvs_compress_block(p, q_episodes[e], k, v, total, sens, alpha, o["scores"],
                                     o["kept"], o["k"], o["v"], 0, ws=o["ws"])
        o["k_per_layer"] = got
    return outputs


def split_packed(x: torch.Tensor, k_per_layer: Sequence[int], kv_heads: int) -> List[torch.Tensor]:
    """Per-layer views [Hkv, k_l, ...] of a tensor in the packed kept layout."""
    out, off = [], 0
    for kl in k_per_layer:
        n = kv_heads * int(kl)
        out.append(x[off:off + n].view(kv_heads, int(kl), *x.shape[1:]))
        off += n
    return out
