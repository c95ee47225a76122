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
            for before any compression.  Scoring reads only K, so with
            overlap_v each compression gathers K on the caller's stream and V
            on a second stream, where it overlaps the next step's scoring.
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
                 q_per_step: int, device="cuda", overlap_v: bool = False):
        self.L, self.Hq, self.Hkv, self.d = layers, q_heads, kv_heads, head_dim
        self.dtype = dtype
        self.B, self.M, self.S, self.nq = block_len, budget_m, n_sinks, q_per_step
        self.cap = budget_m + block_len
        shape = (layers, kv_heads, self.cap, head_dim)
        self.k = [torch.empty(shape, dtype=dtype, device=device) for _ in range(2)]
        self.v = [torch.empty(shape, dtype=dtype, device=device) for _ in range(2)]
        self.scores = torch.empty(layers * kv_heads * self.cap, dtype=torch.float32, device=device)
        # Two kept lists: the V gather of step b (second stream) still reads
        # one while step b + 1 selects into the other.
        self._kept = [torch.empty(layers * kv_heads * budget_m, dtype=torch.int32, device=device)
                      for _ in range(2)]
        self._kept_free: List[Optional[torch.cuda.Event]] = [None, None]
        self._ki = 0
        self.kept = self._kept[0]        # the latest compression's kept positions
        self.side = torch.cuda.Stream(device=device) if overlap_v else None
        self._v_done: Optional[torch.cuda.Event] = None
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
        self.join()
        self.cur = 0
        self.n = 0
        self._tok = None   # (k_tokens, v_tokens) while the cache is their rows [0, n)

    def join(self) -> None:
        """Makes the caller's stream wait for the V gathers in flight."""
        if self._v_done is not None:
            torch.cuda.current_stream().wait_event(self._v_done)
            self._v_done = None

    def _compress(self, compress_k: Callable, gather_v: Callable, nxt: int,
                  v_reads: Sequence[torch.Tensor] = ()) -> None:
        """One compression: compress_k(kept, v_out) scores, selects and gathers
        K (and V when v_out is given) on the caller's stream and returns the
        per-layer budgets; gather_v(kept, budgets) gathers V.  v_reads are the
        caller's tensors the V gather reads: with overlap_v they are marked as
        used on the second stream, so the caching allocator keeps their memory
        until that gather has finished even if the caller frees them first."""
        i = self._ki
        self._ki ^= 1
        kept = self._kept[i]
        main = torch.cuda.current_stream()
        if self._kept_free[i] is not None:   # the V gather that last read this list
            main.wait_event(self._kept_free[i])
        if self.side is None:
            compress_k(kept, self.v[nxt])
        else:
            kl = compress_k(kept, None)
            ready = torch.cuda.Event()
            ready.record(main)
            with torch.cuda.stream(self.side):
                self.side.wait_event(ready)
                for t in v_reads:
                    t.record_stream(self.side)
                gather_v(kept, kl)
                done = torch.cuda.Event()
                done.record(self.side)
            self._kept_free[i] = done
            self._v_done = done
        self.kept = kept

    def _materialize(self) -> None:
        """Copies a cache still held as token rows [0, n) into the cache buffer."""
        if self._tok is None:
            return
        self.join()
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
        self.join()
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
        that compression reads one strided segment and nothing is copied.

        With overlap_v the V gather of this step may still be reading v_tokens
        on the second stream when step() returns.  Freeing v_tokens is safe
        (its memory is not reused before the gather ends), but writing into it
        in place is not: call join() first."""
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
            self._compress(
                lambda kept, v_out: api.kvs_compress_block(
                    p, q_step, k_tokens, v_tokens, self.M * self.L, None, 0.0, self.scores,
                    kept, self.k[nxt], v_out, out_row_stride=self.cap, ws=self.ws),
                lambda kept, kl: api.kvs_compact(p, None, v_tokens, kept, kl, None, self.v[nxt],
                                                 out_row_stride=self.cap),
                nxt, (v_tokens,))
            self._tok = None
            self.cur = nxt
            self.n = self.M
            return True
        if self.n + nb > self.M and self.n % 8 == 0:
            p = self.problem(self.n + nb, row_stride=0)
            cur, n = self.cur, self.n
            self._compress(
                lambda kept, v_out: api.kvs_compress_block_seg(
                    p, q_step, self.k[cur], self.v[cur], n, self.cap, k_tokens, v_tokens, r0, T,
                    self.M * self.L, None, 0.0, self.scores, kept, self.k[nxt], v_out,
                    out_row_stride=self.cap, ws=self.ws),
                lambda kept, kl: api.kvs_compact_seg(
                    p, None, self.v[cur], n, self.cap, None, v_tokens, r0, T, kept, kl, None,
                    self.v[nxt], out_row_stride=self.cap),
                nxt, (v_tokens,))
            self.cur = nxt
            self.n = self.M
            return True
        self.join()   # the V buffer may still be written by the last V gather
        api.kvs_append_rows(slabs, self.d, self.dtype, k_tokens, T, r0, nb,
                            self.k[self.cur], self.cap, self.n)
        api.kvs_append_rows(slabs, self.d, self.dtype, v_tokens, T, r0, nb,
                            self.v[self.cur], self.cap, self.n)
        self.n += nb
        if self.n <= self.M:
            return False
        p = self.problem(self.n)
        cur = self.cur
        self._compress(
            lambda kept, v_out: api.kvs_compress_block(
                p, q_step, self.k[cur], self.v[cur], self.M * self.L, None, 0.0, self.scores,
                kept, self.k[nxt], v_out, out_row_stride=self.cap, ws=self.ws),
            lambda kept, kl: api.kvs_compact(p, None, self.v[cur], kept, kl, None, self.v[nxt],
                                             out_row_stride=self.cap),
            nxt)
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
        self.join()
        return scored

    def cache_view(self):
        """The current cache (k, v) [L, Hkv, n, d] where it lies: the cache
        buffer, or the token buffer's leading rows before any compression."""
        self.join()
        if self._tok is not None:
            return self._tok[0][:, :, :self.n], self._tok[1][:, :, :self.n]
        return self.k[self.cur][:, :, :self.n], self.v[self.cur][:, :, :self.n]

    def cache(self):
        """Views of the current cache in the cache buffer: (k, v) [L, Hkv, n, d]."""
        self.join()
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
