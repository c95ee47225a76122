"""Python binding of the C ABI (include/kvs.h), one function per entry point.

Argument marshalling only: torch tensors become device pointers, host arrays
become ctypes arrays, the current torch stream becomes the hipStream_t, and a
nonzero status raises KvsError.  Every step of the computation runs in
libkvs.so's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Union

import numpy as np
import torch

from . import _lib
from ._lib import KVS_BF16, KVS_F32, KvsProblem

Tensorish = Union[torch.Tensor, int, None]


class KvsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib.lib().kvs_status_string(status).decode()
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)} ({text})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KvsError(status, where)


def _dev(x: Tensorish, name: str) -> Optional[int]:
    """Device pointer of a contiguous GPU tensor (or a raw int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _i64(vals: Optional[Sequence[int]]):
    if vals is None:
        return None
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def _f64(vals: Optional[Sequence[float]]):
    if vals is None:
        return None
    return (ctypes.c_double * len(vals))(*[float(v) for v in vals])


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KVS_BF16
    if t == torch.float32:
        return KVS_F32
    raise ValueError(f"unsupported dtype {t}")


def make_problem(layers: int, q_heads: int, kv_heads: int, head_dim: int, n_cache: int,
                 n_sinks: int, chunk_size: int, q_per_chunk: int, dtype: Union[int, torch.dtype],
                 kv_row_stride: int = 0) -> KvsProblem:
    if isinstance(dtype, torch.dtype):
        dtype = dtype_code(dtype)
    return KvsProblem(layers, q_heads, kv_heads, head_dim, n_cache, n_sinks, chunk_size,
                      q_per_chunk, kv_row_stride, dtype, 0)


# --- entry points, same names as the C ABI -------------------------------------

def kvs_status_string(status: int) -> str:
    return _lib.lib().kvs_status_string(status).decode()


def kvs_version() -> int:
    return _lib.lib().kvs_version()


def kvs_check_problem(p: KvsProblem) -> int:
    return _lib.lib().kvs_check_problem(ctypes.byref(p))


def kvs_num_chunks(p: KvsProblem) -> int:
    return _lib.lib().kvs_num_chunks(ctypes.byref(p))


def kvs_num_queries(p: KvsProblem) -> int:
    return _lib.lib().kvs_num_queries(ctypes.byref(p))


def kvs_workspace_bytes(p: KvsProblem) -> int:
    return int(_lib.lib().kvs_workspace_bytes(ctypes.byref(p)))


def kvs_layer_budgets(layers: int, total: int, sens: Optional[Sequence[float]], alpha: float,
                      n_cache: int, n_sinks: int) -> np.ndarray:
    out = (ctypes.c_int64 * layers)()
    _check(_lib.lib().kvs_layer_budgets(layers, total, _f64(sens), float(alpha), n_cache,
                                        n_sinks, out), "kvs_layer_budgets")
    return np.array(out[:], dtype=np.int64)


def kvs_score(p: KvsProblem, q: Tensorish, k: Tensorish, scores: Tensorish, ws: Tensorish,
              ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_score(ctypes.byref(p), _dev(q, "q"), _dev(k, "k"),
                                _dev(scores, "scores"), _dev(ws, "ws"), ws_bytes,
                                _stream(stream)), "kvs_score")


def _ws_or_new(p: KvsProblem, ws: Tensorish, ws_bytes: Optional[int], like: Tensorish):
    """The caller's workspace and its size, or a new one of kvs_workspace_bytes(p)."""
    if ws is None:
        ws = torch.empty(max(kvs_workspace_bytes(p), 256), dtype=torch.uint8,
                         device=like.device if isinstance(like, torch.Tensor) else "cuda")
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    return ws, ws_bytes


def kvs_select(p: KvsProblem, scores: Tensorish, k_per_layer: Sequence[int], kept: Tensorish,
               ws: Tensorish = None, ws_bytes: Optional[int] = None, stream=None) -> None:
    ws, ws_bytes = _ws_or_new(p, ws, ws_bytes, scores)
    _check(_lib.lib().kvs_select(ctypes.byref(p), _dev(scores, "scores"), _i64(k_per_layer),
                                 _dev(kept, "kept"), _dev(ws, "ws"), ws_bytes, _stream(stream)),
           "kvs_select")


def kvs_compact(p: KvsProblem, k: Tensorish, v: Tensorish, kept: Tensorish,
                k_per_layer: Sequence[int], k_out: Tensorish, v_out: Tensorish,
                out_row_stride: int = 0, stream=None) -> None:
    _check(_lib.lib().kvs_compact(ctypes.byref(p), _dev(k, "k"), _dev(v, "v"), _dev(kept, "kept"),
                                  _i64(k_per_layer), _dev(k_out, "k_out"), _dev(v_out, "v_out"),
                                  out_row_stride, _stream(stream)), "kvs_compact")


def kvs_compress_block(p: KvsProblem, q: Tensorish, k: Tensorish, v: Tensorish, total_budget: int,
                       sens: Optional[Sequence[float]], alpha: float, scores: Tensorish,
                       kept: Tensorish, k_out: Tensorish, v_out: Tensorish,
                       out_row_stride: int = 0, ws: Tensorish = None,
                       ws_bytes: Optional[int] = None, stream=None) -> np.ndarray:
    """Returns the per-layer budgets chosen on the host."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    kl = (ctypes.c_int64 * p.layers)()
    _check(_lib.lib().kvs_compress_block(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), total_budget, _f64(sens),
        float(alpha), _dev(scores, "scores"), _dev(kept, "kept"), _dev(k_out, "k_out"),
        _dev(v_out, "v_out"), out_row_stride, kl, _dev(ws, "ws"), ws_bytes, _stream(stream)),
        "kvs_compress_block")
    return np.array(kl[:], dtype=np.int64)


def kvs_compress_block_noalloc(p: KvsProblem, q: Tensorish, k: Tensorish, v: Tensorish,
                               total_budget: int, sens: Optional[Sequence[float]], alpha: float,
                               scores: Tensorish, kept: Tensorish, k_out: Tensorish,
                               v_out: Tensorish, out_row_stride: int = 0,
                               stream=None) -> np.ndarray:
    """kvs_compress_block with the library's own per-GPU scratch instead of a
    workspace (for callers that cannot allocate); returns the per-layer budgets."""
    kl = (ctypes.c_int64 * p.layers)()
    _check(_lib.lib().kvs_compress_block_noalloc(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), total_budget, _f64(sens),
        float(alpha), _dev(scores, "scores"), _dev(kept, "kept"), _dev(k_out, "k_out"),
        _dev(v_out, "v_out"), out_row_stride, kl, _stream(stream)),
        "kvs_compress_block_noalloc")
    return np.array(kl[:], dtype=np.int64)


def kvs_compress_block_seg(p: KvsProblem, q: Tensorish, k_head: Tensorish, v_head: Tensorish,
                           head_rows: int, head_row_stride: int, k_tail: Tensorish,
                           v_tail: Tensorish, tail_row0: int, tail_row_stride: int,
                           total_budget: int, sens: Optional[Sequence[float]], alpha: float,
                           scores: Tensorish, kept: Tensorish, k_out: Tensorish,
                           v_out: Tensorish, out_row_stride: int = 0, ws: Tensorish = None,
                           ws_bytes: Optional[int] = None, stream=None) -> np.ndarray:
    """kvs_compress_block on a cache held as two segments; returns the per-layer budgets."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    seg = _lib.KvsKvSegments(_dev(k_head, "k_head"), _dev(v_head, "v_head"), head_rows,
                             head_row_stride, _dev(k_tail, "k_tail"), _dev(v_tail, "v_tail"),
                             tail_row0, tail_row_stride)
    kl = (ctypes.c_int64 * p.layers)()
    _check(_lib.lib().kvs_compress_block_seg(
        ctypes.byref(p), _dev(q, "q"), ctypes.byref(seg), total_budget, _f64(sens),
        float(alpha), _dev(scores, "scores"), _dev(kept, "kept"), _dev(k_out, "k_out"),
        _dev(v_out, "v_out"), out_row_stride, kl, _dev(ws, "ws"), ws_bytes, _stream(stream)),
        "kvs_compress_block_seg")
    return np.array(kl[:], dtype=np.int64)


def kvs_compact_seg(p: KvsProblem, k_head: Tensorish, v_head: Tensorish, head_rows: int,
                    head_row_stride: int, k_tail: Tensorish, v_tail: Tensorish, tail_row0: int,
                    tail_row_stride: int, kept: Tensorish, k_per_layer: Sequence[int],
                    k_out: Tensorish, v_out: Tensorish, out_row_stride: int = 0,
                    stream=None) -> None:
    """kvs_compact on a cache held as two segments; k_out or v_out may be None."""
    seg = _lib.KvsKvSegments(_dev(k_head, "k_head"), _dev(v_head, "v_head"), head_rows,
                             head_row_stride, _dev(k_tail, "k_tail"), _dev(v_tail, "v_tail"),
                             tail_row0, tail_row_stride)
    _check(_lib.lib().kvs_compact_seg(ctypes.byref(p), ctypes.byref(seg), _dev(kept, "kept"),
                                      _i64(k_per_layer), _dev(k_out, "k_out"),
                                      _dev(v_out, "v_out"), out_row_stride, _stream(stream)),
           "kvs_compact_seg")


def kvs_query_workspace_bytes(p: KvsProblem) -> int:
    return int(_lib.lib().kvs_query_workspace_bytes(ctypes.byref(p)))


def kvs_query_counts(p: KvsProblem, rho: float) -> np.ndarray:
    """n_q of every chunk (host only)."""
    R = kvs_num_chunks(p)
    counts = (ctypes.c_int64 * max(R, 1))()
    total = ctypes.c_int64(0)
    _check(_lib.lib().kvs_query_counts(ctypes.byref(p), float(rho), counts, ctypes.byref(total)),
           "kvs_query_counts")
    return np.array(counts[:R], dtype=np.int64)


def kvs_query_select(p: KvsProblem, scores: Tensorish, rho: float, positions: Tensorish,
                     ws: Tensorish = None, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws is None:
        ws = torch.empty(max(kvs_query_workspace_bytes(p), 256), dtype=torch.uint8,
                         device=scores.device)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_query_select(ctypes.byref(p), _dev(scores, "scores"), float(rho),
                                       _dev(positions, "positions"), _dev(ws, "ws"), ws_bytes,
                                       _stream(stream)), "kvs_query_select")


def kvs_select_global(p: KvsProblem, scores: Tensorish, total_budget: int, kept: Tensorish,
                      offsets: Tensorish, ws: Tensorish = None, ws_bytes: Optional[int] = None,
                      stream=None) -> None:
    ws, ws_bytes = _ws_or_new(p, ws, ws_bytes, scores)
    _check(_lib.lib().kvs_select_global(ctypes.byref(p), _dev(scores, "scores"), int(total_budget),
                                        _dev(kept, "kept"), _dev(offsets, "offsets"),
                                        _dev(ws, "ws"), ws_bytes, _stream(stream)),
           "kvs_select_global")


def kvs_compact_ragged(p: KvsProblem, k: Tensorish, v: Tensorish, kept: Tensorish,
                       offsets: Tensorish, total_rows: int, k_out: Tensorish, v_out: Tensorish,
                       stream=None) -> None:
    _check(_lib.lib().kvs_compact_ragged(ctypes.byref(p), _dev(k, "k"), _dev(v, "v"),
                                         _dev(kept, "kept"), _dev(offsets, "offsets"),
                                         int(total_rows), _dev(k_out, "k_out"),
                                         _dev(v_out, "v_out"), _stream(stream)),
           "kvs_compact_ragged")


def kvs_compress_global(p: KvsProblem, q: Tensorish, k: Tensorish, v: Tensorish,
                        total_budget: int, scores: Tensorish, kept: Tensorish, offsets: Tensorish,
                        k_out: Tensorish, v_out: Tensorish, ws: Tensorish = None,
                        ws_bytes: Optional[int] = None, stream=None) -> None:
    ws, ws_bytes = _ws_or_new(p, ws, ws_bytes, k)
    _check(_lib.lib().kvs_compress_global(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), int(total_budget),
        _dev(scores, "scores"), _dev(kept, "kept"), _dev(offsets, "offsets"),
        _dev(k_out, "k_out"), _dev(v_out, "v_out"), _dev(ws, "ws"), ws_bytes, _stream(stream)),
        "kvs_compress_global")


def kvs_decode_workspace_bytes(p: KvsProblem, max_rows: int) -> int:
    return int(_lib.lib().kvs_decode_workspace_bytes(ctypes.byref(p), int(max_rows)))


def kvs_decode_ragged(p: KvsProblem, q: Tensorish, k_out: Tensorish, v_out: Tensorish,
                      offsets: Tensorish, max_rows: int, out: Tensorish, ws: Tensorish = None,
                      ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws is None:
        ws = torch.empty(max(kvs_decode_workspace_bytes(p, max_rows), 256), dtype=torch.uint8,
                         device=q.device)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_decode_ragged(ctypes.byref(p), _dev(q, "q"), _dev(k_out, "k_out"),
                                        _dev(v_out, "v_out"), _dev(offsets, "offsets"),
                                        int(max_rows), _dev(out, "out"), _dev(ws, "ws"),
                                        ws_bytes, _stream(stream)), "kvs_decode_ragged")


def kvs_similarity_workspace_bytes(p: KvsProblem) -> int:
    return int(_lib.lib().kvs_similarity_workspace_bytes(ctypes.byref(p)))


def kvs_key_similarity(p: KvsProblem, k_full: Tensorish, k_block: Tensorish,
                       similarity: Tensorish, ws: Tensorish = None,
                       ws_bytes: Optional[int] = None, stream=None) -> None:
    """similarity: a float64 GPU tensor of p.layers elements."""
    if ws is None:
        ws = torch.empty(max(kvs_similarity_workspace_bytes(p), 256), dtype=torch.uint8,
                         device=similarity.device)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_key_similarity(ctypes.byref(p), _dev(k_full, "k_full"),
                                         _dev(k_block, "k_block"), _dev(similarity, "similarity"),
                                         _dev(ws, "ws"), ws_bytes, _stream(stream)),
           "kvs_key_similarity")


def kvs_sensitivity(similarity: Sequence[float]) -> np.ndarray:
    """Host: 1 - similarity per layer."""
    n = len(similarity)
    out = (ctypes.c_double * n)()
    _check(_lib.lib().kvs_sensitivity(n, _f64(similarity), out), "kvs_sensitivity")
    return np.array(out[:], dtype=np.float64)


def kvs_kmeans_workspace_bytes(n: int, dim: int, clusters: int) -> int:
    return int(_lib.lib().kvs_kmeans_workspace_bytes(n, dim, clusters))


def kvs_kmeans(x: Tensorish, init: Tensorish, rounds: int, centroids: Tensorish,
               assign: Tensorish, ws: Tensorish = None, ws_bytes: Optional[int] = None,
               stream=None) -> None:
    """x [n, dim] and init [clusters, dim] fp32 GPU tensors; writes centroids and assign."""
    n, dim = x.shape
    clusters = init.shape[0]
    if ws is None:
        ws = torch.empty(max(kvs_kmeans_workspace_bytes(n, dim, clusters), 256),
                         dtype=torch.uint8, device=x.device)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_kmeans(_dev(x, "x"), n, dim, clusters, _dev(init, "init"), int(rounds),
                                 _dev(centroids, "centroids"), _dev(assign, "assign"),
                                 _dev(ws, "ws"), ws_bytes, _stream(stream)), "kvs_kmeans")


def kvs_medoids_workspace_bytes(n: int, dim: int, clusters: int) -> int:
    return int(_lib.lib().kvs_medoids_workspace_bytes(n, dim, clusters))


def kvs_medoids(x: Tensorish, assign: Tensorish, clusters: int, medoid: Tensorish,
                totals: Tensorish, ws: Tensorish = None, ws_bytes: Optional[int] = None,
                stream=None) -> None:
    n, dim = x.shape
    if ws is None:
        ws = torch.empty(max(kvs_medoids_workspace_bytes(n, dim, clusters), 256),
                         dtype=torch.uint8, device=x.device)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(_lib.lib().kvs_medoids(_dev(x, "x"), n, dim, _dev(assign, "assign"), clusters,
                                  _dev(medoid, "medoid"), _dev(totals, "totals"), _dev(ws, "ws"),
                                  ws_bytes, _stream(stream)), "kvs_medoids")


def kvs_match_episodes(q: Tensorish, centroids: Tensorish, episode: Tensorish,
                       stream=None) -> None:
    m, dim = q.shape
    _check(_lib.lib().kvs_match_episodes(_dev(q, "q"), m, dim, _dev(centroids, "centroids"),
                                         centroids.shape[0], _dev(episode, "episode"),
                                         _stream(stream)), "kvs_match_episodes")


def kvs_append_rows(slabs: int, head_dim: int, dtype: Union[int, torch.dtype], src: Tensorish,
                    src_row_stride: int, src_row0: int, n_rows: int, dst: Tensorish,
                    dst_row_stride: int, dst_row0: int, stream=None) -> None:
    if isinstance(dtype, torch.dtype):
        dtype = dtype_code(dtype)
    _check(_lib.lib().kvs_append_rows(slabs, head_dim, dtype, _dev(src, "src"), src_row_stride,
                                      src_row0, n_rows, _dev(dst, "dst"), dst_row_stride,
                                      dst_row0, _stream(stream)), "kvs_append_rows")


def workspace(p: KvsProblem, device="cuda") -> torch.Tensor:
    """A workspace tensor of kvs_workspace_bytes(p) bytes (at least 256)."""
    n = max(kvs_workspace_bytes(p), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def kvs_trace_enable(on: bool) -> None:
    _check(_lib.lib().kvs_trace_enable(1 if on else 0), "kvs_trace_enable")


def kvs_trace_only(name: Optional[str]) -> None:
    """Record only launches of kernel `name` (None: every launch)."""
    _check(_lib.lib().kvs_trace_only(name.encode() if name else None), "kvs_trace_only")


def kvs_trace_summary() -> dict:
    """{kernel name: {"count", "total_ms", "min_ms", "max_ms", "avg_ms"}}; clears the record."""
    cap = 64
    buf = (_lib.KvsTraceEntry * cap)()
    n = ctypes.c_int32(0)
    _check(_lib.lib().kvs_trace_summary(buf, cap, ctypes.byref(n)), "kvs_trace_summary")
    out = {}
    for e in buf[:min(n.value, cap)]:
        out[e.name.decode()] = {"count": e.count, "total_ms": e.total_ms, "min_ms": e.min_ms,
                                "max_ms": e.max_ms,
                                "avg_ms": e.total_ms / e.count if e.count else 0.0}
    return out
