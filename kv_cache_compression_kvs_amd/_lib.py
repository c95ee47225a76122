"""ctypes loader for libkvs.so (the C ABI declared in include/kvs.h).

torch is imported before the library is opened: torch ships its own HIP
runtime with the same soname as /opt/rocm's, and loading torch first makes the
library bind to that one copy, so torch's streams and allocations are valid
handles for libkvs.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (see module docstring: must precede the CDLL load)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvs.so")

c_int32, c_int64, c_double, c_void_p, c_size_t = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                                  ctypes.c_void_p, ctypes.c_size_t)
P_I64 = ctypes.POINTER(ctypes.c_int64)
P_F64 = ctypes.POINTER(ctypes.c_double)

KVS_F32, KVS_BF16 = 0, 1
STATUS_NAMES = {0: "KVS_OK", 1: "KVS_E_NULL", 2: "KVS_E_SHAPE", 3: "KVS_E_DTYPE",
                4: "KVS_E_BUDGET", 5: "KVS_E_ALIGN", 6: "KVS_E_WORKSPACE", 7: "KVS_E_HIP",
                8: "KVS_E_SCRATCH"}


class KvsProblem(ctypes.Structure):
    """Mirror of struct kvs_problem."""
    _fields_ = [("layers", c_int32), ("q_heads", c_int32), ("kv_heads", c_int32),
                ("head_dim", c_int32), ("n_cache", c_int64), ("n_sinks", c_int64),
                ("chunk_size", c_int64), ("q_per_chunk", c_int64), ("kv_row_stride", c_int64),
                ("dtype", c_int32), ("flags", c_int32)]


class KvsKvSegments(ctypes.Structure):
    """Mirror of struct kvs_kv_segments."""
    _fields_ = [("k_head", c_void_p), ("v_head", c_void_p), ("head_rows", c_int64),
                ("head_row_stride", c_int64), ("k_tail", c_void_p), ("v_tail", c_void_p),
                ("tail_row0", c_int64), ("tail_row_stride", c_int64)]


class KvsTraceEntry(ctypes.Structure):
    """Mirror of struct kvs_trace_entry."""
    _fields_ = [("name", ctypes.c_char * 48), ("count", c_int64), ("total_ms", c_double),
                ("min_ms", c_double), ("max_ms", c_double)]


class KvsLibraryMissing(RuntimeError):
    pass


# name -> (restype, argtypes); one line per entry point of include/kvs.h
SIGNATURES = {
    "kvs_status_string": (ctypes.c_char_p, [c_int32]),
    "kvs_version": (c_int32, []),
    "kvs_check_problem": (c_int32, [ctypes.POINTER(KvsProblem)]),
    "kvs_num_chunks": (c_int64, [ctypes.POINTER(KvsProblem)]),
    "kvs_num_queries": (c_int64, [ctypes.POINTER(KvsProblem)]),
    "kvs_workspace_bytes": (c_size_t, [ctypes.POINTER(KvsProblem)]),
    "kvs_layer_budgets": (c_int32, [c_int32, c_int64, P_F64, c_double, c_int64, c_int64, P_I64]),
    "kvs_score": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p, c_void_p,
                            c_size_t, c_void_p]),
    "kvs_select": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, P_I64, c_void_p, c_void_p,
                             c_size_t, c_void_p]),
    "kvs_compact": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p, P_I64,
                              c_void_p, c_void_p, c_int64, c_void_p]),
    "kvs_compress_block": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p,
                                     c_int64, P_F64, c_double, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_int64, P_I64, c_void_p, c_size_t, c_void_p]),
    "kvs_compress_block_noalloc": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p,
                                             c_void_p, c_int64, P_F64, c_double, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_int64, P_I64,
                                             c_void_p]),
    "kvs_compress_block_seg": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p,
                                         ctypes.POINTER(KvsKvSegments), c_int64, P_F64, c_double,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_int64, P_I64,
                                         c_void_p, c_size_t, c_void_p]),
    "kvs_compact_seg": (c_int32, [ctypes.POINTER(KvsProblem), ctypes.POINTER(KvsKvSegments),
                                  c_void_p, P_I64, c_void_p, c_void_p, c_int64, c_void_p]),
    "kvs_query_workspace_bytes": (c_size_t, [ctypes.POINTER(KvsProblem)]),
    "kvs_query_counts": (c_int32, [ctypes.POINTER(KvsProblem), c_double, P_I64, P_I64]),
    "kvs_query_select": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_double, c_void_p,
                                   c_void_p, c_size_t, c_void_p]),
    "kvs_select_global": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_int64, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvs_compact_ragged": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_int64, c_void_p, c_void_p, c_void_p]),
    "kvs_compress_global": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p,
                                      c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
    "kvs_decode_workspace_bytes": (c_size_t, [ctypes.POINTER(KvsProblem), c_int64]),
    "kvs_decode_ragged": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvs_similarity_workspace_bytes": (c_size_t, [ctypes.POINTER(KvsProblem)]),
    "kvs_key_similarity": (c_int32, [ctypes.POINTER(KvsProblem), c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "kvs_sensitivity": (c_int32, [c_int32, P_F64, P_F64]),
    "kvs_kmeans_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int32]),
    "kvs_kmeans": (c_int32, [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_int32, c_void_p,
                             c_void_p, c_void_p, c_size_t, c_void_p]),
    "kvs_medoids_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int32]),
    "kvs_medoids": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_void_p,
                              c_void_p, c_size_t, c_void_p]),
    "kvs_match_episodes": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_int32, c_void_p,
                                     c_void_p]),
    "kvs_append_rows": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_int64, c_int64, c_int64,
                                  c_void_p, c_int64, c_int64, c_void_p]),
    "kvs_trace_enable": (c_int32, [c_int32]),
    "kvs_trace_only": (c_int32, [ctypes.c_char_p]),
    "kvs_trace_summary": (c_int32, [ctypes.POINTER(KvsTraceEntry), c_int32,
                                    ctypes.POINTER(c_int32)]),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises KvsLibraryMissing if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise KvsLibraryMissing(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m kv_cache_compression_kvs_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
        return _lib
