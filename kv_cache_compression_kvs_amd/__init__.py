"""Query-agnostic KV-cache eviction on MI355X (gfx950): the Python binding of libkvs.

The computation lives in libkvs.so (HIP kernels behind the C ABI of
include/kvs.h); this package only marshals arguments and sequences calls.
"""
from ._lib import (KVS_BF16, KVS_F32, KvsKvSegments, KvsLibraryMissing,  # noqa: F401
                   KvsProblem, LIB_PATH)
from .api import (KvsError, kvs_append_rows, kvs_check_problem, kvs_compact,  # noqa: F401
                  kvs_compact_ragged, kvs_compact_seg, kvs_compress_block,
                  kvs_compress_block_noalloc, kvs_compress_block_seg,
                  kvs_compress_global, kvs_decode_ragged, kvs_decode_workspace_bytes,
                  kvs_key_similarity, kvs_kmeans, kvs_kmeans_workspace_bytes,
                  kvs_layer_budgets, kvs_match_episodes, kvs_medoids, kvs_medoids_workspace_bytes, kvs_select_global,
                  kvs_sensitivity, kvs_similarity_workspace_bytes,
                  kvs_num_chunks, kvs_num_queries, kvs_query_counts, kvs_query_select,
                  kvs_query_workspace_bytes, kvs_score, kvs_select, kvs_status_string,
                  kvs_trace_enable, kvs_trace_only, kvs_trace_summary, kvs_version,
                  kvs_workspace_bytes, make_problem, workspace)
