/*
 * kvs.h: C ABI of libkvs, query-agnostic KV-cache eviction on MI355X (gfx950).
 *
 * The method (sources, cited by page title and section):
 *   - KV² summary, "KV²가 전체 문맥 재계산 없이 KV 캐시를 압축한다":
 *       "어떻게 동작하나": a few leading sink tokens are kept as they are; the
 *       rest of the prefilled cache is cut into chunks of size m, and each chunk
 *       owns a set of reconstruction queries.
 *       "무엇과 다른가": those queries are appended after the cache and attend
 *       the whole cache; the score of a position in chunk C_r is the largest
 *       attention any of C_r's queries pays to it; after every chunk is scored
 *       the sinks are pinned to the top score and the lowest entries are
 *       evicted down to the budget.
 *       "전제와 한계": serving needs the cache compacted per head, which a
 *       masking backend does not do.
 *   - EpiCache review, "[26'ICML] EpiCache":
 *       "방법: 3단계" (2) and Fig. 1(b): the history is read block by block and
 *       the cache is compressed back to a fixed budget after every block, using
 *       an episode's prompt as the scoring queries.
 *       "+α: 레이어별 예산 배분": sensitive layers get a larger share of the
 *       budget, with sharpness alpha.
 *
 * Conventions shared by every entry point:
 *   - Device tensors are caller-owned, row-major and contiguous unless a stride
 *     argument says otherwise, and 16-byte aligned.  The library keeps no
 *     pointer after a call returns and allocates no device memory; scratch
 *     space comes from a caller workspace sized by kvs_workspace_bytes().
 *   - Every device call only enqueues work on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream).  Outputs are valid once the stream
 *     has reached that point.  No call synchronises the device.
 *   - Return value: a kvs_status.  Arguments are validated before anything is
 *     enqueued; on any error other than KVS_E_HIP the outputs are untouched.
 *     KVS_E_HIP means a launch failed and the outputs are undefined.
 *   - Scores are fp32 in [0, 1]; kept positions are int32 and ascending within
 *     each (layer, KV head).
 */
#ifndef KVS_H_
#define KVS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest layer count the per-layer tables carry in kernel arguments. */
#define KVS_MAX_LAYERS 256

typedef enum kvs_status {
  KVS_OK = 0,
  KVS_E_NULL = 1,      /* a required pointer is NULL */
  KVS_E_SHAPE = 2,     /* sizes inconsistent or unsupported */
  KVS_E_DTYPE = 3,     /* element type not supported */
  KVS_E_BUDGET = 4,    /* a budget outside [n_sinks, n_cache], or bad sensitivities */
  KVS_E_ALIGN = 5,     /* a device pointer is not 16-byte aligned */
  KVS_E_WORKSPACE = 6, /* workspace smaller than kvs_workspace_bytes() */
  KVS_E_HIP = 7,       /* a HIP launch or runtime call failed */
  KVS_E_SCRATCH = 8    /* needs more than KVS_NOALLOC_SCRATCH_BYTES of scratch */
} kvs_status;

/* Scratch that kvs_compress_block_noalloc holds per GPU (64 MiB). */
#define KVS_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

typedef enum kvs_dtype {
  KVS_F32 = 0,  /* float32 queries and keys (scored with fp32 vector arithmetic) */
  KVS_BF16 = 1  /* bfloat16 queries and keys (scored on bf16 MFMA, fp32 accumulate) */
} kvs_dtype;

/*
 * One scoring problem.  L = layers, Hq / Hkv = query / KV heads (Hq a multiple
 * of Hkv, G = Hq/Hkv; query head h reads KV head h / G), d = head_dim in {64,128},
 * N = n_cache, S = n_sinks, m = chunk_size >= 1, nq = q_per_chunk >= 1.
 * Chunk r covers positions [S + r*m, min(S + (r+1)*m, N)) for
 * r < R = ceil((N - S) / m) (R = 0 when N <= S), and owns query rows
 * [r*nq, (r+1)*nq); the query tensor therefore has Nq = R*nq rows per head.
 *
 * Layouts:
 *   Q       [L, Hq, Nq, d]  of dtype
 *   K, V    [L, Hkv, kv_row_stride, d] of dtype; rows [0, N) of every
 *           (layer, KV head) slab are read.  kv_row_stride = 0 means N.
 *   scores  [L, Hkv, N] fp32
 *
 * Size limits (KVS_E_SHAPE otherwise): N <= 2^31 - 1; one (layer, KV head)
 * slab of keys, N * d * 4 bytes, and one KV head's query rows,
 * G * Nq * d * 4 bytes, each below 4 GiB (the kernels address them with
 * 32-bit offsets); every launch grid below 2^31 workgroups.
 */
typedef struct kvs_problem {
  int32_t layers;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t head_dim;
  int64_t n_cache;
  int64_t n_sinks;
  int64_t chunk_size;
  int64_t q_per_chunk;
  int64_t kv_row_stride;
  int32_t dtype;   /* kvs_dtype */
  int32_t flags;   /* reserved, must be 0 */
} kvs_problem;

/* Text for a status code (static storage; never NULL). */
const char* kvs_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int kvs_version(void);

/* Pure host check of a problem description; touches no device. */
int kvs_check_problem(const kvs_problem* p);

/* Number of chunks R and scoring queries per head Nq = R * nq (host only). */
int64_t kvs_num_chunks(const kvs_problem* p);
int64_t kvs_num_queries(const kvs_problem* p);

/* Bytes of device workspace kvs_score, kvs_select and kvs_compress_block need
 * for this problem (0 if the problem is invalid).  Host only.  On long caches
 * this includes the per-split statistics that let every pass-1 workgroup
 * stream at most 32K keys; a call given less workspace, but enough for the
 * plan without that cap, splits the keys less (scores equal up to rounding),
 * and a call given too little for that returns KVS_E_WORKSPACE. */
size_t kvs_workspace_bytes(const kvs_problem* p);

/*
 * Per-layer budgets (EpiCache review, "+α: 레이어별 예산 배분"), host only.
 * Writes k_out[l], the kept positions per KV head of layer l, sinks included.
 * With sens == NULL the split is uniform; otherwise layer l's share is
 * T * sens[l]^alpha / sum_j sens[j]^alpha.  Each layer gets the floor of its
 * share and the leftover units go one each to the largest fractional parts,
 * lower layer first on ties, so sum(k_out) == total exactly.
 * Errors: KVS_E_NULL (k_out), KVS_E_SHAPE (layers outside [1, KVS_MAX_LAYERS]),
 * KVS_E_BUDGET (total < 0, a sensitivity not finite and > 0, alpha not finite
 * and >= 0, or any k_out[l] outside [n_sinks, n_cache]).  k_out is written
 * only on success.
 */
int kvs_layer_budgets(int32_t layers, int64_t total, const double* sens, double alpha,
                      int64_t n_cache, int64_t n_sinks, int64_t* k_out);

/*
 * Scores (KV² summary, "무엇과 다른가"): for every (layer l, KV head g) and
 * position i of chunk r,
 *     scores[l,g,i] = max over heads h of group g and rows j of chunk r of
 *                     softmax_i'( q[l,h,j] . k[l,g,i'] / sqrt(d) )[i]
 * with the softmax over all N positions; sink positions i < S get 1.0.
 * q, k: device, per the layouts above.  scores: device [L, Hkv, N] fp32, fully
 * written.  ws: device workspace, kvs_workspace_bytes(p) bytes for the
 * planned key split (see there).
 */
int kvs_score(const kvs_problem* p, const void* q, const void* k, float* scores,
              void* ws, size_t ws_bytes, void* stream);

/*
 * Selection (KV² summary, "무엇과 다른가": evict the lowest to the budget).
 * For each (l, g) keeps [0, S) plus the k_l - S positions of [S, N) that come
 * first in the order (score descending, position ascending), and writes them
 * ascending.  k_per_layer: HOST array [L] with S <= k_l <= N.
 * kept: device int32, packed layer after layer and head after head: the list
 * of (l, g) starts at Hkv * sum_{l'<l} k_l' + g * k_l and has k_l entries.
 * Scores compare as floats (-0 equals +0); every NaN, of either sign and any
 * payload, orders above +inf, and NaNs tie with each other (lower position first).
 * ws: device workspace of kvs_workspace_bytes(p) bytes, 256-byte aligned; it
 * is used (and then required, else KVS_E_NULL / KVS_E_WORKSPACE /
 * KVS_E_ALIGN) only when N - S exceeds 131072 candidates per (l, g).
 */
int kvs_select(const kvs_problem* p, const float* scores, const int64_t* k_per_layer,
               int32_t* kept, void* ws, size_t ws_bytes, void* stream);

/*
 * Headwise compaction (KV² summary, "전제와 한계"): copies row kept[.., t] of
 * each (l, g) slab of K and V to output row t of that slab, bit for bit.
 * kept: device int32 in kvs_select's packed layout.  An entry outside [0, N) is
 * skipped: its output row is left as it was.
 * k_per_layer: HOST [L].
 * k_out, v_out: device.  out_row_stride == 0: packed like kept (row
 * Hkv * sum_{l'<l} k_l' + g * k_l + t).  out_row_stride > 0: slab (l, g)
 * starts at row (l * Hkv + g) * out_row_stride (needs k_l <= out_row_stride).
 * The outputs must not overlap K or V.  Either k_out or v_out (not both) may
 * be NULL: that tensor is not compacted and its input may be NULL as well.
 */
int kvs_compact(const kvs_problem* p, const void* k, const void* v, const int32_t* kept,
                const int64_t* k_per_layer, void* k_out, void* v_out,
                int64_t out_row_stride, void* stream);

/*
 * One full compression of a prefilled cache: kvs_layer_budgets, kvs_score,
 * kvs_select and kvs_compact in sequence.  total_budget, sens and alpha are
 * as in kvs_layer_budgets (with n_cache = N); the chosen budgets are written
 * to the HOST array k_per_layer_out [L] when it is not NULL.  If
 * total_budget >= L * N every position is kept (the cache is copied through
 * and scores are still written).  scores, kept, k_out, v_out, out_row_stride
 * and ws are as in the calls above; kept needs Hkv * sum_l k_l entries.
 * v_out may be NULL: V is then neither read nor compacted, for a caller that
 * compacts it apart with kvs_compact or kvs_compact_seg (for example on a
 * second stream, beside the next step's scoring, which reads only K).
 */
int kvs_compress_block(const kvs_problem* p, const void* q, const void* k, const void* v,
                       int64_t total_budget, const double* sens, double alpha,
                       float* scores, int32_t* kept, void* k_out, void* v_out,
                       int64_t out_row_stride, int64_t* k_per_layer_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * kvs_compress_block for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as kvs_compress_block, minus
 * the workspace: the scratch the kernels need comes from a device array of
 * KVS_NOALLOC_SCRATCH_BYTES built into the library, one per GPU (the GPU of
 * `stream`, or the current device for a NULL stream), which that GPU holds
 * from the first call on it until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 * Returns KVS_E_SCRATCH, before touching the device, when even the scoring
 * plan without the key-stream cap (see kvs_workspace_bytes) needs more scratch
 * than that; the 131,072-token KV² shape of 36 layers x 32 query heads needs
 * about 60 MB that way.  kvs_compress_block given a larger workspace splits
 * pass 1's keys further, so the two agree bit for bit when kvs_compress_block
 * gets a workspace of KVS_NOALLOC_SCRATCH_BYTES. Every call on
 * one GPU shares its array and finds the previous call's contents there; the
 * kernels write everything they read from it first.  Calls that overlap on
 * one GPU (two streams, two threads) race on the array: serialise them.
 */
int kvs_compress_block_noalloc(const kvs_problem* p, const void* q, const void* k,
                               const void* v, int64_t total_budget, const double* sens,
                               double alpha, float* scores, int32_t* kept, void* k_out,
                               void* v_out, int64_t out_row_stride, int64_t* k_per_layer_out,
                               void* stream);

/*
 * The cache of one compression split in two buffers, as in the block-prefill
 * loop (EpiCache review, "방법: 3단계" (2), Fig. 1(b)) when the kept cache and
 * the newly prefilled block are scored together without first copying the
 * block behind the cache.  For every slab s = l * Hkv + g, cache row i is
 *   row s * head_row_stride + i of k_head / v_head          for i < head_rows,
 *   row s * tail_row_stride + tail_row0 + (i - head_rows)
 *                                  of k_tail / v_tail        for i >= head_rows.
 * Rows are head_dim elements of the problem's dtype; all four pointers are
 * device memory, 16-byte aligned, and are read only.
 */
typedef struct kvs_kv_segments {
  const void* k_head;
  const void* v_head;
  int64_t head_rows;
  int64_t head_row_stride;
  const void* k_tail;
  const void* v_tail;
  int64_t tail_row0;
  int64_t tail_row_stride;
} kvs_kv_segments;

/*
 * kvs_compress_block on a cache given as two segments (kvs_kv_segments).  The
 * results are those of kvs_compress_block on the concatenated cache, bit for
 * bit: the kept rows of both segments are gathered into k_out / v_out, which
 * must overlap none of the four inputs.  p->kv_row_stride must be 0 (the
 * strides come with the segments).  head_rows must lie in [0, N] and be a
 * multiple of 8 unless it equals N; head_row_stride >= head_rows when
 * head_rows > 0; tail_row0 >= 0 and tail_row_stride >= tail_row0 + N -
 * head_rows when head_rows < N.  Errors as kvs_compress_block, with
 * KVS_E_NULL for seg == NULL or a needed pointer and KVS_E_SHAPE for the
 * constraints above.
 */
int kvs_compress_block_seg(const kvs_problem* p, const void* q, const kvs_kv_segments* seg,
                           int64_t total_budget, const double* sens, double alpha,
                           float* scores, int32_t* kept, void* k_out, void* v_out,
                           int64_t out_row_stride, int64_t* k_per_layer_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * kvs_compact on a cache given as two segments (kvs_kv_segments, with the
 * constraints of kvs_compress_block_seg): the headwise compaction (KV²
 * summary, "전제와 한계") of the concatenated cache, bit for bit.  kept,
 * k_per_layer, out_row_stride and the NULL rules for k_out / v_out are those
 * of kvs_compact; only the segments' pointers of a compacted tensor are read.
 * Errors: as kvs_compact, and KVS_E_NULL for seg == NULL, KVS_E_SHAPE for
 * invalid segments.
 */
int kvs_compact_seg(const kvs_problem* p, const kvs_kv_segments* seg, const int32_t* kept,
                    const int64_t* k_per_layer, void* k_out, void* v_out,
                    int64_t out_row_stride, void* stream);

/*
 * Stage-1 query selection (KV² summary, "어떻게 동작하나"), also the selection
 * half of the refinement pass of "무엇과 다른가" when `scores` are stage-2
 * scores.  The token score of position i is the mean over layers and KV heads
 * of scores[l, g, i]; it is ranked by the float32 sum over the L * Hkv units in
 * layer-major order (same order as the mean, up to rounding).  Each chunk r of
 * p (positions [S + r*m, min(S + (r+1)*m, N))) keeps its
 *     n_q(r) = max(floor(rho * |C_r|), 1)
 * best positions (the product in IEEE double), ties to the lower position.
 *
 * kvs_query_counts (host only): n_q(r) for r < R into counts[R] and their sum
 *   into *total (either may be NULL).
 * kvs_query_select: scores device [L, Hkv, N] fp32 (e.g. kvs_score's output;
 *   q_heads, head_dim and q_per_chunk of p are not used but must be valid).
 *   positions: device int32, chunk after chunk, each chunk's n_q(r) positions
 *   ascending; chunk r starts at r * n_q of a full chunk, so the list has the
 *   total of kvs_query_counts entries.  ws: device workspace of at least
 *   kvs_query_workspace_bytes(p) bytes (the token sums).
 * Errors: KVS_E_SHAPE as kvs_check_problem; KVS_E_BUDGET for rho outside
 * (0, 1] or NaN; KVS_E_NULL, KVS_E_ALIGN (scores, positions 4-byte, ws
 * 256-byte aligned), KVS_E_WORKSPACE.  With no chunk (N <= S) nothing is
 * written.
 */
size_t kvs_query_workspace_bytes(const kvs_problem* p);
int kvs_query_counts(const kvs_problem* p, double rho, int64_t* counts, int64_t* total);
int kvs_query_select(const kvs_problem* p, const float* scores, double rho, int32_t* positions,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Global eviction (KV² summary, "무엇과 다른가": the chunks' local scores are
 * gathered into one global tensor, the sinks pinned to the top, and the
 * lowest entries evicted down to the target budget; "전제와 한계": each head
 * then keeps its own number of positions).  One budget over every (layer,
 * KV head, position): each unit u = l * Hkv + g keeps its sinks [0, S), and
 * the total_budget - L*Hkv*S best non-sink entries of the whole tensor, in the
 * order (score descending, unit ascending, position ascending), are kept too.
 *
 * kvs_select_global: scores device [L, Hkv, N] fp32.  kept: device int32
 *   [total_budget], unit after unit, each unit's positions ascending (sinks
 *   first).  offsets: device int64 [L*Hkv + 1]; unit u's list is
 *   kept[offsets[u] .. offsets[u+1]), offsets[0] = 0 and
 *   offsets[L*Hkv] = total_budget.  ws: device workspace of at least
 *   kvs_workspace_bytes(p) bytes, 256-byte aligned.
 * kvs_compact_ragged: copies row kept[t] of unit u's K and V slab (the
 *   layout of kvs_problem, kv_row_stride included) to row t of k_out / v_out
 *   ([total_rows, d] of the problem's dtype, must not overlap K or V), for
 *   every t in [offsets[u], offsets[u+1]).  kept and offsets as written by
 *   kvs_select_global with total_rows = offsets[L*Hkv]; an entry of kept
 *   outside [0, N) leaves its output row untouched.
 * kvs_compress_global: kvs_score, kvs_select_global and kvs_compact_ragged
 *   in sequence; one workspace serves all three.
 * Errors: as kvs_check_problem; KVS_E_SHAPE when L*Hkv*N exceeds 2^31 - 1
 * (device counts are 32-bit) or total_rows lies outside [0, L*Hkv*N];
 * KVS_E_BUDGET when total_budget lies outside [L*Hkv*min(S, N), L*Hkv*N];
 * KVS_E_NULL, KVS_E_ALIGN (kept 4-byte, offsets 8-byte, rows 16-byte, ws
 * 256-byte), KVS_E_WORKSPACE.
 */
int kvs_select_global(const kvs_problem* p, const float* scores, int64_t total_budget,
                      int32_t* kept, int64_t* offsets, void* ws, size_t ws_bytes, void* stream);
int kvs_compact_ragged(const kvs_problem* p, const void* k, const void* v, const int32_t* kept,
                       const int64_t* offsets, int64_t total_rows, void* k_out, void* v_out,
                       void* stream);
int kvs_compress_global(const kvs_problem* p, const void* q, const void* k, const void* v,
                        int64_t total_budget, float* scores, int32_t* kept, int64_t* offsets,
                        void* k_out, void* v_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode attention over a headwise-compacted cache with a different length
 * per head (KV² summary, "전제와 한계": serving needs an attention kernel that
 * accepts such a cache).  For every layer l and query head h, with unit
 * u = l * Hkv + h / G:
 *     out[l, h, :] = sum_j softmax_j(q[l, h] . k_out[j] / sqrt(d)) v_out[j, :]
 * over the rows j in [offsets[u], offsets[u+1]) of k_out / v_out; a unit with
 * no row gives zeros.  One new token per query head: q device [L, Hq, d] of
 * the problem's dtype; k_out, v_out device [rows, d] of that dtype (e.g.
 * kvs_compact_ragged's output); offsets device int64 [L*Hkv + 1],
 * non-decreasing, with sum of the row counts <= max_rows; out device fp32
 * [L, Hq, d].  Only layers, q_heads, kv_heads, head_dim and dtype of p are
 * used (the rest must still be valid).  A caller serving one layer at a time
 * passes a problem with layers = 1 and offsets + l * Hkv (offsets are
 * absolute row numbers).  ws: device workspace of at least
 * kvs_decode_workspace_bytes(p, max_rows) bytes, 256-byte aligned.
 * Errors: as kvs_check_problem; KVS_E_SHAPE (max_rows < 0 or a grid too
 * large), KVS_E_NULL, KVS_E_ALIGN (q, rows, out 16-byte, offsets 8-byte, ws
 * 256-byte), KVS_E_WORKSPACE.  Offsets that break the row-count bound give
 * unspecified values.
 */
size_t kvs_decode_workspace_bytes(const kvs_problem* p, int64_t max_rows);
int kvs_decode_ragged(const kvs_problem* p, const void* q, const void* k_out, const void* v_out,
                      const int64_t* offsets, int64_t max_rows, float* out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * Layer sensitivity calibration (EpiCache review, "+α: 레이어별 예산 배분" and
 * Fig. 4(a): a layer's keys move under block prefill by a layer-specific
 * amount, a property of the model measured on one calibration sample; layers
 * whose keys move more are more sensitive and get more budget).
 *
 * kvs_key_similarity: similarity[l] = mean over KV heads g and positions
 *   i < N of cos(k_full[l, g, i, :], k_block[l, g, i, :]), fp32 per row and
 *   a fixed-order float64 mean (a pair with a zero row counts as cosine 0;
 *   0 when N = 0).  k_full, k_block: device [L, Hkv, kv_row_stride, d] of the
 *   problem's dtype (keys of the same tokens from a full prefill and from a
 *   block-wise prefill).  similarity: device float64 [L].  Uses layers,
 *   kv_heads, head_dim, n_cache, kv_row_stride and dtype of p.  ws: device
 *   workspace of kvs_similarity_workspace_bytes(p) bytes, 256-byte aligned.
 *   Errors: as kvs_check_problem; KVS_E_NULL, KVS_E_WORKSPACE, KVS_E_ALIGN
 *   (keys 16-byte, similarity 8-byte, ws 256-byte), KVS_E_SHAPE (more than
 *   65535 slabs).
 * kvs_sensitivity (host only): sens[l] = 1 - similarity[l], the input of
 *   kvs_layer_budgets.  KVS_E_BUDGET if a similarity is not in [-1, 1].
 */
size_t kvs_similarity_workspace_bytes(const kvs_problem* p);
int kvs_key_similarity(const kvs_problem* p, const void* k_full, const void* k_block,
                       double* similarity, void* ws, size_t ws_bytes, void* stream);
int kvs_sensitivity(int32_t layers, const double* similarity, double* sens);

/*
 * Episode clustering and matching (EpiCache review, "방법: 3단계" (1) and (3),
 * Fig. 3(a) and (c): the history's segments are embedded and clustered by
 * K-means into E episodes, each represented by its medoid segment; a new
 * question's embedding picks the closest episode).  Embeddings are fp32 rows
 * of dim floats, dim a multiple of 4 in [4, 2048]; 1 <= clusters <= 16.
 *
 * kvs_kmeans: Lloyd's algorithm from init (device [clusters, dim]): `rounds`
 *   times, every point takes the centroid at the least squared Euclidean
 *   distance (ties to the lower one) and each centroid moves to the mean of
 *   its points (an empty cluster keeps its centroid); then one more
 *   assignment.  x: device [n, dim]; centroids: device [clusters, dim] out
 *   (may equal init); assign: device int32 [n] out.  ws: device workspace of
 *   kvs_kmeans_workspace_bytes(n, dim, clusters) bytes (needed when n > 0 and
 *   rounds > 0), 256-byte aligned.
 * kvs_medoids: totals[i] = sum of Euclidean distances from point i to the
 *   points of its cluster (device fp32 [n] out); medoid[e] = the member of
 *   cluster e with the least total, ties to the lower index, -1 if empty
 *   (device int32 [clusters] out).  assign: device int32 [n] in [0, clusters).
 *   A label outside [0, clusters) is not an error: such a point sums its
 *   distances to the points with the same label and belongs to no medoid.
 *   n <= 32 * 65535.  ws: device workspace of kvs_medoids_workspace_bytes(n,
 *   dim, clusters) bytes (about n * n / 8 + 8 n bytes: one partial sum per
 *   point and 32-point tile, and the points' order by cluster), 256-byte
 *   aligned.
 * kvs_match_episodes: episode[j] = the centroid nearest to query row j (as in
 *   the assignment), q: device [m, dim], episode: device int32 [m].
 * Errors: KVS_E_SHAPE (sizes above), KVS_E_NULL, KVS_E_ALIGN (rows 16-byte,
 * int32 arrays 4-byte, ws 256-byte), KVS_E_WORKSPACE.
 */
size_t kvs_kmeans_workspace_bytes(int64_t n, int64_t dim, int32_t clusters);
int kvs_kmeans(const float* x, int64_t n, int64_t dim, int32_t clusters, const float* init,
               int32_t rounds, float* centroids, int32_t* assign, void* ws, size_t ws_bytes,
               void* stream);
size_t kvs_medoids_workspace_bytes(int64_t n, int64_t dim, int32_t clusters);
int kvs_medoids(const float* x, int64_t n, int64_t dim, const int32_t* assign, int32_t clusters,
                int32_t* medoid, float* totals, void* ws, size_t ws_bytes, void* stream);
int kvs_match_episodes(const float* q, int64_t m, int64_t dim, const float* centroids,
                       int32_t clusters, int32_t* episode, void* stream);

/*
 * Block append for the block-prefill loop (EpiCache review, "방법: 3단계" (2),
 * Fig. 1(b)): for each of `slabs` (layer, KV head) slabs copies rows
 * [src_row0, src_row0 + n_rows) of src (slab stride src_row_stride rows) to
 * rows [dst_row0, dst_row0 + n_rows) of dst (slab stride dst_row_stride rows).
 * Rows are head_dim elements of dtype.  src and dst must not overlap.
 */
int kvs_append_rows(int32_t slabs, int32_t head_dim, int32_t dtype,
                    const void* src, int64_t src_row_stride, int64_t src_row0,
                    int64_t n_rows, void* dst, int64_t dst_row_stride, int64_t dst_row0,
                    void* stream);

/*
 * Per-kernel timing (tracing).  While enabled, each kernel launch the library
 * enqueues is bracketed by two HIP events on its stream; kvs_trace_summary
 * waits for those events and reports, per kernel name, the launch count and
 * total / min / max duration in milliseconds, then clears the record.  Events
 * are pooled, so steady-state tracing allocates nothing.  Disabled by default.
 */
typedef struct kvs_trace_entry {
  char name[48];
  int64_t count;
  double total_ms;
  double min_ms;
  double max_ms;
} kvs_trace_entry;

int kvs_trace_enable(int on);

/* Restricts recording to launches whose kernel name (as reported by
 * kvs_trace_summary, e.g. "score_pass1_bf16") equals `name`; NULL or "" records
 * every launch again.  The string is copied.  Always returns KVS_OK. */
int kvs_trace_only(const char* name);

/* Writes up to max_entries entries to out (host) and the number of distinct
 * kernels seen to *n_entries.  Blocks until the recorded events complete. */
int kvs_trace_summary(kvs_trace_entry* out, int max_entries, int* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H_ */
