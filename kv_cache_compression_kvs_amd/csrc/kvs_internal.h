// Internal interface between the C ABI layer (kvs_api.cpp, pure host C++) and
// the HIP launchers (*.hip).  Nothing here is exported.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/kvs.h"

namespace kvs {

// Launch geometry and workspace layout of one kvs_score call.  Computed on the
// host from the problem and the workspace the call is given (the cap): the
// plan that kvs_workspace_bytes sizes for is the one with no cap, and a call
// with a smaller workspace gets the plan that fits it, if any.
struct ScorePlan {
  int64_t n_chunks = 0;       // R
  int64_t n_queries = 0;      // Nq = R * nq
  int64_t rows_per_unit = 0;  // G * Nq: the query rows that read one KV head
  int64_t total_rows = 0;     // L * Hq * Nq
  int64_t units = 0;          // L * Hkv
  int64_t row_blocks = 0;     // pass-1 workgroups along the rows of a unit
  int64_t splits = 1;         // pass-1 workgroups along the keys
  int64_t keys_per_split = 0; // multiple of the pass-1 key tile
  int64_t p2_tiles = 0;       // pass-2 key tiles per chunk
  size_t off_c2 = 0;          // workspace offsets (bytes)
  size_t off_pm = 0;
  size_t off_pl = 0;
  size_t ws_bytes = 0;
};

// Per-layer budget table carried in kernel arguments.
struct LayerTable {
  int32_t k[KVS_MAX_LAYERS];     // kept rows per (layer, KV head)
  int64_t off[KVS_MAX_LAYERS];   // Hkv * sum_{l' < l} k[l']
};

ScorePlan plan_score(const kvs_problem& p, size_t ws_cap = SIZE_MAX);

// Device address of the allocation-free scratch array on the GPU of `stream`
// (the current device when stream is NULL); KVS_OK or KVS_E_HIP.
int noalloc_scratch(void* stream, void** addr);

// Where the cached rows live.  Row i of slab s = l * Hkv + g is row
// s * head_stride + i of the head buffers for i < split, and row
// s * tail_stride + tail_row0 + (i - split) of the tail buffers otherwise.
// A single buffer is the case split = N (the tail is then never read).
struct KvSrc {
  const void* k_head = nullptr;
  const void* v_head = nullptr;
  int64_t head_stride = 0;
  const void* k_tail = nullptr;
  const void* v_tail = nullptr;
  int64_t tail_stride = 0;
  int64_t tail_row0 = 0;
  int64_t split = 0;
};

// Launchers.  Each returns 0 on success or a nonzero HIP error code.
int launch_score_bf16(const kvs_problem& p, const ScorePlan& pl, const void* q,
                      const KvSrc& kv, float* scores, void* ws, void* stream);
int launch_score_f32(const kvs_problem& p, const ScorePlan& pl, const void* q,
                     const KvSrc& kv, float* scores, void* ws, void* stream);
int launch_fill(float* dst, int64_t n, float value, void* stream);
int launch_select(const kvs_problem& p, const float* scores, const LayerTable& t,
                  int32_t* kept, void* ws, void* stream);
int launch_select_global(const kvs_problem& p, const float* scores, int64_t total,
                         int32_t* kept, int64_t* offsets, void* ws, void* stream);
int launch_query_select(const kvs_problem& p, const float* scores, double rho, int32_t* out,
                        float* psum, void* stream);
int launch_compact(const kvs_problem& p, const KvSrc& kv, const int32_t* kept,
                   const LayerTable& t, int32_t k_max, void* k_out, void* v_out,
                   int64_t out_row_stride, void* stream);
int launch_compact_ragged(const kvs_problem& p, const KvSrc& kv, const int32_t* kept,
                          const int64_t* offsets, int64_t total, void* k_out, void* v_out,
                          void* stream);
int launch_decode(const kvs_problem& p, const void* q, const void* k, const void* v,
                  const int64_t* offsets, int64_t max_rows, float* out, void* ws, void* stream);
int launch_similarity(const kvs_problem& p, const void* k_full, const void* k_block,
                      double* similarity, void* ws, void* stream);
size_t kmeans_ws_bytes(int64_t n, int64_t dim, int32_t clusters);
int launch_nearest(const float* x, int64_t n, int64_t dim, const float* centroids,
                   int32_t clusters, int32_t* out, void* stream);
int launch_kmeans(const float* x, int64_t n, int64_t dim, int32_t clusters, const float* init,
                  int32_t rounds, float* centroids, int32_t* assign, void* ws, void* stream);
size_t medoid_ws_bytes(int64_t n);
int launch_medoids(const float* x, int64_t n, int64_t dim, const int32_t* assign, int32_t clusters,
                   int32_t* medoid, float* totals, void* ws, void* stream);
int launch_append(int32_t slabs, int64_t row_bytes, const void* src, int64_t src_stride,
                  int64_t src_row0, int64_t n_rows, void* dst, int64_t dst_stride,
                  int64_t dst_row0, void* stream);

// Multi-workgroup radix select: candidates per workgroup, the largest
// per-unit candidate count the single-workgroup select handles, and the
// workspace it carves (per-unit mode for long caches, and the global mode).
constexpr int64_t kSelSpan = 4096;
constexpr int64_t kSelSingleMax = 32 * 1024;
// Per-unit selection of more candidates than this takes the one-workgroup
// streaming select (a sampled bracket and one read of the scores) instead of
// the LDS-resident radix select: measured on the 32K-token KV² shape (32,764
// candidates per unit), 35 against 69 microseconds per call.
constexpr int64_t kSelLongMin = 8 * 1024;
// Per-unit selection streams up to this many candidates per unit in one
// workgroup (bitmaps of them in LDS) and needs no workspace up to it.
constexpr int64_t kSelLongMax = 128 * 1024;

// Per-unit selection takes the multi-workgroup path (and the caller's
// workspace) beyond kSelLongMax candidates per unit.
inline bool select_uses_multi(const kvs_problem& p) {
  return p.n_cache - (p.n_sinks < p.n_cache ? p.n_sinks : p.n_cache) > kSelLongMax;
}

struct SelectWs {
  size_t off_hist = 0, off_state = 0, off_cnt = 0, off_before = 0, off_ekeep = 0, off_tot = 0;
  size_t bytes = 0;
};

inline SelectWs select_ws_layout(const kvs_problem& p) {
  auto r256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  const size_t units = (size_t)p.layers * (size_t)p.kv_heads;
  const int64_t nc = p.n_cache - (p.n_sinks < p.n_cache ? p.n_sinks : p.n_cache);
  const size_t nch = (size_t)((nc + kSelSpan - 1) / kSelSpan);
  SelectWs w;
  size_t off = 0;
  w.off_hist = off;
  off += r256(units * 8 * 256 * 4);  // one 256-bin histogram per XCD and segment
  w.off_state = off;
  off += r256(units * 16);
  w.off_cnt = off;
  off += r256(units * (nch ? nch : 1) * 8);
  w.off_before = off;
  off += r256(units * (nch ? nch : 1) * 8);
  w.off_ekeep = off;
  off += r256(units * 4);
  w.off_tot = off;
  off += r256(units * 8);
  w.bytes = off;
  return w;
}

// Decode over a ragged cache: rows per split workgroup, and the workspace
// (split prefix, per-split partial max / sum / accumulators) for at most
// max_rows kept rows in total.
constexpr int kDecodeRows = 512;

struct DecodeWs {
  int64_t slots = 0;  // split workgroups: ceil(max_rows / kDecodeRows) + units
  size_t off_sp = 0, off_ml = 0, off_acc = 0, bytes = 0;
};

DecodeWs decode_ws_layout(const kvs_problem& p, int64_t max_rows);

// Key similarity: rows of one slab per workgroup (its partial sum is one
// float of workspace).
constexpr int64_t kSimRows = 1024;

// Episode clustering limits: clusters per K-means and embedding width.
constexpr int kMaxClusters = 16;
constexpr int64_t kMaxEmbedDim = 2048;
constexpr int64_t kMaxMedoidPoints = 32 * 65535;  // 32-point tiles, grid y below 2^16

// Pass-1 tiling constants shared by the planner and the kernels.
constexpr int kP1Waves = 4;       // pass-1 waves per workgroup, 64 query rows each
constexpr int kP1Rows = kP1Waves * 64;  // query rows per pass-1 workgroup
constexpr int kP1Keys = 128;      // keys per pass-1 LDS tile
constexpr int kP1Ring = 2;        // pass-1 LDS tiles in flight
constexpr int kP2Waves = 4;       // pass-2 waves per workgroup, 64 keys each
constexpr int kP2Keys = kP2Waves * 64;  // keys per pass-2 workgroup
constexpr int kP2Ring = 3;        // pass-2 LDS query tiles in flight
constexpr int kMaxSplits = 64;
// Longest key stream of one pass-1 workgroup on long caches, when the
// workspace holds the per-split statistics that takes.  Measured at the KV²
// 131K shape: 4 splits of 32K keys cut pass 1's fetched bytes from 600 GB to
// 100-115 GB per launch (its row blocks stay closer in step in each L2) and
// its time by 0.3%, for 484 MB more workspace.
constexpr int64_t kP1StreamKeys = 32 * 1024;
constexpr int kP1Slots = 2048 / kP1Waves;  // resident pass-1 workgroups: 2 waves per SIMD, 1,024 SIMDs
// fp32 path: query rows per pass-1 workgroup (one wave each) and positions
// per pass-2 workgroup.
constexpr int kF32P1Rows = 4;
constexpr int kF32P2Keys = 64;

}  // namespace kvs
