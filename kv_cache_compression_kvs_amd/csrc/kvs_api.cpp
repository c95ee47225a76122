// C ABI of libkvs: argument validation, launch planning, per-layer budgets and
// dispatch to the HIP launchers.  Pure host C++; every check runs before any
// work is enqueued, so a rejected call leaves all outputs untouched.
#include <algorithm>
#include <cassert>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int64_t kMaxGrid = 0x7fffffffLL;
constexpr int kVersion = 10000;  // 1.0.0

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int64_t chunks_of(const kvs_problem& p) {
  if (p.n_cache <= p.n_sinks) return 0;
  return cdiv(p.n_cache - p.n_sinks, p.chunk_size);
}

int check(const kvs_problem* p) {
  if (!p) return KVS_E_NULL;
  if (p->layers < 1 || p->layers > KVS_MAX_LAYERS) return KVS_E_SHAPE;
  if (p->q_heads < 1 || p->kv_heads < 1 || p->q_heads % p->kv_heads) return KVS_E_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return KVS_E_SHAPE;
  if (p->n_cache < 0 || p->n_cache > INT32_MAX) return KVS_E_SHAPE;
  if (p->n_sinks < 0 || p->chunk_size < 1 || p->q_per_chunk < 1) return KVS_E_SHAPE;
  if (p->kv_row_stride != 0 && p->kv_row_stride < p->n_cache) return KVS_E_SHAPE;
  // one (layer, KV head) slab of keys is addressed with 32-bit byte offsets
  if (p->n_cache * p->head_dim * 4 >= (int64_t(1) << 32)) return KVS_E_SHAPE;
  if (p->dtype != KVS_F32 && p->dtype != KVS_BF16) return KVS_E_DTYPE;
  if (p->flags != 0) return KVS_E_SHAPE;
  // the scoring kernels index a chunk's rows (G * nq of them) in 32 bits
  if ((int64_t)(p->q_heads / p->kv_heads) * p->q_per_chunk >= (int64_t(1) << 31)) return KVS_E_SHAPE;
  const int64_t R = chunks_of(*p);
  const int64_t nq_total = R * p->q_per_chunk;
  if (R > 0 && nq_total / R != p->q_per_chunk) return KVS_E_SHAPE;
  // one KV head's query rows (G * R * nq of them) are addressed with 32-bit
  // byte offsets as well
  if (nq_total > INT32_MAX ||
      (int64_t)(p->q_heads / p->kv_heads) * nq_total * p->head_dim * 4 >= (int64_t(1) << 32))
    return KVS_E_SHAPE;
  const ScorePlan pl = plan_score(*p);
  // every launch grid must fit the 31-bit x dimension
  if (p->dtype == KVS_BF16 && pl.units * pl.splits * pl.row_blocks + 8 > kMaxGrid)
    return KVS_E_SHAPE;
  if (pl.units * pl.n_chunks * std::max<int64_t>(pl.p2_tiles, 1) + 8 > kMaxGrid) return KVS_E_SHAPE;
  if (pl.total_rows / 256 + 1 > kMaxGrid) return KVS_E_SHAPE;  // the split merge, one row per thread
  if (p->dtype == KVS_F32 && pl.row_blocks + 1 > kMaxGrid) return KVS_E_SHAPE;
  return KVS_OK;
}

int to_status(int hip_err) { return hip_err ? KVS_E_HIP : KVS_OK; }

// Largest-remainder split of `total` by sens^alpha (EpiCache review,
// "+α: 레이어별 예산 배분").  Returns a status; k is written only on success.
int budgets(int32_t L, int64_t total, const double* sens, double alpha, int64_t n_cache,
            int64_t n_sinks, int64_t* k) {
  if (!k) return KVS_E_NULL;
  if (L < 1 || L > KVS_MAX_LAYERS) return KVS_E_SHAPE;
  if (total < 0) return KVS_E_BUDGET;
  std::vector<double> w(L, 1.0);
  if (sens) {
    if (!std::isfinite(alpha) || alpha < 0) return KVS_E_BUDGET;
    for (int l = 0; l < L; ++l) {
      if (!std::isfinite(sens[l]) || !(sens[l] > 0)) return KVS_E_BUDGET;
      w[l] = std::pow(sens[l], alpha);
    }
  }
  double sum = 0;
  for (int l = 0; l < L; ++l) sum += w[l];
  if (!(sum > 0) || !std::isfinite(sum)) return KVS_E_BUDGET;
  std::vector<int64_t> base(L);
  std::vector<double> frac(L);
  int64_t used = 0;
  for (int l = 0; l < L; ++l) {
    const double share = (double)total * w[l] / sum;
    const double fl = std::floor(share);
    base[l] = (int64_t)fl;
    frac[l] = share - fl;
    used += base[l];
  }
  int64_t left = total - used;
  std::vector<int> order(L);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return frac[a] > frac[b]; });
  for (int i = 0; i < L && left > 0; ++i, --left) base[order[i]] += 1;
  if (left != 0) return KVS_E_BUDGET;  // only if rounding drifted by more than L
  for (int l = 0; l < L; ++l)
    if (base[l] < n_sinks || base[l] > n_cache) return KVS_E_BUDGET;
  std::memcpy(k, base.data(), sizeof(int64_t) * L);
  return KVS_OK;
}

int build_table(const kvs_problem& p, const int64_t* kpl, bool for_select, int64_t out_stride,
                LayerTable* t, int32_t* k_max) {
  if (!kpl) return KVS_E_NULL;
  const int64_t s_eff = std::min(p.n_sinks, p.n_cache);
  int64_t off = 0, mx = 0;
  for (int l = 0; l < p.layers; ++l) {
    const int64_t kl = kpl[l];
    if (kl < 0 || kl > p.n_cache) return KVS_E_BUDGET;
    if (for_select && kl < s_eff) return KVS_E_BUDGET;
    if (out_stride > 0 && kl > out_stride) return KVS_E_BUDGET;
    t->k[l] = (int32_t)kl;
    t->off[l] = off;
    off += (int64_t)p.kv_heads * kl;
    mx = std::max(mx, kl);
  }
  *k_max = (int32_t)mx;
  return KVS_OK;
}

// The single-buffer layout of K and V: rows [0, N) of each slab at stride
// kv_row_stride (0: N).
KvSrc single_src(const kvs_problem& p, const void* k, const void* v) {
  KvSrc kv;
  const int64_t stride = p.kv_row_stride ? p.kv_row_stride : p.n_cache;
  kv.k_head = k;
  kv.v_head = v;
  kv.head_stride = stride;
  kv.k_tail = k;
  kv.v_tail = v;
  kv.tail_stride = stride;
  kv.tail_row0 = p.n_cache;
  kv.split = p.n_cache;
  return kv;
}

// Shape checks of a two-segment cache (kvs_kv_segments) against p.
int check_segments(const kvs_problem& p, const kvs_kv_segments& seg) {
  const int64_t N = p.n_cache;
  const int64_t h = seg.head_rows;
  if (p.kv_row_stride != 0) return KVS_E_SHAPE;  // strides come with the segments
  if (h < 0 || h > N || (h % 8 != 0 && h != N)) return KVS_E_SHAPE;
  if (h > 0 && seg.head_row_stride < h) return KVS_E_SHAPE;
  if (h < N && (seg.tail_row0 < 0 || seg.tail_row_stride < seg.tail_row0 + (N - h)))
    return KVS_E_SHAPE;
  return KVS_OK;
}

KvSrc segment_src(const kvs_kv_segments& seg) {
  KvSrc kv;
  kv.k_head = seg.k_head;
  kv.v_head = seg.v_head;
  kv.head_stride = seg.head_row_stride;
  kv.k_tail = seg.k_tail;
  kv.v_tail = seg.v_tail;
  kv.tail_stride = seg.tail_row_stride;
  kv.tail_row0 = seg.tail_row0;
  kv.split = seg.head_rows;
  return kv;
}

// Null and alignment checks of the buffers a call reads (K if need_k, V if
// need_v).
int check_src(const kvs_problem& p, const KvSrc& kv, bool need_k, bool need_v) {
  if (p.n_cache == 0) return KVS_OK;
  const bool head = kv.split > 0, tail = kv.split < p.n_cache;
  if (need_k && ((head && !kv.k_head) || (tail && !kv.k_tail))) return KVS_E_NULL;
  if (need_v && ((head && !kv.v_head) || (tail && !kv.v_tail))) return KVS_E_NULL;
  if (need_k && ((head && !aligned(kv.k_head, 16)) || (tail && !aligned(kv.k_tail, 16))))
    return KVS_E_ALIGN;
  if (need_v && ((head && !aligned(kv.v_head, 16)) || (tail && !aligned(kv.v_tail, 16))))
    return KVS_E_ALIGN;
  return KVS_OK;
}

int do_score(const kvs_problem& p, const void* q, const KvSrc& kv, float* scores, void* ws,
             size_t ws_bytes) {
  const ScorePlan pl = plan_score(p, ws_bytes);
  if (p.n_cache > 0 && !scores) return KVS_E_NULL;
  if (int st = check_src(p, kv, true, false)) return st;
  if (pl.n_queries > 0 && !q) return KVS_E_NULL;
  if (pl.ws_bytes > 0 && !ws) return KVS_E_NULL;
  if (ws_bytes < pl.ws_bytes) return KVS_E_WORKSPACE;
  if ((q && !aligned(q, 16)) || (scores && !aligned(scores, 4)) || (ws && !aligned(ws, 256)))
    return KVS_E_ALIGN;
  return KVS_OK;
}

// The multi-workgroup select (long caches) needs the caller's workspace.
int check_select_ws(const kvs_problem& p, const void* ws, size_t ws_bytes) {
  if (!select_uses_multi(p)) return KVS_OK;
  if (!ws) return KVS_E_NULL;
  if (ws_bytes < select_ws_layout(p).bytes) return KVS_E_WORKSPACE;
  if (!aligned(ws, 256)) return KVS_E_ALIGN;
  return KVS_OK;
}

// Global eviction budget: every unit keeps its sinks, at most every position.
int check_global(const kvs_problem& p, int64_t total) {
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  if (units * p.n_cache > INT32_MAX) return KVS_E_SHAPE;  // counts are 32-bit on the device
  const int64_t s_eff = std::min(p.n_sinks, p.n_cache);
  if (total < units * s_eff || total > units * p.n_cache) return KVS_E_BUDGET;
  return KVS_OK;
}

// ws_bytes must be the size do_score accepted: the plan depends on it.
int enqueue_score(const kvs_problem& p, const void* q, const KvSrc& kv, float* scores, void* ws,
                  size_t ws_bytes, void* stream) {
  if (p.n_cache == 0) return KVS_OK;
  const ScorePlan pl = plan_score(p, ws_bytes);
  if (pl.n_chunks == 0)  // every position is a sink
    return to_status(launch_fill(scores, (int64_t)p.layers * p.kv_heads * p.n_cache, 1.0f, stream));
  if (p.dtype == KVS_BF16) return to_status(launch_score_bf16(p, pl, q, kv, scores, ws, stream));
  return to_status(launch_score_f32(p, pl, q, kv, scores, ws, stream));
}

// kvs_layer_budgets, kvs_score, kvs_select and kvs_compact in sequence, on a
// problem check() has accepted.
int compress(const kvs_problem& p, const void* q, const KvSrc& kv, int64_t total_budget,
             const double* sens, double alpha, float* scores, int32_t* kept, void* k_out,
             void* v_out, int64_t out_row_stride, int64_t* k_per_layer_out, void* ws,
             size_t ws_bytes, void* stream) {
  if (out_row_stride < 0) return KVS_E_SHAPE;
  std::vector<int64_t> kl(p.layers);
  int st;
  if (total_budget >= (int64_t)p.layers * p.n_cache) {
    std::fill(kl.begin(), kl.end(), p.n_cache);  // everything fits: copy through
  } else {
    st = budgets(p.layers, total_budget, sens, alpha, p.n_cache, p.n_sinks, kl.data());
    if (st) return st;
  }
  LayerTable t;
  int32_t kmax = 0;
  st = build_table(p, kl.data(), true, out_row_stride, &t, &kmax);
  if (st) return st;
  st = do_score(p, q, kv, scores, ws, ws_bytes);
  if (st) return st;
  if ((st = check_select_ws(p, ws, ws_bytes))) return st;
  if ((st = check_src(p, kv, true, v_out != nullptr))) return st;
  if (p.n_cache > 0 && (!kept || !k_out)) return KVS_E_NULL;
  if ((kept && !aligned(kept, 4)) || (k_out && !aligned(k_out, 16)) ||
      (v_out && !aligned(v_out, 16)))
    return KVS_E_ALIGN;
  if (k_per_layer_out) std::memcpy(k_per_layer_out, kl.data(), sizeof(int64_t) * p.layers);
  if (p.n_cache == 0) return KVS_OK;
  st = enqueue_score(p, q, kv, scores, ws, ws_bytes, stream);
  if (st) return st;
  st = to_status(launch_select(p, scores, t, kept, ws, stream));
  if (st) return st;
  if (kmax == 0) return KVS_OK;
  return to_status(launch_compact(p, kv, kept, t, kmax, k_out, v_out, out_row_stride, stream));
}

}  // namespace

namespace {

// Bytes of the scoring workspace: -c2/c1 per row, and (m, l) per row and split
// when the keys are split.  The layout below carves exactly this.
size_t score_ws_bytes(int64_t total_rows, int64_t splits) {
  size_t b = round256(sizeof(float) * (size_t)total_rows);
  if (splits > 1) b += 2 * round256(sizeof(float) * (size_t)total_rows * (size_t)splits);
  return b;
}

}  // namespace

ScorePlan plan_score(const kvs_problem& p, size_t ws_cap) {
  ScorePlan pl;
  const int64_t N = std::max<int64_t>(p.n_cache, 0);
  const int64_t Hkv = std::max(p.kv_heads, 1);
  const int64_t G = std::max<int64_t>(p.q_heads / Hkv, 1);
  pl.n_chunks = chunks_of(p);
  pl.n_queries = pl.n_chunks * std::max<int64_t>(p.q_per_chunk, 1);
  pl.rows_per_unit = G * pl.n_queries;
  pl.total_rows = (int64_t)p.layers * p.q_heads * pl.n_queries;
  pl.units = (int64_t)p.layers * p.kv_heads;
  if (pl.n_queries == 0 || N == 0) {
    pl.row_blocks = 0;
    pl.splits = 1;
    pl.keys_per_split = 0;
    pl.p2_tiles = 0;
    pl.ws_bytes = 0;
    return pl;
  }
  const int64_t chunk_len = std::min(p.chunk_size, N - std::min(p.n_sinks, N));
  if (p.dtype == KVS_BF16) {
    pl.row_blocks = cdiv(pl.rows_per_unit, kP1Rows);
    // Splitting the keys multiplies the workgroups; pick the split count that
    // best fills whole rounds of the resident slots (two pass-1 workgroups on
    // each of the 256 CUs) against a small cost per split (each split re-reads
    // its query rows and adds a merge).  Measured on the block-loop shape:
    // 3 splits (2,016 workgroups, 3.9 rounds) beat 2, 4, 6 and 8 by 3-5%.
    const int64_t base = pl.units * pl.row_blocks;
    const int64_t by_keys = std::max<int64_t>(1, cdiv(N, 4 * kP1Keys));
    const int64_t max_s = std::min<int64_t>({(int64_t)8, (int64_t)kMaxSplits, by_keys});
    int64_t splits = 1;
    double best = 0.0;
    for (int64_t sp = 1; sp <= max_s; ++sp) {
      const double wgs = (double)(base * sp);
      const double rounds = std::ceil(wgs / kP1Slots);
      const double cost = (1.0 + 0.3 * (rounds * kP1Slots / wgs - 1.0)) * (1.0 + 0.015 * (double)sp);
      if (sp == 1 || cost < best) {
        best = cost;
        splits = sp;
      }
    }
    // Long caches: at most kP1StreamKeys keys per workgroup, if the workspace
    // holds the statistics of that many splits.
    const int64_t by_stream = std::min<int64_t>(cdiv(N, kP1StreamKeys), kMaxSplits);
    if (by_stream > splits) {
      const int64_t kps = cdiv(cdiv(N, by_stream), kP1Keys) * kP1Keys;
      if (score_ws_bytes(pl.total_rows, cdiv(N, kps)) <= ws_cap) splits = by_stream;
    }
    pl.keys_per_split = cdiv(cdiv(N, splits), kP1Keys) * kP1Keys;
    pl.splits = cdiv(N, pl.keys_per_split);
    pl.p2_tiles = cdiv(chunk_len, kP2Keys);
  } else {
    pl.row_blocks = cdiv(pl.total_rows, kF32P1Rows);
    pl.splits = 1;
    pl.keys_per_split = N;
    pl.p2_tiles = cdiv(chunk_len, kF32P2Keys);
  }
  size_t off = 0;
  pl.off_c2 = off;
  off += round256(sizeof(float) * (size_t)pl.total_rows);
  pl.off_pm = off;
  pl.off_pl = off;
  if (pl.splits > 1) {
    off += round256(sizeof(float) * (size_t)pl.total_rows * (size_t)pl.splits);
    pl.off_pl = off;
    off += round256(sizeof(float) * (size_t)pl.total_rows * (size_t)pl.splits);
  }
  pl.ws_bytes = off;
  assert(pl.ws_bytes == score_ws_bytes(pl.total_rows, pl.splits));
  return pl;
}

}  // namespace kvs

using namespace kvs;

extern "C" {

const char* kvs_status_string(int status) {
  switch (status) {
    case KVS_OK: return "ok";
    case KVS_E_NULL: return "a required pointer is NULL";
    case KVS_E_SHAPE: return "sizes are inconsistent or unsupported";
    case KVS_E_DTYPE: return "element type is not supported";
    case KVS_E_BUDGET: return "a budget lies outside [n_sinks, n_cache] or the sensitivities are invalid";
    case KVS_E_ALIGN: return "a device pointer is not suitably aligned";
    case KVS_E_WORKSPACE: return "workspace is smaller than kvs_workspace_bytes()";
    case KVS_E_HIP: return "a HIP launch or runtime call failed";
    case KVS_E_SCRATCH:
      return "the problem needs more scratch than the allocation-free entry point holds "
             "(KVS_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kvs_version(void) { return kVersion; }

int kvs_check_problem(const kvs_problem* p) { return check(p); }

int64_t kvs_num_chunks(const kvs_problem* p) { return check(p) == KVS_OK ? chunks_of(*p) : -1; }

int64_t kvs_num_queries(const kvs_problem* p) {
  return check(p) == KVS_OK ? chunks_of(*p) * p->q_per_chunk : -1;
}

size_t kvs_workspace_bytes(const kvs_problem* p) {
  if (check(p) != KVS_OK) return 0;
  return std::max(plan_score(*p).ws_bytes, select_ws_layout(*p).bytes);
}

int kvs_layer_budgets(int32_t layers, int64_t total, const double* sens, double alpha,
                      int64_t n_cache, int64_t n_sinks, int64_t* k_out) {
  return budgets(layers, total, sens, alpha, n_cache, n_sinks, k_out);
}

int kvs_score(const kvs_problem* p, const void* q, const void* k, float* scores, void* ws,
              size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  const KvSrc kv = single_src(*p, k, nullptr);
  st = do_score(*p, q, kv, scores, ws, ws_bytes);
  if (st) return st;
  return enqueue_score(*p, q, kv, scores, ws, ws_bytes, stream);
}

int kvs_select(const kvs_problem* p, const float* scores, const int64_t* k_per_layer,
               int32_t* kept, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  LayerTable t;
  int32_t kmax = 0;
  st = build_table(*p, k_per_layer, true, 0, &t, &kmax);
  if (st) return st;
  if (p->n_cache > 0 && (!scores || !kept)) return KVS_E_NULL;
  if ((scores && !aligned(scores, 4)) || (kept && !aligned(kept, 4))) return KVS_E_ALIGN;
  if ((st = check_select_ws(*p, ws, ws_bytes))) return st;
  return to_status(launch_select(*p, scores, t, kept, ws, stream));
}

int kvs_compact(const kvs_problem* p, const void* k, const void* v, const int32_t* kept,
                const int64_t* k_per_layer, void* k_out, void* v_out, int64_t out_row_stride,
                void* stream) {
  int st = check(p);
  if (st) return st;
  if (out_row_stride < 0) return KVS_E_SHAPE;
  LayerTable t;
  int32_t kmax = 0;
  st = build_table(*p, k_per_layer, false, out_row_stride, &t, &kmax);
  if (st) return st;
  if (kmax == 0) return KVS_OK;
  if (!kept || (!k_out && !v_out) || (k_out && !k) || (v_out && !v)) return KVS_E_NULL;
  if ((k_out && (!aligned(k, 16) || !aligned(k_out, 16))) ||
      (v_out && (!aligned(v, 16) || !aligned(v_out, 16))) || !aligned(kept, 4))
    return KVS_E_ALIGN;
  return to_status(launch_compact(*p, single_src(*p, k, v), kept, t, kmax, k_out, v_out,
                                  out_row_stride, stream));
}

int kvs_compact_seg(const kvs_problem* p, const kvs_kv_segments* seg, const int32_t* kept,
                    const int64_t* k_per_layer, void* k_out, void* v_out, int64_t out_row_stride,
                    void* stream) {
  int st = check(p);
  if (st) return st;
  if (!seg) return KVS_E_NULL;
  if ((st = check_segments(*p, *seg))) return st;
  if (out_row_stride < 0) return KVS_E_SHAPE;
  LayerTable t;
  int32_t kmax = 0;
  st = build_table(*p, k_per_layer, false, out_row_stride, &t, &kmax);
  if (st) return st;
  if (kmax == 0) return KVS_OK;
  const KvSrc kv = segment_src(*seg);
  if (!kept || (!k_out && !v_out)) return KVS_E_NULL;
  if ((st = check_src(*p, kv, k_out != nullptr, v_out != nullptr))) return st;
  if ((k_out && !aligned(k_out, 16)) || (v_out && !aligned(v_out, 16)) || !aligned(kept, 4))
    return KVS_E_ALIGN;
  return to_status(launch_compact(*p, kv, kept, t, kmax, k_out, v_out, out_row_stride, stream));
}

int kvs_compress_block(const kvs_problem* p, const void* q, const void* k, const void* v,
                       int64_t total_budget, const double* sens, double alpha, float* scores,
                       int32_t* kept, void* k_out, void* v_out, int64_t out_row_stride,
                       int64_t* k_per_layer_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  return compress(*p, q, single_src(*p, k, v), total_budget, sens, alpha, scores, kept, k_out,
                  v_out, out_row_stride, k_per_layer_out, ws, ws_bytes, stream);
}

int kvs_compress_block_noalloc(const kvs_problem* p, const void* q, const void* k,
                               const void* v, int64_t total_budget, const double* sens,
                               double alpha, float* scores, int32_t* kept, void* k_out,
                               void* v_out, int64_t out_row_stride, int64_t* k_per_layer_out,
                               void* stream) {
  int st = check(p);
  if (st) return st;
  // scratch the kernels of this call use: the scoring plan's, and the
  // multi-workgroup select's when the cache takes that path
  size_t need = plan_score(*p, KVS_NOALLOC_SCRATCH_BYTES).ws_bytes;
  if (select_uses_multi(*p)) need = std::max(need, select_ws_layout(*p).bytes);
  if (need > (size_t)KVS_NOALLOC_SCRATCH_BYTES) return KVS_E_SCRATCH;
  void* ws = nullptr;
  if ((st = noalloc_scratch(stream, &ws))) return st;
  return compress(*p, q, single_src(*p, k, v), total_budget, sens, alpha, scores, kept, k_out,
                  v_out, out_row_stride, k_per_layer_out, ws, KVS_NOALLOC_SCRATCH_BYTES, stream);
}

int kvs_compress_block_seg(const kvs_problem* p, const void* q, const kvs_kv_segments* seg,
                           int64_t total_budget, const double* sens, double alpha,
                           float* scores, int32_t* kept, void* k_out, void* v_out,
                           int64_t out_row_stride, int64_t* k_per_layer_out, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if (!seg) return KVS_E_NULL;
  if ((st = check_segments(*p, *seg))) return st;
  return compress(*p, q, segment_src(*seg), total_budget, sens, alpha, scores, kept,
                  k_out, v_out, out_row_stride, k_per_layer_out, ws, ws_bytes, stream);
}

size_t kvs_query_workspace_bytes(const kvs_problem* p) {
  if (check(p) != KVS_OK) return 0;
  const int64_t nc = p->n_cache - std::min(p->n_sinks, p->n_cache);
  return round256(sizeof(float) * (size_t)nc);
}

int kvs_query_counts(const kvs_problem* p, double rho, int64_t* counts, int64_t* total) {
  int st = check(p);
  if (st) return st;
  if (!(rho > 0.0 && rho <= 1.0)) return KVS_E_BUDGET;
  const int64_t R = chunks_of(*p);
  const int64_t S = std::min(p->n_sinks, p->n_cache);
  int64_t sum = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t len = std::min(p->chunk_size, p->n_cache - (S + r * p->chunk_size));
    const int64_t nq = std::max<int64_t>((int64_t)std::floor(rho * (double)len), 1);
    if (counts) counts[r] = nq;
    sum += nq;
  }
  if (total) *total = sum;
  return KVS_OK;
}

int kvs_query_select(const kvs_problem* p, const float* scores, double rho, int32_t* positions,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if (!(rho > 0.0 && rho <= 1.0)) return KVS_E_BUDGET;
  if (chunks_of(*p) == 0) return KVS_OK;  // every position is a sink: no queries
  const size_t need = kvs_query_workspace_bytes(p);
  if (!scores || !positions || !ws) return KVS_E_NULL;
  if (ws_bytes < need) return KVS_E_WORKSPACE;
  if (!aligned(scores, 4) || !aligned(positions, 4) || !aligned(ws, 256)) return KVS_E_ALIGN;
  if ((int64_t)p->layers * p->kv_heads * p->n_cache >= (int64_t(1) << 40)) return KVS_E_SHAPE;
  return to_status(launch_query_select(*p, scores, rho, positions, static_cast<float*>(ws), stream));
}

int kvs_select_global(const kvs_problem* p, const float* scores, int64_t total_budget,
                      int32_t* kept, int64_t* offsets, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if ((st = check_global(*p, total_budget))) return st;
  if (!offsets || !ws || (p->n_cache > 0 && !scores) || (total_budget > 0 && !kept))
    return KVS_E_NULL;
  if (ws_bytes < select_ws_layout(*p).bytes) return KVS_E_WORKSPACE;
  if ((scores && !aligned(scores, 4)) || (kept && !aligned(kept, 4)) || !aligned(offsets, 8) ||
      !aligned(ws, 256))
    return KVS_E_ALIGN;
  return to_status(launch_select_global(*p, scores, total_budget, kept, offsets, ws, stream));
}

int kvs_compact_ragged(const kvs_problem* p, const void* k, const void* v, const int32_t* kept,
                       const int64_t* offsets, int64_t total_rows, void* k_out, void* v_out,
                       void* stream) {
  int st = check(p);
  if (st) return st;
  if (total_rows < 0 || total_rows > (int64_t)p->layers * p->kv_heads * p->n_cache)
    return KVS_E_SHAPE;
  if (!offsets) return KVS_E_NULL;
  if (total_rows == 0) return KVS_OK;
  if (!k || !v || !kept || !k_out || !v_out) return KVS_E_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) ||
      !aligned(kept, 4) || !aligned(offsets, 8))
    return KVS_E_ALIGN;
  return to_status(launch_compact_ragged(*p, single_src(*p, k, v), kept, offsets, total_rows,
                                         k_out, v_out, stream));
}

int kvs_compress_global(const kvs_problem* p, const void* q, const void* k, const void* v,
                        int64_t total_budget, float* scores, int32_t* kept, int64_t* offsets,
                        void* k_out, void* v_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if ((st = check_global(*p, total_budget))) return st;
  const KvSrc kv = single_src(*p, k, v);
  if ((st = do_score(*p, q, kv, scores, ws, ws_bytes))) return st;
  if ((st = check_src(*p, kv, true, true))) return st;
  if (!offsets || !ws) return KVS_E_NULL;
  if (total_budget > 0 && (!kept || !k_out || !v_out)) return KVS_E_NULL;
  if (ws_bytes < select_ws_layout(*p).bytes) return KVS_E_WORKSPACE;
  if ((kept && !aligned(kept, 4)) || !aligned(offsets, 8) || (k_out && !aligned(k_out, 16)) ||
      (v_out && !aligned(v_out, 16)) || !aligned(ws, 256))
    return KVS_E_ALIGN;
  if ((st = enqueue_score(*p, q, kv, scores, ws, ws_bytes, stream))) return st;
  if ((st = to_status(launch_select_global(*p, scores, total_budget, kept, offsets, ws, stream))))
    return st;
  if (total_budget == 0) return KVS_OK;
  return to_status(launch_compact_ragged(*p, kv, kept, offsets, total_budget, k_out, v_out,
                                         stream));
}

size_t kvs_decode_workspace_bytes(const kvs_problem* p, int64_t max_rows) {
  if (check(p) != KVS_OK || max_rows < 0) return 0;
  return decode_ws_layout(*p, max_rows).bytes;
}

int kvs_decode_ragged(const kvs_problem* p, const void* q, const void* k_out, const void* v_out,
                      const int64_t* offsets, int64_t max_rows, float* out, void* ws,
                      size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if (max_rows < 0) return KVS_E_SHAPE;
  const DecodeWs w = decode_ws_layout(*p, max_rows);
  if (w.slots + 8 > kMaxGrid || (int64_t)p->layers * p->q_heads > kMaxGrid) return KVS_E_SHAPE;
  if (!q || !offsets || !out || !ws || (max_rows > 0 && (!k_out || !v_out))) return KVS_E_NULL;
  if (ws_bytes < w.bytes) return KVS_E_WORKSPACE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(offsets, 8) || !aligned(ws, 256) ||
      (k_out && !aligned(k_out, 16)) || (v_out && !aligned(v_out, 16)))
    return KVS_E_ALIGN;
  return to_status(launch_decode(*p, q, k_out, v_out, offsets, max_rows, out, ws, stream));
}

size_t kvs_similarity_workspace_bytes(const kvs_problem* p) {
  if (check(p) != KVS_OK) return 0;
  return round256(sizeof(float) * (size_t)p->layers * p->kv_heads *
                  (size_t)std::max<int64_t>(cdiv(p->n_cache, kSimRows), 1));
}

int kvs_key_similarity(const kvs_problem* p, const void* k_full, const void* k_block,
                       double* similarity, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  if (!similarity || !ws || (p->n_cache > 0 && (!k_full || !k_block))) return KVS_E_NULL;
  if (ws_bytes < kvs_similarity_workspace_bytes(p)) return KVS_E_WORKSPACE;
  if (!aligned(similarity, 8) || !aligned(ws, 256) || (k_full && !aligned(k_full, 16)) ||
      (k_block && !aligned(k_block, 16)))
    return KVS_E_ALIGN;
  if (cdiv(p->n_cache, kSimRows) > kMaxGrid || (int64_t)p->layers * p->kv_heads > 65535)
    return KVS_E_SHAPE;
  return to_status(launch_similarity(*p, k_full, k_block, similarity, ws, stream));
}

int kvs_sensitivity(int32_t layers, const double* similarity, double* sens) {
  if (!similarity || !sens) return KVS_E_NULL;
  if (layers < 1 || layers > KVS_MAX_LAYERS) return KVS_E_SHAPE;
  for (int l = 0; l < layers; ++l)
    if (!(similarity[l] >= -1.0 && similarity[l] <= 1.0)) return KVS_E_BUDGET;
  for (int l = 0; l < layers; ++l) sens[l] = 1.0 - similarity[l];
  return KVS_OK;
}

namespace kvs {
namespace {
int check_embed(int64_t n, int64_t dim, int32_t clusters) {
  if (n < 0 || n > INT32_MAX || dim < 4 || dim > kMaxEmbedDim || dim % 4 != 0) return KVS_E_SHAPE;
  if (clusters < 1 || clusters > kMaxClusters) return KVS_E_SHAPE;
  return KVS_OK;
}
}  // namespace
}  // namespace kvs

size_t kvs_kmeans_workspace_bytes(int64_t n, int64_t dim, int32_t clusters) {
  if (check_embed(n, dim, clusters)) return 0;
  return kmeans_ws_bytes(n, dim, clusters);
}

int kvs_kmeans(const float* x, int64_t n, int64_t dim, int32_t clusters, const float* init,
               int32_t rounds, float* centroids, int32_t* assign, void* ws, size_t ws_bytes,
               void* stream) {
  if (int st = check_embed(n, dim, clusters)) return st;
  if (rounds < 0) return KVS_E_SHAPE;
  if (!init || !centroids || (n > 0 && (!x || !assign)) || (n > 0 && rounds > 0 && !ws))
    return KVS_E_NULL;
  if (n > 0 && rounds > 0 && ws_bytes < kmeans_ws_bytes(n, dim, clusters)) return KVS_E_WORKSPACE;
  if (!aligned(init, 16) || !aligned(centroids, 16) || (x && !aligned(x, 16)) ||
      (assign && !aligned(assign, 4)) || (ws && !aligned(ws, 256)))
    return KVS_E_ALIGN;
  return to_status(launch_kmeans(x, n, dim, clusters, init, rounds, centroids, assign, ws, stream));
}

size_t kvs_medoids_workspace_bytes(int64_t n, int64_t dim, int32_t clusters) {
  if (check_embed(n, dim, clusters) || n > kMaxMedoidPoints) return 0;
  return std::max<size_t>(medoid_ws_bytes(n), 256);
}

int kvs_medoids(const float* x, int64_t n, int64_t dim, const int32_t* assign, int32_t clusters,
                int32_t* medoid, float* totals, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_embed(n, dim, clusters)) return st;
  if (n > kMaxMedoidPoints) return KVS_E_SHAPE;
  if (!medoid || (n > 0 && (!x || !assign || !totals || !ws))) return KVS_E_NULL;
  if (n > 0 && ws_bytes < medoid_ws_bytes(n)) return KVS_E_WORKSPACE;
  if (!aligned(medoid, 4) || (x && !aligned(x, 16)) || (assign && !aligned(assign, 4)) ||
      (totals && !aligned(totals, 4)) || (ws && !aligned(ws, 256)))
    return KVS_E_ALIGN;
  return to_status(launch_medoids(x, n, dim, assign, clusters, medoid, totals, ws, stream));
}

int kvs_match_episodes(const float* q, int64_t m, int64_t dim, const float* centroids,
                       int32_t clusters, int32_t* episode, void* stream) {
  if (int st = check_embed(m, dim, clusters)) return st;
  if (m == 0) return KVS_OK;
  if (!q || !centroids || !episode) return KVS_E_NULL;
  if (!aligned(q, 16) || !aligned(centroids, 16) || !aligned(episode, 4)) return KVS_E_ALIGN;
  return to_status(launch_nearest(q, m, dim, centroids, clusters, episode, stream));
}

int kvs_append_rows(int32_t slabs, int32_t head_dim, int32_t dtype, const void* src,
                    int64_t src_row_stride, int64_t src_row0, int64_t n_rows, void* dst,
                    int64_t dst_row_stride, int64_t dst_row0, void* stream) {
  if (slabs < 0 || n_rows < 0 || src_row0 < 0 || dst_row0 < 0) return KVS_E_SHAPE;
  if (head_dim != 64 && head_dim != 128) return KVS_E_SHAPE;
  if (dtype != KVS_F32 && dtype != KVS_BF16) return KVS_E_DTYPE;
  if (src_row0 + n_rows > src_row_stride || dst_row0 + n_rows > dst_row_stride) return KVS_E_SHAPE;
  if (slabs == 0 || n_rows == 0) return KVS_OK;
  if (!src || !dst) return KVS_E_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return KVS_E_ALIGN;
  const int64_t row_bytes = (int64_t)head_dim * (dtype == KVS_F32 ? 4 : 2);
  if (cdiv(n_rows, 64) > kMaxGrid) return KVS_E_SHAPE;
  return to_status(launch_append(slabs, row_bytes, src, src_row_stride, src_row0, n_rows, dst,
                                 dst_row_stride, dst_row0, stream));
}

}  // extern "C"
