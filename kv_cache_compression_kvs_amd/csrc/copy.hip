// Row movers: headwise compaction and block append.
//
// Compaction (KV² summary, "전제와 한계": serving needs the cache physically
// compacted per head): output row t of slab (l, g) is K[l, g, kept[t]] (and
// the same for V).  Append (EpiCache review, "방법: 3단계" (2), Fig. 1(b)):
// the next block's rows are copied behind the kept cache.
//
// Both are pure HBM streams.  A row is head_dim * element bytes (128-512 B);
// each lane moves one 16-byte piece, a 256-thread workgroup moves
// 256 / pieces_per_row rows per pass and four passes per launch slot, with all
// loads issued before the stores so that eight 16-byte reads per lane
// (K and V) are in flight.  Loads and stores carry the nontemporal hint: the
// streams are far larger than the caches and are not re-read by this kernel.
#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct CompactArgs {
  const uint8_t* kh;  // rows [0, split) of each slab, slab stride h_stride rows
  const uint8_t* vh;
  const uint8_t* kt;  // rows [split, n_cache): row t_row0 + (i - split), slab stride t_stride
  const uint8_t* vt;
  const int32_t* kept;
  uint8_t* ko;
  uint8_t* vo;
  int64_t row_bytes, h_stride, t_stride, t_row0, split, out_stride, n_cache;
  int32_t Hkv;
  LayerTable t;
};

// PLANES: bit 0 moves K, bit 1 moves V (a caller may compact the two apart,
// e.g. V on a second stream while the next step scores with K).
template <int LPR, int PLANES>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  constexpr int RPP = kThreads / LPR;
  const int64_t unit = blockIdx.y;
  const int64_t l = unit / a.Hkv, g = unit % a.Hkv;
  const int64_t kl = a.t.k[l];
  const int64_t t0 = (int64_t)blockIdx.x * (RPP * kUnroll);
  if (t0 >= kl) return;
  const int32_t* kp = a.kept + a.t.off[l] + g * kl;
  const int64_t slab = l * a.Hkv + g;
  const int64_t hoff = slab * a.h_stride * a.row_bytes;
  const int64_t toff = (slab * a.t_stride + a.t_row0 - a.split) * a.row_bytes;  // + i * row_bytes
  const int64_t orow0 = a.out_stride ? (l * a.Hkv + g) * a.out_stride : a.t.off[l] + g * kl;
  uint8_t* ko = (PLANES & 1) ? a.ko + orow0 * a.row_bytes : nullptr;
  uint8_t* vo = (PLANES & 2) ? a.vo + orow0 * a.row_bytes : nullptr;
  const int piece = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;

  // Every load is unconditional (from a clamped, in-bounds row) so that all of
  // them are in flight at once; only the stores are guarded.
  int64_t idx[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) idx[u] = kp[min(t0 + u * RPP + rsub, kl - 1)];
  u32x4 kb[kUnroll], vb[kUnroll];
  bool ok[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    ok[u] = t0 + u * RPP + rsub < kl && idx[u] >= 0 && idx[u] < a.n_cache;  // rows outside the cache are skipped
    const int64_t i = ok[u] ? idx[u] : 0;
    const bool head = i < a.split;
    const int64_t src = (head ? hoff : toff) + i * a.row_bytes + piece * 16;
    if (PLANES & 1) kb[u] = __builtin_nontemporal_load((const u32x4*)((head ? a.kh : a.kt) + src));
    if (PLANES & 2) vb[u] = __builtin_nontemporal_load((const u32x4*)((head ? a.vh : a.vt) + src));
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t t = t0 + u * RPP + rsub;
    if (ok[u]) {
      const int64_t dst = t * a.row_bytes + piece * 16;
      if (PLANES & 1) __builtin_nontemporal_store(kb[u], (u32x4*)(ko + dst));
      if (PLANES & 2) __builtin_nontemporal_store(vb[u], (u32x4*)(vo + dst));
    }
  }
}

template <int LPR>
__global__ __launch_bounds__(kThreads) void append_kernel(const uint8_t* src, int64_t src_stride,
                                                          int64_t src_row0, int64_t n_rows,
                                                          uint8_t* dst, int64_t dst_stride,
                                                          int64_t dst_row0, int64_t row_bytes) {
  constexpr int RPP = kThreads / LPR;
  const int64_t slab = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * (RPP * kUnroll);
  const uint8_t* s = src + (slab * src_stride + src_row0) * row_bytes;
  uint8_t* d = dst + (slab * dst_stride + dst_row0) * row_bytes;
  const int piece = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  u32x4 b[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t t = min(t0 + u * RPP + rsub, n_rows - 1);  // unconditional, in bounds
    b[u] = __builtin_nontemporal_load((const u32x4*)(s + t * row_bytes + piece * 16));
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t t = t0 + u * RPP + rsub;
    if (t < n_rows) __builtin_nontemporal_store(b[u], (u32x4*)(d + t * row_bytes + piece * 16));
  }
}

// Ragged compaction (global eviction): output row t belongs to the unit u
// with offsets[u] <= t < offsets[u + 1] and is row kept[t] of that unit's
// slab.  The grid covers the rows; the first wave finds the workgroup's first
// unit by counting the units that start at or before its first row (one load
// per lane per 64 units, all independent), and each row walks forward from it
// (a workgroup's rows rarely cross more than one unit boundary).
struct RaggedArgs {
  const uint8_t* kh;
  const uint8_t* vh;
  const uint8_t* kt;
  const uint8_t* vt;
  const int32_t* kept;
  const int64_t* offsets;
  uint8_t* ko;
  uint8_t* vo;
  int64_t row_bytes, h_stride, t_stride, t_row0, split, n_cache, total;
  int32_t units;
};

template <int LPR>
__global__ __launch_bounds__(kThreads) void compact_ragged_kernel(RaggedArgs a) {
  constexpr int RPP = kThreads / LPR;
  __shared__ int32_t first_unit;
  const int64_t t0 = (int64_t)blockIdx.x * (RPP * kUnroll);
  if (threadIdx.x < 64) {
    // The last unit whose list starts at or before t0.  offsets is
    // non-decreasing with offsets[0] = 0, so that is the count of units
    // starting at or before t0, minus one: independent loads, one per lane
    // and 64 units, instead of a binary search's chain of dependent ones.
    int32_t c = 0;
    for (int32_t j = threadIdx.x; j < a.units; j += 64) c += a.offsets[j] <= t0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
    if (threadIdx.x == 0) first_unit = c > 0 ? c - 1 : 0;
  }
  __syncthreads();
  const int piece = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  int64_t slab[kUnroll], idx[kUnroll];
  bool ok[kUnroll];
  const int32_t u0 = first_unit;
  // the workgroup's rows nearly always lie in u0 or the units right after it:
  // u0's end is loaded once, and only rows past it walk on
  const int64_t end0 = u0 + 1 < a.units ? a.offsets[u0 + 1] : INT64_MAX;
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t t = t0 + k * RPP + rsub;
    int32_t u = u0;
    if (t >= end0) {
      ++u;
      while (u + 1 < a.units && a.offsets[u + 1] <= t) ++u;
    }
    const int64_t i = a.kept[min(t, a.total - 1)];
    ok[k] = t < a.total && i >= 0 && i < a.n_cache;  // rows outside the cache are skipped
    idx[k] = ok[k] ? i : 0;
    slab[k] = u;
  }
  u32x4 kb[kUnroll], vb[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int64_t i = idx[k];
    const bool head = i < a.split;
    const int64_t src = head ? (slab[k] * a.h_stride + i) * a.row_bytes
                             : (slab[k] * a.t_stride + a.t_row0 + (i - a.split)) * a.row_bytes;
    kb[k] = __builtin_nontemporal_load((const u32x4*)((head ? a.kh : a.kt) + src + piece * 16));
    vb[k] = __builtin_nontemporal_load((const u32x4*)((head ? a.vh : a.vt) + src + piece * 16));
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    if (ok[k]) {
      const int64_t dst = (t0 + k * RPP + rsub) * a.row_bytes + piece * 16;
      __builtin_nontemporal_store(kb[k], (u32x4*)(a.ko + dst));
      __builtin_nontemporal_store(vb[k], (u32x4*)(a.vo + dst));
    }
  }
}

template <int LPR>
int compact_ragged_lpr(const RaggedArgs& a, hipStream_t st) {
  constexpr int RPP = kThreads / LPR;
  const int64_t gx = ceil_div(a.total, RPP * kUnroll);
  if (gx <= 0 || a.units <= 0) return 0;
  TraceScope ts("compact_ragged", st);
  hipLaunchKernelGGL(compact_ragged_kernel<LPR>, dim3((unsigned)gx), dim3(kThreads), 0, st, a);
  return (int)hipGetLastError();
}

template <int LPR>
int compact_lpr(const CompactArgs& a, int64_t units, int32_t k_max, hipStream_t st) {
  constexpr int RPP = kThreads / LPR;
  const int64_t gx = ceil_div(k_max, RPP * kUnroll);
  if (gx <= 0 || units <= 0 || (!a.ko && !a.vo)) return 0;
  TraceScope ts("compact", st);
  const dim3 grid((unsigned)gx, (unsigned)units), block(kThreads);
  if (a.ko && a.vo) hipLaunchKernelGGL((compact_kernel<LPR, 3>), grid, block, 0, st, a);
  else if (a.ko) hipLaunchKernelGGL((compact_kernel<LPR, 1>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((compact_kernel<LPR, 2>), grid, block, 0, st, a);
  return (int)hipGetLastError();
}

template <int LPR>
int append_lpr(int32_t slabs, int64_t row_bytes, const void* src, int64_t src_stride,
               int64_t src_row0, int64_t n_rows, void* dst, int64_t dst_stride,
               int64_t dst_row0, hipStream_t st) {
  constexpr int RPP = kThreads / LPR;
  const int64_t gx = ceil_div(n_rows, RPP * kUnroll);
  if (gx <= 0 || slabs <= 0) return 0;
  TraceScope ts("append", st);
  hipLaunchKernelGGL(append_kernel<LPR>, dim3((unsigned)gx, (unsigned)slabs), dim3(kThreads), 0,
                     st, static_cast<const uint8_t*>(src), src_stride, src_row0, n_rows,
                     static_cast<uint8_t*>(dst), dst_stride, dst_row0, row_bytes);
  return (int)hipGetLastError();
}

}  // namespace

int launch_compact(const kvs_problem& p, const KvSrc& kv, const int32_t* kept,
                   const LayerTable& t, int32_t k_max, void* k_out, void* v_out,
                   int64_t out_row_stride, void* stream) {
  CompactArgs a;
  a.kh = static_cast<const uint8_t*>(kv.k_head);
  a.vh = static_cast<const uint8_t*>(kv.v_head);
  a.kt = static_cast<const uint8_t*>(kv.k_tail);
  a.vt = static_cast<const uint8_t*>(kv.v_tail);
  a.h_stride = kv.head_stride;
  a.t_stride = kv.tail_stride;
  a.t_row0 = kv.tail_row0;
  a.split = kv.split;
  a.kept = kept;
  a.ko = static_cast<uint8_t*>(k_out);
  a.vo = static_cast<uint8_t*>(v_out);
  a.row_bytes = (int64_t)p.head_dim * (p.dtype == KVS_F32 ? 4 : 2);
  a.out_stride = out_row_stride;
  a.n_cache = p.n_cache;
  a.Hkv = p.kv_heads;
  a.t = t;
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (a.row_bytes) {
    case 128: return compact_lpr<8>(a, units, k_max, st);
    case 256: return compact_lpr<16>(a, units, k_max, st);
    default: return compact_lpr<32>(a, units, k_max, st);
  }
}

int launch_compact_ragged(const kvs_problem& p, const KvSrc& kv, const int32_t* kept,
                          const int64_t* offsets, int64_t total, void* k_out, void* v_out,
                          void* stream) {
  RaggedArgs a;
  a.kh = static_cast<const uint8_t*>(kv.k_head);
  a.vh = static_cast<const uint8_t*>(kv.v_head);
  a.kt = static_cast<const uint8_t*>(kv.k_tail);
  a.vt = static_cast<const uint8_t*>(kv.v_tail);
  a.h_stride = kv.head_stride;
  a.t_stride = kv.tail_stride;
  a.t_row0 = kv.tail_row0;
  a.split = kv.split;
  a.kept = kept;
  a.offsets = offsets;
  a.ko = static_cast<uint8_t*>(k_out);
  a.vo = static_cast<uint8_t*>(v_out);
  a.row_bytes = (int64_t)p.head_dim * (p.dtype == KVS_F32 ? 4 : 2);
  a.n_cache = p.n_cache;
  a.total = total;
  a.units = p.layers * p.kv_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (a.row_bytes) {
    case 128: return compact_ragged_lpr<8>(a, st);
    case 256: return compact_ragged_lpr<16>(a, st);
    default: return compact_ragged_lpr<32>(a, st);
  }
}

int launch_append(int32_t slabs, int64_t row_bytes, const void* src, int64_t src_stride,
                  int64_t src_row0, int64_t n_rows, void* dst, int64_t dst_stride,
                  int64_t dst_row0, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (row_bytes) {
    case 128:
      return append_lpr<8>(slabs, row_bytes, src, src_stride, src_row0, n_rows, dst, dst_stride,
                           dst_row0, st);
    case 256:
      return append_lpr<16>(slabs, row_bytes, src, src_stride, src_row0, n_rows, dst, dst_stride,
                            dst_row0, st);
    default:
      return append_lpr<32>(slabs, row_bytes, src, src_stride, src_row0, n_rows, dst, dst_stride,
                            dst_row0, st);
  }
}

}  // namespace kvs
