// Decode attention over a headwise-compacted cache whose heads keep different
// numbers of rows (KV² summary, "전제와 한계": serving the compressed cache
// needs an attention kernel that accepts a different compressed length per
// head; "무엇과 다른가": the global eviction produces exactly such a cache).
//
// For every layer l and query head h, with KV head g = h / G and unit
// u = l * Hkv + g:
//     out[l, h] = sum_j softmax_j(q[l, h] . k_j / sqrt(d)) v_j
// over the rows j in [offsets[u], offsets[u + 1]) of the packed K / V.  A head
// whose unit keeps no row gets zeros.
//
// The work is HBM-bound: every kept K and V row is read once and serves all G
// heads of its KV head.  A unit's rows are cut into splits of kRows rows, one
// 256-thread workgroup per split (split-K, so that a long head does not leave
// the chip idle while short ones finish):
//   decode_prefix  sp[u] = splits before unit u (one workgroup, ordered scan)
//   decode_split   one pass over the split's rows for a group of heads: each
//                  lane owns one 16-byte piece of a row (the pieces of a row
//                  are summed with DPP lane moves), K and V streamed together,
//                  an online max / sum / p-weighted V sum per thread, merged
//                  by log-sum-exp; writes (max, sum, acc[d]) per head, max in
//                  the base-2 logit domain
//   decode_merge   per (layer, head): log-sum-exp merge of its unit's splits
#include <algorithm>
#include <cfloat>
#include <cmath>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxHG = 4;  // most heads per pass over a split's rows

struct DecodeArgs {
  const void* q;         // [L, Hq, D]
  const void* k;         // [rows, D]
  const void* v;
  const int64_t* offsets;  // [units + 1]
  float* out;            // [L, Hq, D]
  int64_t* sp;           // [units + 1]
  float* part_ml;        // [slots][G][2]
  float* part_acc;       // [slots][G][D]
  int64_t slots;
  int32_t units, Hkv, Hq, G;
  float c1;              // log2(e) / sqrt(D)
};

// Sum of x over the LPR consecutive lanes that hold one row's pieces (LPR in
// {8, 16, 32}), left in every one of them.  Within a 16-lane row the partners
// come from DPP lane moves on the vector ALU (no LDS traffic): row mirror
// (lane p and 15 - p), half-row mirror (p and p ^ 7) and two quad swaps (p ^ 2,
// p ^ 1); the XOR masks 15, 7, 2 and 1 together reach all 16 lanes, so each
// lane ends with the sum over the whole group (8 lanes: the last three).  A
// 32-lane group first adds the other half through a lane shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR == 32) x += __shfl_xor(x, 16, 64);
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x);  // row mirror
  x += dpp_mov<0x141>(x);                            // row half mirror
  x += dpp_mov<0x4E>(x);                             // quad permute [2, 3, 0, 1]
  x += dpp_mov<0xB1>(x);                             // quad permute [1, 0, 3, 2]
  return x;
}


__global__ __launch_bounds__(1024) void decode_prefix(DecodeArgs a) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < a.units; base += 1024) {
    const int64_t u = base + tid;
    int64_t n = 0;
    if (u < a.units) {
      const int64_t rows = a.offsets[u + 1] - a.offsets[u];
      n = rows > 0 ? ceil_div(rows, kDecodeRows) : 0;
    }
    int64_t x = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int64_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int64_t total = carry;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    if (u < a.units) a.sp[u] = before + x - n;
    carry = total;
    __syncthreads();
  }
  if (tid == 0) a.sp[a.units] = carry;
}

// A row piece as 16 raw bytes, widened to fp32 where it is used.
__device__ __forceinline__ u32x4 load_raw(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void widen(const u32x4& w, float (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
}

__device__ __forceinline__ void widen(const u32x4& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// One pass over the split's rows.  Each step the workgroup covers RPI rows
// (a row's pieces on LPR consecutive lanes); the K and V pieces of U steps
// are loaded together, so both streams are in flight at once.  Every thread
// keeps, per head of the group, a running max m (base-2 logits), sum l and
// accumulator acc of 2^(z - m) v over its rows, brought to the steps' max
// once per U steps.  At the end the threads holding the same piece are
// merged by log-sum-exp: across a wave's rows with lane shuffles, then across
// the waves through LDS.  The partial (max, sum, acc) per head goes to
// decode_merge.
template <typename T, int D, int kHG>
__global__ __launch_bounds__(kThreads) void decode_split(DecodeArgs a) {
  constexpr int EPL = 16 / sizeof(T);      // elements per lane piece
  constexpr int LPR = D / EPL;             // lanes per row
  constexpr int RPI = kThreads / LPR;      // rows per step of the workgroup
  constexpr int ITERS = kDecodeRows / RPI;
  constexpr int U = 4;                     // steps whose loads are issued together
  static_assert(kDecodeRows % RPI == 0 && ITERS % U == 0, "whole load groups");
  __shared__ float red_m[kWaves][kHG], red_l[kWaves][kHG];
  __shared__ float racc[kWaves][kHG][D];
  __shared__ int32_t unit_sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t w = blockIdx.x;
  if (tid == 0) {  // last unit whose splits start at or before w
    int32_t lo = 0, hi = a.units - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (a.sp[mid] <= w) lo = mid;
      else hi = mid - 1;
    }
    unit_sh = lo;
  }
  __syncthreads();
  const int64_t u = unit_sh;
  if (w >= a.sp[a.units] || w >= a.slots) return;  // the same for the whole workgroup
  const int64_t s = w - a.sp[u];
  const int64_t r0 = a.offsets[u] + s * kDecodeRows;
  const int64_t r1 = min(r0 + (int64_t)kDecodeRows, a.offsets[u + 1]);
  const int64_t l = u / a.Hkv, g = u % a.Hkv;
  const int piece = tid % LPR, rsub = tid / LPR;
  const T* qbase = static_cast<const T*>(a.q) + (l * a.Hq + g * a.G) * D + piece * EPL;
  const T* kbase = static_cast<const T*>(a.k) + piece * EPL;
  const T* vbase = static_cast<const T*>(a.v) + piece * EPL;

  for (int h0 = 0; h0 < a.G; h0 += kHG) {
    float qf[kHG][EPL];
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      if (h0 + j < a.G) {
        widen(load_raw(qbase + (h0 + j) * D), qf[j]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[j][e] = 0.f;
      }
    }
    // finite start: a thread whose rows are all past the split's end keeps
    // l = 0 and acc = 0, and every rescale factor stays finite
    float m[kHG], lsum[kHG], acc[kHG][EPL];
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      m[j] = -FLT_MAX;
      lsum[j] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
    }
    for (int it = 0; it < ITERS; it += U) {
      u32x4 kr[U], vr[U];
      bool ok[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int64_t row = r0 + (it + q) * RPI + rsub;
        ok[q] = row < r1;
        const int64_t rr = min(row, r1 - 1);
        kr[q] = load_raw(kbase + rr * D);
        vr[q] = load_raw(vbase + rr * D);
      }
      float z[U][kHG];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        float x[EPL];
        widen(kr[q], x);
#pragma unroll
        for (int j = 0; j < kHG; ++j) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) t = fmaf(qf[j][e], x[e], t);
          z[q][j] = row_sum<LPR>(t);
          z[q][j] = ok[q] ? z[q][j] * a.c1 : -INFINITY;
        }
      }
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
        float bm = z[0][j];
#pragma unroll
        for (int q = 1; q < U; ++q) bm = fmaxf(bm, z[q][j]);
        const float mn = fmaxf(m[j], bm);
        const float sc = exp2_hw(m[j] - mn);
        m[j] = mn;
        lsum[j] *= sc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= sc;
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        float x[EPL];
        widen(vr[q], x);
#pragma unroll
        for (int j = 0; j < kHG; ++j) {
          const float p = exp2_hw(z[q][j] - m[j]);  // 0 past the split's end
          lsum[j] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(p, x[e], acc[j][e]);
        }
      }
    }
    // merge the rows of a wave: lanes piece + k LPR hold the same piece
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
        const float mo = __shfl_xor(m[j], off, 64);
        const float lo = __shfl_xor(lsum[j], off, 64);
        const float mn = fmaxf(m[j], mo);
        const float s1 = exp2_hw(m[j] - mn), s2 = exp2_hw(mo - mn);
        m[j] = mn;
        lsum[j] = lsum[j] * s1 + lo * s2;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float ao = __shfl_xor(acc[j][e], off, 64);
          acc[j][e] = acc[j][e] * s1 + ao * s2;
        }
      }
    }
    if (lane < LPR) {
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) racc[wave][j][piece * EPL + e] = acc[j][e];
        if (lane == 0) {
          red_m[wave][j] = m[j];
          red_l[wave][j] = lsum[j];
        }
      }
    }
    __syncthreads();
    // merge the waves
    for (int i = tid; i < kHG * D; i += kThreads) {
      const int j = i / D, e = i % D;
      if (h0 + j < a.G) {
        float M = red_m[0][j];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][j]);
        float t = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) t += racc[ww][j][e] * exp2_hw(red_m[ww][j] - M);
        a.part_acc[(w * a.G + h0 + j) * D + e] = t;
      }
    }
    if (tid < kHG && h0 + tid < a.G) {
      float M = red_m[0][tid];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][tid]);
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) L += red_l[ww][tid] * exp2_hw(red_m[ww][tid] - M);
      a.part_ml[(w * a.G + h0 + tid) * 2] = M;
      a.part_ml[(w * a.G + h0 + tid) * 2 + 1] = L;
    }
    __syncthreads();  // red_m, red_l and racc are reused by the next head group
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge(DecodeArgs a) {
  const int64_t lh = blockIdx.x;  // l * Hq + h
  const int64_t l = lh / a.Hq, h = lh % a.Hq;
  const int64_t u = l * a.Hkv + h / a.G, j = h % a.G;
  const int e = threadIdx.x;
  const int64_t s0 = min(a.sp[u], a.slots), s1 = min(a.sp[u + 1], a.slots);
  // both loops unrolled so that several splits' loads are in flight
  float m = -INFINITY;
#pragma unroll 4
  for (int64_t s = s0; s < s1; ++s) m = fmaxf(m, a.part_ml[(s * a.G + j) * 2]);
  float den = 0.f, num = 0.f;
#pragma unroll 4
  for (int64_t s = s0; s < s1; ++s) {
    const float f = exp2_hw(a.part_ml[(s * a.G + j) * 2] - m);
    den = fmaf(a.part_ml[(s * a.G + j) * 2 + 1], f, den);
    num = fmaf(a.part_acc[(s * a.G + j) * D + e], f, num);
  }
  a.out[lh * D + e] = den > 0.f ? num / den : 0.f;
}

template <typename T, int D>
int decode_run(DecodeArgs a, int64_t n_heads, hipStream_t st) {
  {
    TraceScope ts("decode_prefix", st);
    hipLaunchKernelGGL(decode_prefix, dim3(1), dim3(1024), 0, st, a);
  }
  if (a.slots > 0) {
    // heads per pass: the whole group when it has at most kMaxHG heads (no
    // idle registers), else passes of kMaxHG
    TraceScope ts("decode_split", st);
    const dim3 grid((unsigned)a.slots), block(kThreads);
    switch (std::min(a.G, kMaxHG)) {
      case 1: hipLaunchKernelGGL((decode_split<T, D, 1>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((decode_split<T, D, 2>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((decode_split<T, D, 3>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((decode_split<T, D, kMaxHG>), grid, block, 0, st, a); break;
    }
  }
  TraceScope ts("decode_merge", st);
  hipLaunchKernelGGL(decode_merge<D>, dim3((unsigned)n_heads), dim3(D), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace

DecodeWs decode_ws_layout(const kvs_problem& p, int64_t max_rows) {
  auto r256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  const int64_t G = p.q_heads / std::max(p.kv_heads, 1);
  DecodeWs w;
  w.slots = ceil_div(std::max<int64_t>(max_rows, 0), kDecodeRows) + units;
  size_t off = 0;
  w.off_sp = off;
  off += r256(sizeof(int64_t) * (size_t)(units + 1));
  w.off_ml = off;
  off += r256(sizeof(float) * 2 * (size_t)(w.slots * G));
  w.off_acc = off;
  off += r256(sizeof(float) * (size_t)(w.slots * G * p.head_dim));
  w.bytes = off;
  return w;
}

int launch_decode(const kvs_problem& p, const void* q, const void* k, const void* v,
                  const int64_t* offsets, int64_t max_rows, float* out, void* ws, void* stream) {
  const DecodeWs w = decode_ws_layout(p, max_rows);
  uint8_t* base = static_cast<uint8_t*>(ws);
  DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.offsets = offsets;
  a.out = out;
  a.sp = reinterpret_cast<int64_t*>(base + w.off_sp);
  a.part_ml = reinterpret_cast<float*>(base + w.off_ml);
  a.part_acc = reinterpret_cast<float*>(base + w.off_acc);
  a.slots = w.slots;
  a.units = p.layers * p.kv_heads;
  a.Hkv = p.kv_heads;
  a.Hq = p.q_heads;
  a.G = p.q_heads / p.kv_heads;
  a.c1 = (float)(1.4426950408889634 / std::sqrt((double)p.head_dim));
  const int64_t n_heads = (int64_t)p.layers * p.q_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.dtype == KVS_BF16)
    return p.head_dim == 128 ? decode_run<__bf16, 128>(a, n_heads, st)
                             : decode_run<__bf16, 64>(a, n_heads, st);
  return p.head_dim == 128 ? decode_run<float, 128>(a, n_heads, st)
                           : decode_run<float, 64>(a, n_heads, st);
}

}  // namespace kvs
