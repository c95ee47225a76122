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
//   decode_split   logits of the split's rows for a group of heads (each lane
//                  owns one 16-byte piece of a row; the pieces of a row are
//                  summed with DPP lane moves), per-head max and exp2 in LDS,
//                  then the p-weighted sum of the V rows; writes (max, sum,
//                  acc[d]) per head, max in the base-2 logit domain
//   decode_merge   per (layer, head): log-sum-exp merge of its unit's splits
#include <algorithm>
#include <cmath>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kHG = 4;  // heads per pass over a split's rows

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

__device__ __forceinline__ void load_piece(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x;
  x[1] = v.y;
  x[2] = v.z;
  x[3] = v.w;
}

__device__ __forceinline__ void load_piece(const __bf16* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

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

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

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

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_split(DecodeArgs a) {
  constexpr int EPL = 16 / sizeof(T);      // elements per lane piece
  constexpr int LPR = D / EPL;             // lanes per row
  constexpr int RPI = kThreads / LPR;      // rows per iteration of the workgroup
  constexpr int ITERS = kDecodeRows / RPI;
  static_assert(kDecodeRows % RPI == 0, "whole iterations");
  constexpr int RPT = kDecodeRows / kThreads;   // rows per thread in the softmax step
  static_assert(kDecodeRows % kThreads == 0, "whole rows per thread in the softmax step");
  __shared__ float zs[kDecodeRows][kHG];
  __shared__ float red[kWaves][kHG];
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
  const T* kbase = static_cast<const T*>(a.k);
  const T* vbase = static_cast<const T*>(a.v);

  for (int h0 = 0; h0 < a.G; h0 += kHG) {
    float qf[kHG][EPL];
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      if (h0 + j < a.G) {
        load_piece(qbase + (h0 + j) * D, qf[j]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[j][e] = 0.f;
      }
    }
    // logits of the split's rows
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
      const int rloc = it * RPI + rsub;
      const int64_t row = r0 + rloc;
      float x[EPL];
      load_piece(kbase + min(row, r1 - 1) * D + piece * EPL, x);
      float z[kHG];
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[j][e], x[e], acc);
        z[j] = acc;
      }
#pragma unroll
      for (int j = 0; j < kHG; ++j) z[j] = row_sum<LPR>(z[j]);
      if (piece == 0) {
#pragma unroll
        for (int j = 0; j < kHG; ++j) zs[rloc][j] = row < r1 ? z[j] * a.c1 : -INFINITY;
      }
    }
    __syncthreads();
    // per-head max and sum over the split; thread t owns rows t + q * kThreads
    float zt[RPT][kHG], mx[kHG], sm[kHG];
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        zt[q][j] = zs[tid + q * kThreads][j];
        m = fmaxf(m, zt[q][j]);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      if (lane == 0) red[wave][j] = m;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      mx[j] = red[0][j];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) mx[j] = fmaxf(mx[j], red[ww][j]);
    }
    __syncthreads();  // red is rewritten below
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * kThreads;
        const float p = r < r1 - r0 ? exp2_hw(zt[q][j] - mx[j]) : 0.f;
        zs[r][j] = p;
        t += p;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      if (lane == 0) red[wave][j] = t;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
      sm[j] = red[0][j];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) sm[j] += red[ww][j];
    }
    // p-weighted sum of the V rows
    float acc[kHG][EPL];
#pragma unroll
    for (int j = 0; j < kHG; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
    }
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
      const int rloc = it * RPI + rsub;
      const int64_t row = r0 + rloc;
      float x[EPL];
      load_piece(vbase + min(row, r1 - 1) * D + piece * EPL, x);
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
        const float p = zs[rloc][j];  // 0 past the split's end
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(p, x[e], acc[j][e]);
      }
    }
    // sum over the rows a wave holds (lanes with the same piece), then the waves
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] += __shfl_xor(acc[j][e], off, 64);
      }
    }
    if (lane < LPR) {
#pragma unroll
      for (int j = 0; j < kHG; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) racc[wave][j][piece * EPL + e] = acc[j][e];
      }
    }
    __syncthreads();
    for (int i = tid; i < kHG * D; i += kThreads) {
      const int j = i / D, e = i % D;
      if (h0 + j < a.G) {
        float t = racc[0][j][e];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) t += racc[ww][j][e];
        a.part_acc[(w * a.G + h0 + j) * D + e] = t;
      }
    }
    if (tid < kHG && h0 + tid < a.G) {
      a.part_ml[(w * a.G + h0 + tid) * 2] = mx[tid];
      a.part_ml[(w * a.G + h0 + tid) * 2 + 1] = sm[tid];
    }
    __syncthreads();  // zs, red and racc are reused by the next head group
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge(DecodeArgs a) {
  const int64_t lh = blockIdx.x;  // l * Hq + h
  const int64_t l = lh / a.Hq, h = lh % a.Hq;
  const int64_t u = l * a.Hkv + h / a.G, j = h % a.G;
  const int e = threadIdx.x;
  const int64_t s0 = min(a.sp[u], a.slots), s1 = min(a.sp[u + 1], a.slots);
  float m = -INFINITY;
  for (int64_t s = s0; s < s1; ++s) m = fmaxf(m, a.part_ml[(s * a.G + j) * 2]);
  float den = 0.f, num = 0.f;
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
    TraceScope ts("decode_split", st);
    hipLaunchKernelGGL((decode_split<T, D>), dim3((unsigned)a.slots), dim3(kThreads), 0, st, a);
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
