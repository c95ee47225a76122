// Layer sensitivity calibration (EpiCache review, "+α: 레이어별 예산 배분" and
// Fig. 4(a)): how far the keys a layer computes under block prefill move from
// its full-prefill keys.  similarity[l] is the mean over (KV head, position)
// of the cosine between the two key rows; a pair with a zero row counts as
// cosine 0.  The budget split then uses sensitivity 1 - similarity.
//
// HBM-bound: both key tensors are streamed once.  One 256-thread workgroup per
// (row block, slab); each lane owns one 16-byte piece of a row, so the
// workgroup reads 256 / pieces_per_row rows per step with fully coalesced
// loads, and the pieces' partial dot products and squared norms are summed
// with cross-lane adds.  Each row's cosine is added to the running sum of the
// row's first lane; the workgroup's sum is written to the workspace and a
// second kernel adds a layer's partials in a fixed order in float64, so the
// result does not depend on scheduling.
#include <cmath>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;  // row steps whose loads are issued together

struct SimArgs {
  const void* a;   // [L, Hkv, stride, d]
  const void* b;
  float* partial;  // [slabs][blocks]
  double* out;     // [L]
  int64_t N, stride, blocks;
  int32_t Hkv;
};

__device__ __forceinline__ void piece_f32(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x;
  x[1] = v.y;
  x[2] = v.z;
  x[3] = v.w;
}

__device__ __forceinline__ void piece_f32(const __bf16* p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void similarity_partial(SimArgs a) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPR = D / EPL;
  constexpr int RPI = kThreads / LPR;  // rows per step
  __shared__ float red[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int piece = tid % LPR, rsub = tid / LPR;
  const int64_t slab = blockIdx.y, blk = blockIdx.x;
  const int64_t r0 = blk * kSimRows;
  const int64_t r1 = min(r0 + (int64_t)kSimRows, a.N);
  const T* pa = static_cast<const T*>(a.a) + slab * a.stride * D + piece * EPL;
  const T* pb = static_cast<const T*>(a.b) + slab * a.stride * D + piece * EPL;
  float sum = 0.f;
  for (int64_t base = r0; base < r1; base += (int64_t)RPI * kUnroll) {
    float xa[kUnroll][EPL], xb[kUnroll][EPL];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t row = min(base + k * RPI + rsub, r1 - 1);  // in bounds; masked below
      piece_f32(pa + row * D, xa[k]);
      piece_f32(pb + row * D, xb[k]);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      float dot = 0.f, na = 0.f, nb = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        dot = fmaf(xa[k][e], xb[k][e], dot);
        na = fmaf(xa[k][e], xa[k][e], na);
        nb = fmaf(xb[k][e], xb[k][e], nb);
      }
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) {
        dot += __shfl_xor(dot, off, 64);
        na += __shfl_xor(na, off, 64);
        nb += __shfl_xor(nb, off, 64);
      }
      const float den = sqrtf(na) * sqrtf(nb);
      if (piece == 0 && base + k * RPI + rsub < r1 && den > 0.f) sum += dot / den;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    a.partial[slab * a.blocks + blk] = t;
  }
}

// One workgroup per layer: the layer's partials in (KV head, block) order,
// each thread a fixed stride of them, then a fixed-order tree in LDS.
__global__ __launch_bounds__(kThreads) void similarity_final(SimArgs a) {
  __shared__ double red[kThreads];
  const int64_t l = blockIdx.x;
  const int64_t n = (int64_t)a.Hkv * a.blocks;
  const float* p = a.partial + l * n;
  double t = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) t += (double)p[i];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.out[l] = a.N > 0 ? red[0] / ((double)a.Hkv * (double)a.N) : 0.0;
}

template <typename T, int D>
int similarity_run(const SimArgs& a, int64_t layers, hipStream_t st) {
  if (a.blocks > 0) {
    TraceScope ts("similarity_partial", st);
    hipLaunchKernelGGL((similarity_partial<T, D>), dim3((unsigned)a.blocks, (unsigned)(layers * a.Hkv)),
                       dim3(kThreads), 0, st, a);
  }
  TraceScope ts("similarity_final", st);
  hipLaunchKernelGGL(similarity_final, dim3((unsigned)layers), dim3(kThreads), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_similarity(const kvs_problem& p, const void* k_full, const void* k_block,
                      double* similarity, void* ws, void* stream) {
  SimArgs a;
  a.a = k_full;
  a.b = k_block;
  a.partial = static_cast<float*>(ws);
  a.out = similarity;
  a.N = p.n_cache;
  a.stride = p.kv_row_stride ? p.kv_row_stride : p.n_cache;
  a.blocks = ceil_div(p.n_cache, kSimRows);
  a.Hkv = p.kv_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.dtype == KVS_BF16)
    return p.head_dim == 128 ? similarity_run<__bf16, 128>(a, p.layers, st)
                             : similarity_run<__bf16, 64>(a, p.layers, st);
  return p.head_dim == 128 ? similarity_run<float, 128>(a, p.layers, st)
                           : similarity_run<float, 64>(a, p.layers, st);
}

}  // namespace kvs
