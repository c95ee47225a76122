// Episode clustering and matching (EpiCache review, "방법: 3단계" (1) and (3),
// Fig. 3(a) and (c)): the history's segment embeddings are clustered by
// K-means into E episodes, each episode is represented by its medoid segment,
// and a new question's embedding is matched to the closest episode.
//
// Lloyd's algorithm from caller-given initial centroids, squared Euclidean
// distance, fp32 arithmetic:
//   nearest_kernel   one wave per point: the distance to each centroid is
//                    summed over 16-byte pieces of the row held by the lanes
//                    and reduced across the wave; the least wins, ties to the
//                    lower centroid.  Also serves the question matching.
//   centroid_partial one workgroup per (block of points, 1024 dimensions):
//                    each thread owns four dimensions and adds every point of
//                    the block into that point's cluster row in LDS, so no
//                    two threads touch one accumulator.
//   centroid_final   per (cluster, dimension): the blocks' partials in a fixed
//                    order in float64, divided by the member count; an empty
//                    cluster keeps its centroid.
//   medoid_total     for 8 candidate points (rows staged in LDS) at a time,
//                    every thread walks its share of all points and adds the
//                    Euclidean distance of those in the candidate's cluster;
//                    a fixed-order tree sums the threads.
//   medoid_pick      per cluster, the member with the least total, ties to
//                    the lower index (-1 if the cluster is empty).
#include <cmath>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBlockPoints = 256;  // points per centroid_partial workgroup
constexpr int kSliceDims = 1024;   // dimensions per centroid_partial workgroup
constexpr int kCand = 8;           // candidate points per medoid_total workgroup

__global__ __launch_bounds__(kThreads) void nearest_kernel(const float* __restrict__ x, int64_t n,
                                                           int64_t D, const float* __restrict__ c,
                                                           int32_t E, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (i >= n) return;  // a whole wave
  const float* xr = x + i * D;
  float best = INFINITY;
  int32_t arg = 0;
  for (int32_t e = 0; e < E; ++e) {
    const float* cr = c + (int64_t)e * D;
    float acc = 0.f;
    for (int64_t k = 4 * lane; k < D; k += 256) {
      const float4 a = *reinterpret_cast<const float4*>(xr + k);
      const float4 b = *reinterpret_cast<const float4*>(cr + k);
      const float d0 = a.x - b.x, d1 = a.y - b.y, d2 = a.z - b.z, d3 = a.w - b.w;
      acc = fmaf(d0, d0, acc);
      acc = fmaf(d1, d1, acc);
      acc = fmaf(d2, d2, acc);
      acc = fmaf(d3, d3, acc);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (acc < best) {  // the same on every lane after the full reduction
      best = acc;
      arg = e;
    }
  }
  if (lane == 0) out[i] = arg;
}

__global__ __launch_bounds__(kThreads) void centroid_partial(const float* __restrict__ x, int64_t n,
                                                             int64_t D,
                                                             const int32_t* __restrict__ assign,
                                                             int32_t E, float* __restrict__ psum,
                                                             int32_t* __restrict__ pcnt) {
  __shared__ float acc[kMaxClusters][kSliceDims];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t d0 = (int64_t)blockIdx.y * kSliceDims + 4 * tid;
  const bool mine = d0 < D;  // D is a multiple of 4
  for (int e = 0; e < E; ++e) {
    acc[e][4 * tid + 0] = 0.f;
    acc[e][4 * tid + 1] = 0.f;
    acc[e][4 * tid + 2] = 0.f;
    acc[e][4 * tid + 3] = 0.f;
  }
  int32_t cnt[kMaxClusters];
#pragma unroll
  for (int e = 0; e < kMaxClusters; ++e) cnt[e] = 0;
  const int64_t p0 = blk * kBlockPoints, p1 = min(p0 + kBlockPoints, n);
  for (int64_t i = p0; i < p1; ++i) {
    const int32_t a = assign[i];
    if (mine) {
      const float4 v = *reinterpret_cast<const float4*>(x + i * D + d0);
      acc[a][4 * tid + 0] += v.x;
      acc[a][4 * tid + 1] += v.y;
      acc[a][4 * tid + 2] += v.z;
      acc[a][4 * tid + 3] += v.w;
    }
#pragma unroll
    for (int e = 0; e < kMaxClusters; ++e) cnt[e] += a == e;
  }
  if (mine) {
    for (int e = 0; e < E; ++e) {
      float4 s;
      s.x = acc[e][4 * tid + 0];
      s.y = acc[e][4 * tid + 1];
      s.z = acc[e][4 * tid + 2];
      s.w = acc[e][4 * tid + 3];
      *reinterpret_cast<float4*>(psum + (blk * E + e) * D + d0) = s;
    }
  }
  if (blockIdx.y == 0 && tid == 0)
    for (int e = 0; e < E; ++e) pcnt[blk * E + e] = cnt[e];
}

__global__ __launch_bounds__(kThreads) void centroid_final(const float* __restrict__ psum,
                                                           const int32_t* __restrict__ pcnt,
                                                           int64_t blocks, int64_t D, int32_t E,
                                                           float* __restrict__ c) {
  const int64_t e = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k >= D) return;
  double s = 0.0;
  int64_t cnt = 0;
  for (int64_t b = 0; b < blocks; ++b) {
    s += (double)psum[(b * E + e) * D + k];
    cnt += pcnt[b * E + e];
  }
  if (cnt > 0) c[e * D + k] = (float)(s / (double)cnt);
}

__global__ __launch_bounds__(kThreads) void copy_f32(const float* __restrict__ src,
                                                     float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void medoid_total(const float* __restrict__ x, int64_t n,
                                                         int64_t D,
                                                         const int32_t* __restrict__ assign,
                                                         float* __restrict__ total) {
  __shared__ float cand[kCand * kMaxEmbedDim];  // [kCand][D]
  __shared__ float red[kThreads][kCand];
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * kCand;
  int32_t ca[kCand];
#pragma unroll
  for (int c = 0; c < kCand; ++c) {
    const int64_t i = min(i0 + c, n - 1);
    ca[c] = i0 + c < n ? assign[i] : -1;
    for (int64_t k = tid; k < D; k += kThreads) cand[c * D + k] = x[i * D + k];
  }
  __syncthreads();
  float acc[kCand];
#pragma unroll
  for (int c = 0; c < kCand; ++c) acc[c] = 0.f;
  for (int64_t j = tid; j < n; j += kThreads) {
    const int32_t aj = assign[j];
    bool any = false;
#pragma unroll
    for (int c = 0; c < kCand; ++c) any |= ca[c] == aj;
    if (!any) continue;
    float d2[kCand];
#pragma unroll
    for (int c = 0; c < kCand; ++c) d2[c] = 0.f;
    const float* xr = x + j * D;
    for (int64_t k = 0; k < D; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(xr + k);
#pragma unroll
      for (int c = 0; c < kCand; ++c) {
        const float* cr = cand + c * D + k;  // the same address on every lane: broadcast
        const float e0 = v.x - cr[0], e1 = v.y - cr[1], e2 = v.z - cr[2], e3 = v.w - cr[3];
        d2[c] = fmaf(e0, e0, d2[c]);
        d2[c] = fmaf(e1, e1, d2[c]);
        d2[c] = fmaf(e2, e2, d2[c]);
        d2[c] = fmaf(e3, e3, d2[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < kCand; ++c)
      if (ca[c] == aj) acc[c] += sqrtf(d2[c]);
  }
#pragma unroll
  for (int c = 0; c < kCand; ++c) red[tid][c] = acc[c];
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c < kCand; ++c) red[tid][c] += red[tid + s][c];
    }
    __syncthreads();
  }
  if (tid < kCand && i0 + tid < n) total[i0 + tid] = red[0][tid];
}

__global__ __launch_bounds__(kThreads) void medoid_pick(const int32_t* __restrict__ assign,
                                                        const float* __restrict__ total, int64_t n,
                                                        int32_t E, int32_t* __restrict__ medoid) {
  __shared__ float bv[kThreads];
  __shared__ int64_t bi[kThreads];
  const int tid = threadIdx.x;
  for (int32_t e = 0; e < E; ++e) {
    float v = INFINITY;
    int64_t idx = -1;
    for (int64_t i = tid; i < n; i += kThreads) {
      if (assign[i] == e && (idx < 0 || total[i] < v)) {  // ascending i: ties keep the lower
        v = total[i];
        idx = i;
      }
    }
    bv[tid] = v;
    bi[tid] = idx;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) {
        const int64_t j = bi[tid + s];
        const bool take = j >= 0 && (bi[tid] < 0 || bv[tid + s] < bv[tid] ||
                                     (bv[tid + s] == bv[tid] && j < bi[tid]));
        if (take) {
          bv[tid] = bv[tid + s];
          bi[tid] = j;
        }
      }
      __syncthreads();
    }
    if (tid == 0) medoid[e] = (int32_t)bi[0];
    __syncthreads();
  }
}

}  // namespace

size_t kmeans_ws_bytes(int64_t n, int64_t dim, int32_t clusters) {
  const int64_t blocks = ceil_div(n, kBlockPoints);
  auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  return r256(sizeof(float) * (size_t)(blocks * clusters * dim)) +
         r256(sizeof(int32_t) * (size_t)(blocks * clusters));
}

int launch_nearest(const float* x, int64_t n, int64_t dim, const float* centroids,
                   int32_t clusters, int32_t* out, void* stream) {
  if (n <= 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TraceScope ts("nearest", st);
  hipLaunchKernelGGL(nearest_kernel, dim3((unsigned)ceil_div(n, kWaves)), dim3(kThreads), 0, st,
                     x, n, dim, centroids, clusters, out);
  return (int)hipGetLastError();
}

int launch_kmeans(const float* x, int64_t n, int64_t dim, int32_t clusters, const float* init,
                  int32_t rounds, float* centroids, int32_t* assign, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t cn = (int64_t)clusters * dim;
  {
    TraceScope ts("kmeans_init", st);
    hipLaunchKernelGGL(copy_f32, dim3((unsigned)ceil_div(cn, kThreads)), dim3(kThreads), 0, st,
                       init, centroids, cn);
  }
  if (n <= 0) return (int)hipGetLastError();
  const int64_t blocks = ceil_div(n, kBlockPoints);
  auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  float* psum = static_cast<float*>(ws);
  int32_t* pcnt = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                             r256(sizeof(float) * (size_t)(blocks * cn)));
  for (int32_t r = 0; r < rounds; ++r) {
    if (int e = launch_nearest(x, n, dim, centroids, clusters, assign, stream)) return e;
    {
      TraceScope ts("kmeans_partial", st);
      hipLaunchKernelGGL(centroid_partial, dim3((unsigned)blocks, (unsigned)ceil_div(dim, kSliceDims)),
                         dim3(kThreads), 0, st, x, n, dim, assign, clusters, psum, pcnt);
    }
    TraceScope ts("kmeans_final", st);
    hipLaunchKernelGGL(centroid_final, dim3((unsigned)ceil_div(dim, kThreads), (unsigned)clusters),
                       dim3(kThreads), 0, st, psum, pcnt, blocks, dim, clusters, centroids);
  }
  return launch_nearest(x, n, dim, centroids, clusters, assign, stream);
}

int launch_medoids(const float* x, int64_t n, int64_t dim, const int32_t* assign, int32_t clusters,
                   int32_t* medoid, float* totals, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n > 0) {
    TraceScope ts("medoid_total", st);
    hipLaunchKernelGGL(medoid_total, dim3((unsigned)ceil_div(n, kCand)), dim3(kThreads), 0, st,
                       x, n, dim, assign, totals);
  }
  TraceScope ts("medoid_pick", st);
  hipLaunchKernelGGL(medoid_pick, dim3(1), dim3(kThreads), 0, st, assign, totals, n, clusters,
                     medoid);
  return (int)hipGetLastError();
}

}  // namespace kvs
