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
//   medoid_tile      pairwise distances in 64 x 64 tiles (4 x 4 pairs per
//                    thread, 32-dimension chunks staged in LDS), summed per row
//                    over the pairs that share a cluster; medoid_sum adds the
//                    tiles' row sums in a fixed order.
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
constexpr int kBlockPoints = 32;   // points per centroid_partial workgroup
constexpr int kSliceDims = 1024;   // dimensions per centroid_partial workgroup

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

// Pairwise distances in 64 x 64 tiles: thread (ty, tx) of the 16 x 16 grid owns
// the 4 x 4 pairs (i0 + 4 ty + r, j0 + 4 tx + c); the two row sets stream through
// LDS in chunks of 32 dimensions (stored transposed, so the inner loop reads
// four consecutive rows of one dimension as one 16-byte word).  Each pair adds
// its Euclidean distance to row i's sum if i and j share a cluster; a row's sum
// over the tile goes to part[j tile][i].
constexpr int kTile = 64;
constexpr int kChunk = 32;

__global__ __launch_bounds__(kThreads) void medoid_tile(const float* __restrict__ x, int64_t n,
                                                        int64_t D,
                                                        const int32_t* __restrict__ assign,
                                                        float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float xi[kChunk][kTile];
  __shared__ __attribute__((aligned(16))) float xj[kChunk][kTile];
  __shared__ float rsum[16][kTile];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t i0 = (int64_t)blockIdx.x * kTile, j0 = (int64_t)blockIdx.y * kTile;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  }
  // loader: thread t copies rows (t / 8) and (t / 8) + 32, dimensions
  // 4 * (t % 8) .. +3 of the chunk, for both row sets
  const int lr = tid >> 3, ld = (tid & 7) * 4;
  for (int64_t k0 = 0; k0 < D; k0 += kChunk) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = lr + 32 * h;
      const int64_t gi = min(i0 + row, n - 1), gj = min(j0 + row, n - 1);
      const bool in_d = k0 + ld < D;  // D is a multiple of 4
      float4 a = in_d ? *reinterpret_cast<const float4*>(x + gi * D + k0 + ld) : float4{0, 0, 0, 0};
      float4 b = in_d ? *reinterpret_cast<const float4*>(x + gj * D + k0 + ld) : float4{0, 0, 0, 0};
      xi[ld + 0][row] = a.x;
      xi[ld + 1][row] = a.y;
      xi[ld + 2][row] = a.z;
      xi[ld + 3][row] = a.w;
      xj[ld + 0][row] = b.x;
      xj[ld + 1][row] = b.y;
      xj[ld + 2][row] = b.z;
      xj[ld + 3][row] = b.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kChunk; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&xi[k][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&xj[k][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float d = av[r] - bv[c];
          acc[r][c] = fmaf(d, d, acc[r][c]);
        }
      }
    }
    __syncthreads();
  }
  int32_t ai[4], aj[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = i0 + ty * 4 + r, j = j0 + tx * 4 + r;
    ai[r] = i < n ? assign[i] : -1;
    aj[r] = j < n ? assign[j] : -2;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (ai[r] == aj[c]) t += sqrtf(acc[r][c]);
    rsum[tx][ty * 4 + r] = t;
  }
  __syncthreads();
  if (tid < kTile) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t += rsum[q][tid];
    if (i0 + tid < n) part[(int64_t)blockIdx.y * n + i0 + tid] = t;
  }
}

// total[i] = sum over the j tiles of part[jt][i], in tile order.
__global__ __launch_bounds__(kThreads) void medoid_sum(const float* __restrict__ part, int64_t n,
                                                       int64_t jtiles, float* __restrict__ total) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  float t = 0.f;
  for (int64_t jt = 0; jt < jtiles; ++jt) t += part[jt * n + i];
  total[i] = t;
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
                   int32_t* medoid, float* totals, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n > 0) {
    const int64_t tiles = ceil_div(n, kTile);
    float* part = static_cast<float*>(ws);
    {
      TraceScope ts("medoid_tile", st);
      hipLaunchKernelGGL(medoid_tile, dim3((unsigned)tiles, (unsigned)tiles), dim3(kThreads), 0, st,
                         x, n, dim, assign, part);
    }
    TraceScope ts("medoid_sum", st);
    hipLaunchKernelGGL(medoid_sum, dim3((unsigned)ceil_div(n, kThreads)), dim3(kThreads), 0, st,
                       part, n, tiles, totals);
  }
  TraceScope ts("medoid_pick", st);
  hipLaunchKernelGGL(medoid_pick, dim3(1), dim3(kThreads), 0, st, assign, totals, n, clusters,
                     medoid);
  return (int)hipGetLastError();
}

size_t medoid_ws_bytes(int64_t n) {
  return ((size_t)sizeof(float) * (size_t)(ceil_div(n, kTile) * n) + 255) & ~size_t(255);
}

}  // namespace kvs
