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
//   medoid_order     one workgroup: a stable counting sort of the points by
//                    cluster, so that each cluster is one run of positions.
//   medoid_tile      pairwise distances in 64 x 64 tiles of sorted positions,
//                    only for the tile pairs I <= J whose cluster ranges
//                    overlap; each distance of a same-cluster pair is formed
//                    once and added to both of its points' sums.
//   medoid_sum       a point's total over the tiles that hold its cluster, in
//                    tile order.
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
constexpr int kBatch = 32;         // points whose loads centroid_partial issues together
constexpr int kSliceDims = 1024;   // dimensions per centroid_partial workgroup

__global__ __launch_bounds__(kThreads) void nearest_kernel(const float* __restrict__ x, int64_t n,
                                                           int64_t D, const float* __restrict__ c,
                                                           int32_t E, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (i >= n) return;  // a whole wave
  // the lane's pieces of the row (dimensions 4 lane + 256 p .. +3), loaded once
  constexpr int kPieces = (int)(kMaxEmbedDim / 256);
  const float* xr = x + i * D;
  float4 xa[kPieces];
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int64_t k = 4 * lane + 256 * p;
    if (k < D) xa[p] = *reinterpret_cast<const float4*>(xr + k);
  }
  float best = INFINITY;
  int32_t arg = 0;
  for (int32_t e = 0; e < E; ++e) {
    const float* cr = c + (int64_t)e * D;
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int64_t k = 4 * lane + 256 * p;
      if (k >= D) break;
      const float4 a = xa[p];
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
  // points in index order, their loads issued kBatch at a time so that the
  // batch's latencies overlap
  const int64_t p0 = blk * kBlockPoints, p1 = min(p0 + kBlockPoints, n);
  for (int64_t i0 = p0; i0 < p1; i0 += kBatch) {
    int32_t a[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + u;
      a[u] = i < p1 ? assign[i] : -1;
      if (mine && i < p1) v[u] = *reinterpret_cast<const float4*>(x + i * D + d0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (a[u] < 0) continue;
      if (mine) {
        acc[a[u]][4 * tid + 0] += v[u].x;
        acc[a[u]][4 * tid + 1] += v[u].y;
        acc[a[u]][4 * tid + 2] += v[u].z;
        acc[a[u]][4 * tid + 3] += v[u].w;
      }
#pragma unroll
      for (int e = 0; e < kMaxClusters; ++e) cnt[e] += a[u] == e;
    }
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
#pragma unroll 8
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

// Medoid totals: total_i = sum over the members j of i's cluster of |x_i - x_j|.
// Positions are grouped into tiles of kTile; a tile pair (I, J), I <= J, is
// formed when the two tiles hold a common group.
constexpr int kTile = 32;
constexpr int kOrderThreads = 1024;
constexpr int kGroups = kMaxClusters + 1;

// medoid_order sorts the points by cluster, stably (one workgroup, chunks of
// 1024 points in index order; a point's place is its cluster's running start
// plus the count of same-cluster points before it in the chunk, from per-wave
// ballots).  Outputs: perm[p], the point at sorted position p; skey[p], its
// group; cstart[g], the first position of group g.  Groups are the clusters
// and, last, every label outside [0, clusters), so perm is always a full
// permutation; the distance sums still compare the labels themselves.
// It also lists the tile pairs to form: tile I pairs with the tiles J from I
// up to the one holding the last position of I's last group, and pstart[I] is
// the number of pairs of the tiles before I (pstart[tiles] = all of them).
__global__ __launch_bounds__(kOrderThreads) void medoid_order(const int32_t* __restrict__ assign,
                                                              int64_t n, int32_t E,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ skey,
                                                              int32_t* __restrict__ cstart,
                                                              uint32_t* __restrict__ pstart) {
  constexpr int W = kOrderThreads / 64;
  __shared__ uint32_t wc[W][kGroups];      // per wave and group: count in the current chunk
  __shared__ uint32_t base[kGroups];       // per group: next free position
  __shared__ uint32_t gstart[kGroups + 1]; // per group: first position; [E + 1] = n
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one
  auto group = [&](int64_t i) __attribute__((always_inline)) -> int {
    if (i >= n) return -1;
    const int32_t a = assign[i];
    return (a >= 0 && a < E) ? a : E;
  };
  uint32_t total = 0;  // thread g <= E: size of group g
  for (int64_t c0 = 0; c0 < n; c0 += kOrderThreads) {
    const int g = group(c0 + tid);
    for (int k = 0; k <= E; ++k) {
      const uint64_t m = __ballot(g == k);
      if (lane == 0) wc[wave][k] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (tid <= E)
      for (int w = 0; w < W; ++w) total += wc[w][tid];
    __syncthreads();
  }
  if (tid <= E) wc[0][tid] = total;  // the group sizes, for thread 0's scan
  __syncthreads();
  if (tid == 0) {
    uint32_t s = 0;
    for (int k = 0; k <= E; ++k) {
      base[k] = s;
      gstart[k] = s;
      cstart[k] = (int32_t)s;
      s += wc[0][k];
    }
    gstart[E + 1] = s;  // n
    cstart[E + 1] = (int32_t)s;
  }
  __syncthreads();
  if (wave == 0) {  // the tile-pair list, one tile per lane, 64 tiles per step
    const int64_t tiles = ceil_div(n, kTile);
    uint32_t carry = 0;
    for (int64_t t0 = 0; t0 < tiles; t0 += 64) {
      const int64_t I = t0 + lane;
      uint32_t cnt = 0;
      if (I < tiles) {
        const uint32_t last = (uint32_t)min(I * kTile + kTile - 1, n - 1);
        int g = 0;
        while (gstart[g + 1] <= last) ++g;  // the group holding position `last`
        cnt = (uint32_t)((gstart[g + 1] - 1) / kTile - I + 1);
      }
      uint32_t inc = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, 64);
        if (lane >= off) inc += y;
      }
      if (I < tiles) pstart[I] = carry + inc - cnt;
      carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) pstart[tiles] = carry;
  }
  for (int64_t c0 = 0; c0 < n; c0 += kOrderThreads) {
    const int64_t i = c0 + tid;
    const int g = group(i);
    uint64_t mine = 0;
    for (int k = 0; k <= E; ++k) {
      const uint64_t m = __ballot(g == k);
      if (g == k) mine = m;
      if (lane == 0) wc[wave][k] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (g >= 0) {
      uint32_t pos = base[g] + (uint32_t)__popcll(mine & below);
      for (int w = 0; w < wave; ++w) pos += wc[w][g];
      perm[pos] = (int32_t)i;
      skey[pos] = g;
    }
    __syncthreads();
    if (tid <= E)
      for (int w = 0; w < W; ++w) base[tid] += wc[w][tid];
    __syncthreads();
  }
}

// One workgroup per listed tile pair (I, J), I <= J (workgroups past the list
// exit at once; the listed ones come first, so they spread over the chip).
// Thread (ty, tx) of the 16 x 16 grid owns the 2 x 2 pairs of rows ty, ty + 16
// of tile I and columns tx, tx + 16 of tile J.  The two tiles' rows stream
// through LDS in chunks of 64 dimensions (rows padded by 16 bytes, so the 16
// consecutive rows a quarter-wave reads fall in distinct banks); each step
// reads four dimensions of each of a thread's four rows as 16-byte words.
// Each chunk's global loads are issued into registers before the previous
// chunk is computed, so their latency hides behind it.  A same-cluster pair's
// distance goes to its row sum (rows of I, to part[J][p]) and, for I < J, to
// its column sum (rows of J, to part[I][p]): each distance is formed once and
// serves both points.
constexpr int kChunk = 64;
constexpr int kPad = kChunk + 4;
constexpr int kTileThreads = (kTile / 2) * (kTile / 2);
constexpr int kLoads = 2 * kTile * kChunk / 4 / kTileThreads;  // 16-byte loads per thread per chunk
static_assert(kLoads * kTileThreads * 4 == 2 * kTile * kChunk, "loader covers both tiles");

__global__ __launch_bounds__(kTileThreads) void medoid_tile(const float* __restrict__ x, int64_t n,
                                                            int64_t D,
                                                            const int32_t* __restrict__ assign,
                                                            const int32_t* __restrict__ perm,
                                                            const uint32_t* __restrict__ pstart,
                                                            int64_t tiles,
                                                            float* __restrict__ part) {
  constexpr int TS = kTile / 2;  // threads per tile side
  const uint32_t b = blockIdx.x;
  if (b >= pstart[tiles]) return;  // uniform
  int64_t lo = 0, hi = tiles - 1;  // the last tile I with pstart[I] <= b
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (pstart[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int64_t I = lo, J = I + (b - pstart[I]);
  const int64_t i0 = I * kTile, j0 = J * kTile;
  __shared__ __attribute__((aligned(16))) float xs[2][kTile][kPad];  // [tile I / J][row][dim]
  __shared__ float rbuf[TS][kTile];  // [tx][row of I]: row sums over the thread's columns
  __shared__ float cbuf[TS][kTile];  // [ty][row of J]: column sums over the thread's rows
  const int tid = threadIdx.x, tx = tid % TS, ty = tid / TS;
  // loader: load h of thread t copies dimensions 4 (L % CQ) .. +3 of the
  // chunk for row (L / CQ) % kTile of tile L / (CQ kTile), L = t + h kTileThreads
  constexpr int CQ = kChunk / 4;  // 16-byte pieces per row and chunk
  const float* lsrc[kLoads];
  float* ldst[kLoads];
  int ld[kLoads];
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    const int L = tid + h * kTileThreads;
    const int set = L / (CQ * kTile), row = (L / CQ) % kTile;
    ld[h] = (L % CQ) * 4;
    const int64_t pos = min((set ? j0 : i0) + row, n - 1);
    lsrc[h] = x + (int64_t)perm[pos] * D + ld[h];
    ldst[h] = &xs[set][row][ld[h]];
  }
  float4 pf[kLoads];
  auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < kLoads; ++h)
      pf[h] = k0 + ld[h] < D ? *reinterpret_cast<const float4*>(lsrc[h] + k0)  // D % 4 == 0
                             : float4{0.f, 0.f, 0.f, 0.f};
  };
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  fetch(0);
  for (int64_t k0 = 0; k0 < D; k0 += kChunk) {
#pragma unroll
    for (int h = 0; h < kLoads; ++h) *reinterpret_cast<float4*>(ldst[h]) = pf[h];
    __syncthreads();
    if (k0 + kChunk < D) fetch(k0 + kChunk);
#pragma unroll 4
    for (int k = 0; k < kChunk; k += 4) {
      const float4 a0 = *reinterpret_cast<const float4*>(&xs[0][ty][k]);
      const float4 a1 = *reinterpret_cast<const float4*>(&xs[0][ty + TS][k]);
      const float4 b0 = *reinterpret_cast<const float4*>(&xs[1][tx][k]);
      const float4 b1 = *reinterpret_cast<const float4*>(&xs[1][tx + TS][k]);
      const float av[2][4] = {{a0.x, a0.y, a0.z, a0.w}, {a1.x, a1.y, a1.z, a1.w}};
      const float bv[2][4] = {{b0.x, b0.y, b0.z, b0.w}, {b1.x, b1.y, b1.z, b1.w}};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float d = av[r][q] - bv[c][q];
            acc[r][c] = fmaf(d, d, acc[r][c]);
          }
    }
    __syncthreads();
  }
  int32_t ai[2], aj[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int64_t pi = i0 + ty + r * TS, pj = j0 + tx + r * TS;
    ai[r] = pi < n ? assign[perm[pi]] : -1;
    aj[r] = pj < n ? assign[perm[pj]] : -2;
  }
  float dist[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) dist[r][c] = ai[r] == aj[c] ? sqrtf(acc[r][c]) : 0.f;
#pragma unroll
  for (int r = 0; r < 2; ++r) rbuf[tx][ty + r * TS] = dist[r][0] + dist[r][1];
#pragma unroll
  for (int c = 0; c < 2; ++c) cbuf[ty][tx + c * TS] = dist[0][c] + dist[1][c];
  __syncthreads();
  if (tid < kTile) {
    float t = 0.f;
    for (int q = 0; q < TS; ++q) t += rbuf[q][tid];
    if (i0 + tid < n) part[J * n + i0 + tid] = t;
  } else if (tid < 2 * kTile && I < J) {
    const int col = tid - kTile;
    float t = 0.f;
    for (int q = 0; q < TS; ++q) t += cbuf[q][col];
    if (j0 + col < n) part[I * n + j0 + col] = t;
  }
}

// total[perm[p]] = sum of part[jt][p] over the tiles jt that hold p's group,
// in tile order.  Every such tile pair overlaps p's own tile, so medoid_tile
// wrote each of these entries.
__global__ __launch_bounds__(kThreads) void medoid_sum(const float* __restrict__ part, int64_t n,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ skey,
                                                       const int32_t* __restrict__ cstart,
                                                       float* __restrict__ total) {
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= n) return;
  const int g = skey[p];
  const int64_t t0 = cstart[g] / kTile, t1 = (cstart[g + 1] - 1) / kTile;
  float t = 0.f;
  for (int64_t jt = t0; jt <= t1; ++jt) t += part[jt * n + p];
  total[perm[p]] = t;
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

// Medoid workspace: part [tiles][n] f32 (tiles of kTile positions), then
// perm [n], skey [n], cstart [kGroups + 1] int32 and pstart [tiles + 1]
// uint32, each piece 256-byte aligned.
namespace {
struct MedoidWs {
  size_t off_perm, off_skey, off_cstart, off_pstart, bytes;
};
MedoidWs medoid_ws_layout(int64_t n) {
  auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  MedoidWs w;
  w.off_perm = r256(sizeof(float) * (size_t)(ceil_div(n, kTile) * n));
  w.off_skey = w.off_perm + r256(sizeof(int32_t) * (size_t)n);
  w.off_cstart = w.off_skey + r256(sizeof(int32_t) * (size_t)n);
  w.off_pstart = w.off_cstart + r256(sizeof(int32_t) * (kGroups + 1));
  w.bytes = w.off_pstart + r256(sizeof(uint32_t) * (size_t)(ceil_div(n, kTile) + 1));
  return w;
}
}  // namespace

int launch_medoids(const float* x, int64_t n, int64_t dim, const int32_t* assign, int32_t clusters,
                   int32_t* medoid, float* totals, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n > 0) {
    const int64_t tiles = ceil_div(n, kTile);
    const MedoidWs w = medoid_ws_layout(n);
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* part = reinterpret_cast<float*>(base);
    int32_t* perm = reinterpret_cast<int32_t*>(base + w.off_perm);
    int32_t* skey = reinterpret_cast<int32_t*>(base + w.off_skey);
    int32_t* cstart = reinterpret_cast<int32_t*>(base + w.off_cstart);
    uint32_t* pstart = reinterpret_cast<uint32_t*>(base + w.off_pstart);
    {
      TraceScope ts("medoid_order", st);
      hipLaunchKernelGGL(medoid_order, dim3(1), dim3(kOrderThreads), 0, st, assign, n, clusters,
                         perm, skey, cstart, pstart);
    }
    {
      // every tile pair I <= J at most; the list's length is known on the device only
      TraceScope ts("medoid_tile", st);
      hipLaunchKernelGGL(medoid_tile, dim3((unsigned)(tiles * (tiles + 1) / 2)), dim3(kTileThreads),
                         0, st, x, n, dim, assign, perm, pstart, tiles, part);
    }
    TraceScope ts("medoid_sum", st);
    hipLaunchKernelGGL(medoid_sum, dim3((unsigned)ceil_div(n, kThreads)), dim3(kThreads), 0, st,
                       part, n, perm, skey, cstart, totals);
  }
  TraceScope ts("medoid_pick", st);
  hipLaunchKernelGGL(medoid_pick, dim3(1), dim3(kThreads), 0, st, assign, totals, n, clusters,
                     medoid);
  return (int)hipGetLastError();
}

size_t medoid_ws_bytes(int64_t n) { return medoid_ws_layout(n).bytes; }

}  // namespace kvs
