// Attention scoring of appended queries over an fp32 cache (vector ALU).
//
// Same two-pass decomposition as the bf16 path (KV² summary, "무엇과 다른가"):
// pass 1 finds c2_j = log2 sum_i 2^(z_ji c1) for every query row over all N
// keys; pass 2 takes, for every position i of chunk C_r, the max over the
// chunk's rows of z_ji c1 - c2_j and exponentiates once.  fp32 inputs keep
// fp32 arithmetic end to end (a bf16 downcast would cost ~2^-9 relative per
// logit), so these kernels use fp32 FMAs rather than bf16 MFMA.
//
// Pass 1: one wave per query row; lane l walks keys l, l + 64, ... with its
// own running max and sum, and the wave merges the 64 pairs by log-sum-exp.
// Pass 2: a workgroup takes kP2Keys consecutive positions of a chunk and
// kP2Groups row groups; thread (group, key) takes the max over the rows
// j = group mod kP2Groups, and the groups' maxima meet in LDS.  (These paths
// serve small caches, where one thread per row or per position would leave
// the chip nearly idle: the 2,048-position fp32 workload has 512 rows.)
#include <math.h>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;

// Key rows of one slab: [0, split) at `head`, [split, N) at `tail` (row i at
// tail + (i - split) * D).
struct Keys {
  const float* kh;
  const float* kt;
  int64_t kh_stride, kt_stride, kt_row0, split;
};

__device__ __forceinline__ const float* key_row(const Keys& k, int64_t slab, int64_t i, int D) {
  return i < k.split ? k.kh + (slab * k.kh_stride + i) * D
                     : k.kt + (slab * k.kt_stride + k.kt_row0 + (i - k.split)) * D;
}

constexpr int kRowsPerBlock = kF32P1Rows;     // pass 1: one wave per row
static_assert(kRowsPerBlock * 64 == kThreads, "one wave per row");

template <int D>
__global__ __launch_bounds__(kThreads) void pass1_f32(const float* __restrict__ q, Keys keys,
                                                      float* __restrict__ c2, int64_t total_rows,
                                                      int64_t Nq, int64_t N, int32_t Hq,
                                                      int32_t Hkv, float c1) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= total_rows) return;  // the whole wave: this kernel has no barrier
  const int64_t h_all = row / Nq;                // l * Hq + h
  const int64_t l = h_all / Hq, h = h_all % Hq;
  const int64_t g = h / (Hq / Hkv);
  const float* qr = q + row * D;
  const int64_t slab = l * Hkv + g;
  float qv[D];
#pragma unroll
  for (int t = 0; t < D; ++t) qv[t] = qr[t];
  float m = -INFINITY, s = 0.f;
  // unrolled so that several key rows are in flight: the loop is bound by
  // their load latency, not by the FMAs
#pragma unroll 4
  for (int64_t i = lane; i < N; i += 64) {
    const float* kr = key_row(keys, slab, i, D);
    float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
#pragma unroll
    for (int t = 0; t < D; t += 4) {
      z0 = fmaf(qv[t], kr[t], z0);
      z1 = fmaf(qv[t + 1], kr[t + 1], z1);
      z2 = fmaf(qv[t + 2], kr[t + 2], z2);
      z3 = fmaf(qv[t + 3], kr[t + 3], z3);
    }
    const float z = ((z0 + z1) + (z2 + z3)) * c1;
    if (z > m) {
      s = s * exp2_hw(m - z) + 1.f;
      m = z;
    } else {
      s += exp2_hw(z - m);
    }
  }
  // log-sum-exp merge of the lanes' (max, sum); a lane without keys holds
  // (-inf, 0) and adds nothing
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float mo = __shfl_xor(m, off, 64);
    const float so = __shfl_xor(s, off, 64);
    const float M = fmaxf(m, mo);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    s = s * exp2_hw(m - Ms) + so * exp2_hw(mo - Ms);
    m = M;
  }
  if (lane == 0) c2[row] = m + log2f(s);
}

constexpr int kP2Keys = kF32P2Keys;           // pass 2: positions per workgroup
constexpr int kP2Groups = kThreads / kP2Keys;  // row groups per workgroup

template <int D>
__global__ __launch_bounds__(kThreads) void pass2_f32(const float* __restrict__ q, Keys keys,
                                                      const float* __restrict__ c2,
                                                      float* __restrict__ scores, int64_t Nq,
                                                      int64_t N, int64_t S, int64_t m_chunk,
                                                      int64_t nq, int64_t R, int64_t tiles,
                                                      int32_t Hq, int32_t Hkv, float c1) {
  __shared__ float part[kP2Groups][kP2Keys];
  const int64_t b = blockIdx.x;
  const int64_t tile = b % tiles;
  const int64_t r = (b / tiles) % R;
  const int64_t unit = b / (tiles * R);
  const int64_t l = unit / Hkv, g = unit % Hkv;
  const int32_t G = Hq / Hkv;
  const int64_t c0 = S + r * m_chunk;
  const int64_t c1e = min(c0 + m_chunk, N);
  float* srow = scores + unit * N;
  if (r == 0 && tile == 0) {
    const int64_t ns = min(S, N);
    for (int64_t i = threadIdx.x; i < ns; i += kThreads) srow[i] = 1.0f;
  }
  const int kk = threadIdx.x % kP2Keys, grp = threadIdx.x / kP2Keys;
  const int64_t key = c0 + tile * kP2Keys + kk;
  const bool live = key < c1e;
  // a position past the chunk reads the chunk's last key and is not written
  const float* kr = key_row(keys, l * Hkv + g, live ? key : c1e - 1, D);
  float kv[D];
#pragma unroll
  for (int t = 0; t < D; ++t) kv[t] = kr[t];
  const int64_t unit_row0 = (l * Hq + g * G) * Nq;
  const int64_t rows = (int64_t)G * nq;  // the chunk's rows: head jj / nq, query jj % nq
  float best = -INFINITY;
  for (int64_t jj = grp; jj < rows; jj += kP2Groups) {
    {
      const int64_t hh = jj / nq, j = jj - hh * nq;
      const int64_t row = unit_row0 + hh * Nq + r * nq + j;
      const float* qr = q + row * D;
      float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
#pragma unroll
      for (int t = 0; t < D; t += 4) {
        z0 = fmaf(qr[t], kv[t], z0);
        z1 = fmaf(qr[t + 1], kv[t + 1], z1);
        z2 = fmaf(qr[t + 2], kv[t + 2], z2);
        z3 = fmaf(qr[t + 3], kv[t + 3], z3);
      }
      const float z = ((z0 + z1) + (z2 + z3)) * c1;
      best = fmaxf(best, z - c2[row]);
    }
  }
  part[grp][kk] = best;
  __syncthreads();
  if (grp == 0 && live) {
    float v = part[0][kk];
#pragma unroll
    for (int gi = 1; gi < kP2Groups; ++gi) v = fmaxf(v, part[gi][kk]);
    srow[key] = fminf(exp2_hw(v), 1.0f);
  }
}

template <int D>
int run(const kvs_problem& p, const ScorePlan& pl, const void* q, const KvSrc& kv, float* scores,
        void* ws, hipStream_t st) {
  float* c2 = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_c2);
  const int64_t N = p.n_cache;
  const float c1 = (float)(1.4426950408889634 / sqrt((double)D));
  const float* qf = static_cast<const float*>(q);
  const Keys keys{static_cast<const float*>(kv.k_head), static_cast<const float*>(kv.k_tail),
                  kv.head_stride, kv.tail_stride, kv.tail_row0, kv.split};
  {
  TraceScope t1("score_pass1_f32", st);
  hipLaunchKernelGGL(pass1_f32<D>, dim3((unsigned)pl.row_blocks),
                     dim3(kThreads), 0, st, qf, keys, c2, pl.total_rows, pl.n_queries, N,
                     p.q_heads, p.kv_heads, c1);
  }
  if (hipError_t e = hipGetLastError()) return (int)e;
  const int64_t tiles = pl.p2_tiles;  // kP2Keys positions each, over the longest chunk
  {
  TraceScope t2("score_pass2_f32", st);
  hipLaunchKernelGGL(pass2_f32<D>, dim3((unsigned)(pl.units * pl.n_chunks * tiles)),
                     dim3(kThreads), 0, st, qf, keys, c2, scores, pl.n_queries, N, p.n_sinks,
                     p.chunk_size, p.q_per_chunk, pl.n_chunks, tiles, p.q_heads, p.kv_heads, c1);
  }
  if (hipError_t e = hipGetLastError()) return (int)e;
  return 0;
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float* dst, int64_t n, float value) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = value;
}

}  // namespace

int launch_score_f32(const kvs_problem& p, const ScorePlan& pl, const void* q, const KvSrc& kv,
                     float* scores, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.head_dim == 128) return run<128>(p, pl, q, kv, scores, ws, st);
  return run<64>(p, pl, q, kv, scores, ws, st);
}

int launch_fill(float* dst, int64_t n, float value, void* stream) {
  if (n <= 0) return 0;
  TraceScope ts("fill", static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)ceil_div(n, kThreads)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), dst, n, value);
  return (int)hipGetLastError();
}

}  // namespace kvs
