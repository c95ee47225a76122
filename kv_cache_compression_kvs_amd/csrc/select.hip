// Top-k selection per (layer, KV head) (KV² summary, "무엇과 다른가": after the
// sinks are pinned, the lowest-scoring positions are evicted down to the budget).
//
// One 1024-thread workgroup owns one (layer, KV head).  The candidates are the
// positions [S, N); we need the k - S best under the order (score descending,
// position ascending), listed ascending together with the sinks [0, S).
//
//  1. Scores become order-preserving 32-bit keys (sign-magnitude flip, -0 read
//     as +0).  When N - S fits, the keys are cached in LDS; otherwise every
//     pass re-reads them from global memory (L2 / MALL resident).
//  2. MSB-first radix select in four 8-bit rounds finds the exact key tau of
//     the (k - S)-th best candidate and e, the number of candidates equal to
//     tau that must be kept (the lowest positions among the ties).
//     Histograms live in LDS, one per wave (no contention between waves),
//     summed per bin before the digit is picked.  Each thread loads a batch
//     of keys before counting any, so uncached passes keep many loads in
//     flight instead of waiting on one at a time.
//  3. One ordered sweep writes the output: a block-wide scan of packed
//     (count above tau, count equal to tau) per thread gives each kept
//     position its rank: S + above_before + min(equal_before, e).
// Integer-only atomics on counts: the result does not depend on scheduling.
#include <algorithm>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 16;                // consecutive candidates per thread in the sweep
constexpr int kBatch = 8;                 // candidates per thread per histogram iteration
constexpr int64_t kLdsKeys = 32 * 1024;   // candidates cached in LDS (128 KiB)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SelArgs {
  const float* scores;
  int32_t* kept;
  int64_t N, S;
  int32_t Hkv;
  LayerTable t;
};

// Inclusive scan over the 1024 threads; returns the block total in *total.
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t v = lane < kWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const uint32_t y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane < kWaves) wsum[kWaves + lane] = v;  // inclusive wave prefix
  }
  __syncthreads();
  if (wave > 0) x += wsum[kWaves + wave - 1];
  *total = wsum[2 * kWaves - 1];
  __syncthreads();  // wsum is reused by the next call
  return x;
}

// Radix select and ordered sweep over the nc candidates of one (layer, KV
// head), keys read from the LDS cache (CACHED) or from global memory.  The
// choice is made once per workgroup so that no key load sits behind a
// per-element branch: every load is unconditional, from a clamped position.
//
// Writes the ranks 0 .. need-1 of out: the chosen candidates' positions val0 + i,
// ascending.
template <bool CACHED>
__device__ __forceinline__ void select_body(const float* srow, const uint32_t* keys, uint32_t* hw,
                                            uint32_t* wsum, uint32_t* pick, int32_t* out,
                                            int64_t nc, int64_t need, int64_t val0) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto key_at = [&](int64_t i) __attribute__((always_inline)) -> uint32_t {
    return CACHED ? keys[i] : order_key(srow[i]);
  };

  uint32_t tau = 0u;
  uint32_t e = 0u;
  if (need >= nc) {
    tau = 0u;                 // every candidate is kept
    e = (uint32_t)nc;
  } else {
    uint32_t prefix = 0u, mask = 0u;
    uint32_t rem = (uint32_t)need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < kWaves * 256; b += kThreads) hw[b] = 0u;
      __syncthreads();
      // One histogram per wave, so waves never contend; lanes of a wave that
      // hit the same bin are serialised by the LDS atomic unit.  kBatch
      // candidates per thread (coalesced, kThreads apart) are loaded before
      // any is counted, so that many loads are in flight when the keys come
      // from global memory.
      uint32_t* mine = hw + wave * 256;
      for (int64_t base = 0; base < nc; base += (int64_t)kThreads * kBatch) {
        uint32_t xs[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) xs[j] = key_at(min(base + (int64_t)j * kThreads + tid, nc - 1));
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int64_t i = base + (int64_t)j * kThreads + tid;
          bool active = i < nc && (xs[j] & mask) == prefix;
          const uint32_t bin = (xs[j] >> shift) & 255u;
          // Scores cluster, so most active lanes usually share one bin: count
          // the first active lane's bin for the whole wave with one atomic,
          // then the remaining lanes individually.
          const uint64_t act = __ballot(active);
          if (act != 0ull) {
            const int leader = __ffsll((unsigned long long)act) - 1;
            const uint32_t lb = __shfl(bin, leader, 64);
            const uint64_t same = __ballot(active && bin == lb);
            if (lane == leader) atomicAdd(&mine[lb], (uint32_t)__popcll(same));
            if (active && bin != lb) atomicAdd(&mine[bin], 1u);
          }
        }
      }
      __syncthreads();
      // counts from the top bin down; the digit is where the running count reaches rem
      uint32_t c = 0u;
      if (tid < 256) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += hw[w * 256 + 255 - tid];
      }
      uint32_t tot;
      const uint32_t cum = block_scan(c, wsum, &tot);
      if (tid < 256 && cum >= rem && cum - c < rem) {
        pick[0] = 255u - (uint32_t)tid;
        pick[1] = cum - c;
      }
      __syncthreads();
      prefix |= pick[0] << shift;
      mask |= 255u << shift;
      rem -= pick[1];
      __syncthreads();  // pick is rewritten next round
    }
    tau = prefix;
    e = rem;
  }

  // ordered sweep: kItems consecutive candidates per thread
  uint64_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < nc; base += (int64_t)kThreads * kItems) {
    const int64_t i0 = base + (int64_t)tid * kItems;
    uint32_t x[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) x[j] = key_at(min(i0 + j, nc - 1));
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      if (i0 + j < nc) {
        ngt += x[j] > tau;
        neq += x[j] == tau;
      }
    }
    const uint32_t packed = (ngt << 16) | neq;
    uint32_t tot;
    const uint32_t incl = block_scan(packed, wsum, &tot);
    const uint32_t excl = incl - packed;
    uint64_t gt_before = run_gt + (excl >> 16);
    uint64_t eq_before = run_eq + (excl & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t i = i0 + j;
      // ranks are < need by construction; the bound check only keeps a
      // counting error from ever writing outside this list
      if (i < nc && x[j] > tau) {
        const uint64_t rank = gt_before + (eq_before < e ? eq_before : e);
        if (rank < (uint64_t)need) out[rank] = (int32_t)(val0 + i);
        ++gt_before;
      } else if (i < nc && x[j] == tau) {
        const uint64_t rank = gt_before + eq_before;
        if (eq_before < e && rank < (uint64_t)need) out[rank] = (int32_t)(val0 + i);
        ++eq_before;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
}

// One workgroup per (layer, KV head).  CACHED: the candidates fit the LDS key
// cache.  Otherwise the keys are read from global memory in every pass and
// the kernel needs only the histograms' 16 KiB of LDS, so two workgroups fit
// on a CU.
template <bool CACHED>
__global__ __launch_bounds__(kThreads) void select_kernel(SelArgs a) {
  __shared__ uint32_t keys[CACHED ? kLdsKeys : 1];
  __shared__ uint32_t hw[kWaves * 256];
  __shared__ uint32_t wsum[2 * kWaves];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int64_t l = unit / a.Hkv, g = unit % a.Hkv;
  const int64_t kl = a.t.k[l];
  const int64_t N = a.N;
  const int64_t S = a.S < N ? a.S : N;
  const float* srow = a.scores + unit * N + S;
  int32_t* out = a.kept + a.t.off[l] + g * kl;
  const int64_t nc = N - S;
  const int64_t need = kl - S;

  for (int64_t i = tid; i < S; i += kThreads) out[i] = (int32_t)i;
  if (need <= 0) return;  // only the sinks (uniform: no barrier skipped by part of the group)

  if (CACHED) {
    for (int64_t i = tid; i < nc; i += kThreads) keys[i] = order_key(srow[i]);
    __syncthreads();
  }
  select_body<CACHED>(srow, keys, hw, wsum, pick, out + S, nc, need, S);
}

// Stage-1 query selection (KV² summary, "어떻게 동작하나"): token score =
// mean over layers and KV heads of the per-head scores, ranked by the float32
// sum over the units in layer-major order (the same order as the mean, up to
// rounding, with a rounding both sides can reproduce).  One thread per
// position; a batch of units is loaded before any is added.
constexpr int kSumThreads = 256;
constexpr int kSumBatch = 8;

__global__ __launch_bounds__(kSumThreads) void unit_sum_kernel(const float* __restrict__ scores,
                                                               float* __restrict__ psum, int64_t N,
                                                               int64_t S, int64_t units) {
  const int64_t i = S + (int64_t)blockIdx.x * kSumThreads + threadIdx.x;
  if (i >= N) return;
  const float* col = scores + i;
  float acc = 0.f;
  int64_t u = 0;
  for (; u + kSumBatch <= units; u += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) v[j] = col[(u + j) * N];
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) acc += v[j];
  }
  for (; u < units; ++u) acc += col[u * N];
  psum[i - S] = acc;
}

// Per chunk r: the n_q = max(floor(rho |C_r|), 1) positions with the largest
// token score (ties to the lower position), ascending, at offset r * n_q of a
// full chunk.  One workgroup per chunk.
struct QueryArgs {
  const float* psum;   // token sums of positions [S, N)
  int32_t* out;
  int64_t N, S, m;
  double rho;
};

__device__ __forceinline__ int64_t n_queries_of(double rho, int64_t len) {
  const int64_t n = (int64_t)floor(rho * (double)len);
  return n > 1 ? n : 1;
}

template <bool CACHED>
__global__ __launch_bounds__(kThreads) void query_select_kernel(QueryArgs a) {
  __shared__ uint32_t keys[CACHED ? kLdsKeys : 1];
  __shared__ uint32_t hw[kWaves * 256];
  __shared__ uint32_t wsum[2 * kWaves];
  __shared__ uint32_t pick[2];
  const int64_t r = blockIdx.x;
  const int64_t c0 = a.S + r * a.m;
  const int64_t len = min(a.m, a.N - c0);
  const int64_t nq = n_queries_of(a.rho, len);
  const float* srow = a.psum + (c0 - a.S);
  int32_t* out = a.out + r * n_queries_of(a.rho, a.m);
  if (CACHED) {
    for (int64_t i = threadIdx.x; i < len; i += kThreads) keys[i] = order_key(srow[i]);
    __syncthreads();
  }
  select_body<CACHED>(srow, keys, hw, wsum, pick, out, len, nq, c0);
}

}  // namespace

int launch_select(const kvs_problem& p, const float* scores, const LayerTable& t,
                  int32_t* kept, void* stream) {
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  if (units <= 0 || p.n_cache <= 0) return 0;
  SelArgs a;
  a.scores = scores;
  a.kept = kept;
  a.N = p.n_cache;
  a.S = p.n_sinks;
  a.Hkv = p.kv_heads;
  a.t = t;
  const int64_t nc = p.n_cache - std::min(p.n_sinks, p.n_cache);
  TraceScope ts("select", static_cast<hipStream_t>(stream));
  if (nc <= kLdsKeys)
    hipLaunchKernelGGL(select_kernel<true>, dim3((unsigned)units), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3((unsigned)units), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_query_select(const kvs_problem& p, const float* scores, double rho, int32_t* out,
                        float* psum, void* stream) {
  const int64_t N = p.n_cache, S = std::min(p.n_sinks, p.n_cache);
  if (N <= S) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  {
    TraceScope ts("query_token_sum", st);
    hipLaunchKernelGGL(unit_sum_kernel, dim3((unsigned)ceil_div(N - S, kSumThreads)),
                       dim3(kSumThreads), 0, st, scores, psum, N, S, units);
  }
  if (hipError_t e = hipGetLastError()) return (int)e;
  QueryArgs a;
  a.psum = psum;
  a.out = out;
  a.N = N;
  a.S = S;
  a.m = p.chunk_size;
  a.rho = rho;
  const int64_t R = ceil_div(N - S, p.chunk_size);
  TraceScope ts("query_select", st);
  if (std::min(p.chunk_size, N - S) <= kLdsKeys)
    hipLaunchKernelGGL(query_select_kernel<true>, dim3((unsigned)R), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(query_select_kernel<false>, dim3((unsigned)R), dim3(kThreads), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace kvs
