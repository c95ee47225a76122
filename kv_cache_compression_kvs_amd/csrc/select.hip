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
//     Histograms live in LDS.  Scores cluster in a few exponents, so the top
//     byte has few distinct values: the first round aggregates equal bins
//     across a wave (ballot) before the LDS atomic.
//  3. One ordered sweep writes the output: a block-wide scan of packed
//     (count above tau, count equal to tau) per thread gives each kept
//     position its rank: S + above_before + min(equal_before, e).
// Integer-only atomics on counts: the result does not depend on scheduling.
#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 4;                 // consecutive candidates per thread in the sweep
constexpr int64_t kLdsKeys = 36 * 1024;   // candidates cached in LDS (144 KiB)

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

__global__ __launch_bounds__(kThreads) void select_kernel(SelArgs a) {
  __shared__ uint32_t keys[kLdsKeys];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[2 * kWaves];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x, lane = tid & 63;
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

  const bool cached = nc <= kLdsKeys;
  if (cached) {
    for (int64_t i = tid; i < nc; i += kThreads) keys[i] = order_key(srow[i]);
    __syncthreads();
  }
  auto key_at = [&](int64_t i) -> uint32_t { return cached ? keys[i] : order_key(srow[i]); };

  uint32_t tau = 0u;
  uint32_t e = 0u;
  if (need >= nc) {
    tau = 0u;                 // every candidate is kept
    e = (uint32_t)nc;
  } else {
    uint32_t prefix = 0u, mask = 0u;
    uint32_t rem = (uint32_t)need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int64_t base = 0; base < nc; base += kThreads) {
        const int64_t i = base + tid;
        bool active = false;
        uint32_t bin = 0u;
        if (i < nc) {
          const uint32_t x = key_at(i);
          active = (x & mask) == prefix;
          bin = (x >> shift) & 255u;
        }
        // Aggregate lanes that share a bin: all distinct bins in round one,
        // one pass (the most common case of a uniform wave) afterwards.
        const int passes = (shift == 24) ? 64 : 1;
        for (int it = 0; it < passes; ++it) {
          const uint64_t act = __ballot(active);
          if (act == 0ull) break;
          const int leader = __ffsll((unsigned long long)act) - 1;
          const uint32_t lb = __shfl(bin, leader, 64);
          const uint64_t same = __ballot(active && bin == lb);
          if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
          if (active && bin == lb) active = false;
        }
        if (active) atomicAdd(&hist[bin], 1u);
      }
      __syncthreads();
      // counts from the top bin down; the digit is where the running count reaches rem
      const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
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

  // ordered sweep
  uint64_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < nc; base += (int64_t)kThreads * kItems) {
    const int64_t i0 = base + (int64_t)tid * kItems;
    uint32_t x[kItems];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t i = i0 + j;
      x[j] = 0u;
      if (i < nc) {
        x[j] = key_at(i);
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
      if (i >= nc) break;
      // positions are < k by construction; the bound check only keeps a
      // counting error from ever writing outside this list
      if (x[j] > tau) {
        const uint64_t pos = (uint64_t)S + gt_before + (eq_before < e ? eq_before : e);
        if (pos < (uint64_t)kl) out[pos] = (int32_t)(S + i);
        ++gt_before;
      } else if (x[j] == tau) {
        const uint64_t pos = (uint64_t)S + gt_before + eq_before;
        if (eq_before < e && pos < (uint64_t)kl) out[pos] = (int32_t)(S + i);
        ++eq_before;
      }
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
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
  TraceScope ts("select", static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)units), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace kvs
