// Top-k selection per (layer, KV head) (KV² summary, "무엇과 다른가": after the
// sinks are pinned, the lowest-scoring positions are evicted down to the budget).
//
// The candidates are the positions [S, N); we need the k - S best under the
// order (score descending, position ascending), listed ascending together
// with the sinks [0, S).  Up to 32K candidates per (layer, KV head), one
// 1024-thread workgroup owns one (layer, KV head) with its keys cached in
// LDS; up to 128K candidates a 512-thread workgroup per (layer, KV head)
// streams the keys twice (further below), and longer caches and the global
// eviction use the multi-workgroup select at the end.
//
//  1. Scores become order-preserving 32-bit keys (sign-magnitude flip, -0 read
//     as +0), cached in LDS (the query selection's chunks can exceed the cache;
//     then every pass re-reads them from global memory, L2 / MALL resident).
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
#include <type_traits>

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
static_assert(kLdsKeys == kSelSingleMax, "longer units go to the multi-workgroup select");

// Order-preserving 32-bit key of a score: -0 reads as +0, and every NaN
// (either sign, any payload) takes the one key above that of +inf, so NaNs
// tie with each other and the lower position wins among them.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFFFFFu;
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

// Inclusive scan over the NT threads of the workgroup (wsum holds 2 * NT / 64
// words); returns the block total in *total.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
  constexpr int kWaves = NT / 64;
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

// Adds one count per active lane to hist[bin] (a histogram in LDS).  Scores
// cluster, so most of a wave's active lanes usually share one bin: the lowest
// active lane's bin is counted for every lane that shares it with one atomic;
// the lanes left after that add individually.  (Peeling up to four bins this
// way measured slower on the 32K-candidate select: 80 against 69 us.)
constexpr int kPeel = 1;

__device__ __forceinline__ void wave_count(uint32_t* hist, bool active, uint32_t bin, int lane) {
  uint64_t act = __ballot(active);
#pragma unroll
  for (int r = 0; r < kPeel; ++r) {
    if (act == 0ull) return;  // the same on every lane
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = act & __ballot(bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    act &= ~same;
  }
  if ((act >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Word of the LDS key cache that holds candidate i.  Within each 16-word
// group the low 4 bits are XORed with bits 5-8 of i, so that the ordered
// sweep's reads (thread t takes kItems = 16 consecutive candidates, 16 words
// apart from its neighbour's) spread over the banks instead of piling onto a
// few, while the coalesced reads of consecutive candidates stay conflict-free.
__device__ __forceinline__ int64_t kswz(int64_t i) { return i ^ ((i >> 5) & 15); }
static_assert(kItems == 16, "the key cache swizzle is laid out for 16 candidates per thread");

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
    return CACHED ? keys[kswz(i)] : order_key(srow[i]);
  };

  // The candidates kept are those whose key, masked by tmask, is above tau,
  // and the first e (by position) of those equal to it.
  uint32_t tau = 0u, tmask = 0xFFFFFFFFu;
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
          wave_count(mine, i < nc && (xs[j] & mask) == prefix, (xs[j] >> shift) & 255u, lane);
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
        pick[2] = c;  // candidates in the chosen bin
      }
      __syncthreads();
      prefix |= pick[0] << shift;
      mask |= 255u << shift;
      rem -= pick[1];
      // Every candidate of the chosen bin is kept: the keys above the bin and
      // the whole bin are exactly the need best, and the lower digits need not
      // be resolved.  (Equal keys share every bin, so no tie is split.)
      const bool whole_bin = pick[2] == rem;
      __syncthreads();  // pick is rewritten next round
      if (whole_bin) break;  // uniform: every thread read the same pick
    }
    tau = prefix;
    tmask = mask;
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
        ngt += (x[j] & tmask) > tau;
        neq += (x[j] & tmask) == tau;
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
      if (i < nc && (x[j] & tmask) > tau) {
        const uint64_t rank = gt_before + (eq_before < e ? eq_before : e);
        if (rank < (uint64_t)need) out[rank] = (int32_t)(val0 + i);
        ++gt_before;
      } else if (i < nc && (x[j] & tmask) == tau) {
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
  __shared__ uint32_t pick[3];

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
    for (int64_t i = tid; i < nc; i += kThreads) keys[kswz(i)] = order_key(srow[i]);
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
  __shared__ uint32_t pick[3];
  const int64_t r = blockIdx.x;
  const int64_t c0 = a.S + r * a.m;
  const int64_t len = min(a.m, a.N - c0);
  const int64_t nq = n_queries_of(a.rho, len);
  const float* srow = a.psum + (c0 - a.S);
  int32_t* out = a.out + r * n_queries_of(a.rho, a.m);
  if (CACHED) {
    for (int64_t i = threadIdx.x; i < len; i += kThreads) keys[kswz(i)] = order_key(srow[i]);
    __syncthreads();
  }
  select_body<CACHED>(srow, keys, hw, wsum, pick, out, len, nq, c0);
}


// ---------------------------------------------------------------------------
// Per-unit select for long caches: kSelLongMin < candidates <= kLongMax.
//
// One 512-thread workgroup per (layer, KV head).  The cost of a pass over the
// unit's keys is the work per key, which one CU does alone, so the common
// path streams the keys once with a few operations per key:
//   sample  8K keys (512 blocks of 16 consecutive positions, evenly spread,
//           held in registers) are histogrammed on their top 12 bits and then,
//           inside the two bins that matter, on the next 10.  That brackets
//           the keys whose rank in the sample lies within 4 standard
//           deviations (binomial) of the expected rank of tau, the need-th
//           best: thresholds Thi (upper, inclusive) and Tlo (lower, inclusive).
//   pass    every key above Thi is marked in a bitmap of the unit's candidates
//           (one ballot per 64 consecutive keys) and counted; the keys in
//           [Tlo, Thi] are counted and stored in LDS with their positions, one
//           region per wave.
// The counts are exact: if fewer than need keys lie above Thi and at least
// need lie at or above Tlo, and every region held its keys, then tau is among
// the stored keys.  Otherwise (heavy ties, or a sample far from the data) the
// kernel starts over without the sample: histograms of the keys' top 12 bits,
// then the next 10 and the last 10 (one read each, as far as needed) give the
// bin of tau, and one more read marks the keys above it and stores or marks
// the bin.  Either way an 8-bit radix select over the stored keys gives tau
// and e (the number of keys equal to tau that are kept); stored keys above tau
// join the bitmap and those equal to it a second one, and an ordered sweep
// over the bitmaps (consecutive words per thread, a block scan of the counts)
// writes every marked-above position and the e lowest tied ones, ascending.
// The sample only steers the work; the result does not depend on it.
constexpr int kLT = 512;
constexpr int kLW = kLT / 64;
constexpr int kLBatch = 16;                 // keys per thread per streaming step
constexpr int64_t kLongMax = kSelLongMax;   // candidates per unit (bitmaps of 16 KiB each)
constexpr int kLongWords = (int)(kLongMax / 32);
constexpr int kCandMax = 5120;              // (key, position) pairs stored in LDS
constexpr int kRegion = kCandMax / kLW;     // store region of one wave in the sampled pass
constexpr int kSampleBlocks = 512;          // sampled blocks of 16 consecutive keys
constexpr int kSampleKeys = kSampleBlocks * 16;
constexpr int kSPT = kSampleKeys / kLT;     // sampled keys per thread
constexpr double kSigmas = 4.0;
static_assert(2 * kCandMax >= 4096 + 2 * 1024, "the sample histograms share the store");

// Calls f(i, v, valid) for the scores v of the keys [0, nc) in steps of
// kLT * kLBatch: key i = base + j * kLT + tid, so each wave covers 64
// consecutive keys per j.  Full steps use buffer loads at scalar offsets (the
// row is 4-byte aligned and every offset lies inside it); the ragged last
// step uses loads clamped into the row.  Each step's loads are issued before
// any of its keys is used.
template <typename F>
__device__ __forceinline__ void stream_scores(const float* srow, int64_t nc, F&& f) {
  const int tid = threadIdx.x;
  constexpr int kStep = kLT * kLBatch;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(srow), (short)0, (int)(nc * 4), kBufferFlags);
  const int nfull = (int)(nc / kStep);
  for (int st = 0; st < nfull; ++st) {
    uint32_t v[kLBatch];
#pragma unroll
    for (int j = 0; j < kLBatch; ++j)
      v[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, (st * kStep + j * kLT) * 4, 0);
#pragma unroll
    for (int j = 0; j < kLBatch; ++j) f((int64_t)st * kStep + j * kLT + tid, __uint_as_float(v[j]), true);
  }
  const int64_t base = (int64_t)nfull * kStep;
  if (base < nc) {
    float v[kLBatch];
#pragma unroll
    for (int j = 0; j < kLBatch; ++j) v[j] = srow[min(base + (int64_t)j * kLT + tid, nc - 1)];
#pragma unroll
    for (int j = 0; j < kLBatch; ++j) {
      const int64_t i = base + (int64_t)j * kLT + tid;
      f(i, v[j], i < nc);
    }
  }
}

// The smallest non-NaN float whose key is >= u, so that for every non-NaN x,
// order_key(x) >= u exactly when x >= it (NaN when no float qualifies: then
// the comparison is false for every x).
__device__ __forceinline__ float key_floor_float(uint64_t u) {
  if (u <= 0x007FFFFFull) return -INFINITY;               // at or below the key of -inf
  if (u > 0xFF800000ull) return __uint_as_float(0x7FC00000u);  // above the key of +inf
  if (u >= 0x80000000ull) return __uint_as_float((uint32_t)u & 0x7FFFFFFFu);  // +0 .. +inf
  if (u == 0x7FFFFFFFull) return 0.f;                     // no key: -0 reads as +0
  return __uint_as_float(~(uint32_t)u);                  // negative floats
}

// Bin of the target-th largest key (1-based) of a histogram of nb bins, each
// thread summing nb / kLT consecutive bins from the top; writes (bin, count
// of the bins above it) to out[0..1].  Call with 1 <= target <= the total.
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t nb, uint32_t target,
                                         uint32_t* wsum, uint32_t* out) {
  const int tid = threadIdx.x;
  const uint32_t per = nb / kLT;
  uint32_t c = 0u;
  for (uint32_t q = 0; q < per; ++q) c += hist[nb - 1u - tid * per - q];
  uint32_t tot;
  const uint32_t cum = block_scan<kLT>(c, wsum, &tot);
  if (cum >= target && cum - c < target) {
    uint32_t run = cum - c;
    for (uint32_t q = 0; q < per; ++q) {
      const uint32_t bin = nb - 1u - tid * per - q;
      const uint32_t h = hist[bin];
      if (run + h >= target) {
        out[0] = bin;
        out[1] = run;
        break;
      }
      run += h;
    }
  }
}

// find_bin for two targets with one block scan (t1 or t2 zero: not wanted);
// writes (bin, count above) of t1 to out[0..1] and of t2 to out[2..3].
__device__ __forceinline__ void find_bin2(const uint32_t* hist, uint32_t nb, uint32_t t1, uint32_t t2,
                                          uint32_t* wsum, uint32_t* out) {
  const int tid = threadIdx.x;
  const uint32_t per = nb / kLT;
  uint32_t c = 0u;
  for (uint32_t q = 0; q < per; ++q) c += hist[nb - 1u - tid * per - q];
  uint32_t tot;
  const uint32_t cum = block_scan<kLT>(c, wsum, &tot);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t target = k ? t2 : t1;
    if (target != 0u && cum >= target && cum - c < target) {
      uint32_t run = cum - c;
      for (uint32_t q = 0; q < per; ++q) {
        const uint32_t bin = nb - 1u - tid * per - q;
        const uint32_t h = hist[bin];
        if (run + h >= target) {
          out[2 * k] = bin;
          out[2 * k + 1] = run;
          break;
        }
        run += h;
      }
    }
  }
}

// find_bin by one wave (lane l sums the nb / 64 bins nb-1-l*per .. from the
// top), with no workgroup barrier; the writing lane stores (bin, count above).
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, uint32_t nb, uint32_t target,
                                              uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t per = nb / 64;
  const uint32_t top = nb - 1u - (uint32_t)lane * per;  // this lane's highest bin
  uint32_t c = 0u;
  for (uint32_t q = 0; q < per; ++q) c += hist[top - q];
  uint32_t cum = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(cum, off, 64);
    if (lane >= off) cum += y;
  }
  if (cum >= target && cum - c < target) {
    uint32_t run = cum - c;
    for (uint32_t q = 0; q < per; ++q) {
      const uint32_t h = hist[top - q];
      if (run + h >= target) {
        out[0] = top - q;
        out[1] = run;
        break;
      }
      run += h;
    }
  }
}

// The 8-bit digit of a 256-bin histogram where the count from the top
// reaches rem, found by one wave (lane l holds bins 255-4l .. 252-4l): writes
// (digit, count of the bins above it) to out[0..1].  1 <= rem <= the total.
__device__ __forceinline__ void pick_digit_wave(const uint32_t* h8, uint32_t rem, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  uint32_t b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) b[q] = h8[255 - 4 * lane - q];
  const uint32_t c = b[0] + b[1] + b[2] + b[3];
  uint32_t cum = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(cum, off, 64);
    if (lane >= off) cum += y;
  }
  if (cum >= rem && cum - c < rem) {
    uint32_t run = cum - c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (run + b[q] >= rem) {
        out[0] = 255u - (uint32_t)(4 * lane + q);
        out[1] = run;
        break;
      }
      run += b[q];
    }
  }
}

// The need-th best key (tau) and e among the keys stored in per-wave regions
// (region w holds n[w] keys at keys + w * stride).  prefix / mask hold the
// bits already fixed (every stored key matches them) and rem the rank to
// find among the stored keys; 8-bit digits from bit s_top down.  On return
// prefix is tau and rem is e.
__device__ __forceinline__ void resolve_regions(const uint32_t* keys, int stride, const uint32_t* n,
                                                int s_top, uint32_t& prefix, uint32_t& mask,
                                                uint32_t& rem, uint32_t* h8, uint32_t* st) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* mine = keys + wave * stride;
  const uint32_t nw = n[wave];
  for (int s = s_top;; s -= 8) {
    const int sh = s > 0 ? s : 0;
    if (tid < 256) h8[tid] = 0u;
    __syncthreads();
    for (uint32_t b0 = 0; b0 < nw; b0 += 64) {
      const uint32_t i = b0 + lane;
      const bool in = i < nw;
      const uint32_t x = in ? mine[i] : 0u;
      wave_count(h8, in && (x & mask) == prefix, (x >> sh) & 255u, lane);
    }
    __syncthreads();
    if (wave == 0) pick_digit_wave(h8, rem, st);
    __syncthreads();
    prefix |= st[0] << sh;
    mask |= 255u << sh;
    rem -= st[1];
    if (sh == 0) break;
  }
}

// Two workgroups per CU (at most 128 VGPRs): more units than CUs still run in one round.
__global__ __launch_bounds__(kLT, 4) void select_long_kernel(SelArgs a) {
  __shared__ uint32_t store[2 * kCandMax];  // sample histograms, then keys | positions
  __shared__ __attribute__((aligned(8))) uint32_t gtb[kLongWords];  // candidates above tau
  __shared__ uint32_t eqb[kLongWords];      // candidates equal to tau
  __shared__ uint32_t h8[256];
  __shared__ uint32_t wsum[2 * kLW];
  __shared__ uint32_t cnt_s[2 * kLW];       // per wave: keys above the bracket, keys stored
  __shared__ uint32_t st[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t unit = blockIdx.x;
  const int64_t l = unit / a.Hkv, g = unit % a.Hkv;
  const int64_t kl = a.t.k[l];
  const int64_t N = a.N;
  const int64_t S = a.S < N ? a.S : N;
  const float* srow = a.scores + unit * N + S;
  int32_t* out = a.kept + a.t.off[l] + g * kl;
  const int64_t nc = N - S;  // in (kSelLongMin, kLongMax]
  const int64_t need = kl - S;

  for (int64_t i = tid; i < S; i += kLT) out[i] = (int32_t)i;
  if (need <= 0) return;  // only the sinks (uniform over the workgroup)
  int32_t* dst = out + S;
  if (need >= nc) {       // every candidate
    for (int64_t i = tid; i < nc; i += kLT) dst[i] = (int32_t)(S + i);
    return;
  }
  const int64_t words = (nc + 31) / 32;
  uint32_t prefix = 0u, mask = 0u, rem = 0u;
  bool sampled = true;

  // ---- sample: the bracket [Tlo, Thi] --------------------------------------
  // ranks (1-based, from the top) of the bracket's ends in the sample
  const double pk = (double)need / (double)nc;
  const double mu = pk * kSampleKeys;
  const double sd = sqrt(kSampleKeys * pk * (1.0 - pk));
  const int64_t r_hi = (int64_t)floor(mu - kSigmas * sd - 2.0);
  const int64_t r_lo = (int64_t)ceil(mu + kSigmas * sd + 2.0);
  const bool has_hi = r_hi >= 1;
  const bool has_lo = r_lo <= kSampleKeys;
  uint64_t Thi = 0xFFFFFFFFull, Tlo = 0ull;  // keys in [Tlo, Thi] are stored, above Thi marked
  if (has_hi || has_lo) {
    uint32_t sk[kSPT];
#pragma unroll
    for (int r = 0; r < kSPT; ++r) {
      const int j = r * kLT + tid;  // block j / 16, key j % 16
      const int64_t b0 = (int64_t)(j >> 4) * (nc - 16) / (kSampleBlocks - 1);
      sk[r] = order_key(srow[b0 + (j & 15)]);
    }
    uint32_t* h1 = store;          // 4096 bins
    uint32_t* h2a = store + 4096;  // 1024 bins inside the upper end's bin
    uint32_t* h2b = store + 5120;  // 1024 bins inside the lower end's bin
    for (int b = tid; b < 4096 + 2048; b += kLT) store[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSPT; ++r) wave_count(h1, true, sk[r] >> 20, lane);
    __syncthreads();
    find_bin2(h1, 4096u, has_hi ? (uint32_t)r_hi : 0u, has_lo ? (uint32_t)r_lo : 0u, wsum, st);
    __syncthreads();
    const uint32_t bin_hi = st[0], above_hi = st[1], bin_lo = st[2], above_lo = st[3];
#pragma unroll
    for (int r = 0; r < kSPT; ++r) {
      const uint32_t b = sk[r] >> 20, sub = (sk[r] >> 10) & 1023u;
      wave_count(h2a, has_hi && b == bin_hi, sub, lane);
      wave_count(h2b, has_lo && b == bin_lo, sub, lane);
    }
    __syncthreads();
    if (has_hi && wave == 0) find_bin_wave(h2a, 1024u, (uint32_t)r_hi - above_hi, st + 4);
    if (has_lo && wave == 1) find_bin_wave(h2b, 1024u, (uint32_t)r_lo - above_lo, st + 6);
    __syncthreads();
    if (has_hi) Thi = (bin_hi << 20) | (st[4] << 10) | 1023u;
    if (has_lo) Tlo = (bin_lo << 20) | (st[6] << 10);
  }
  if (tid == 0) st[7] = 0u;  // set if the pass reads a NaN (read after the pass's barrier)
  for (int64_t w = tid; w < words; w += kLT) {
    gtb[w] = 0u;
    eqb[w] = 0u;
  }
  __syncthreads();  // st and store are rewritten below

  // ---- one pass: mark above Thi, store [Tlo, Thi] ----------------------------
  // For a non-NaN score x: key above Thi <=> x >= f_above, key >= Tlo <=> x >= f_lo.
  // A NaN fails both tests, so a unit with a NaN score is redone from its keys.
  // Stored keys hold the raw score bits until the pass ends.
  {
    const float f_above = key_floor_float(Thi + 1);
    const float f_lo = key_floor_float(Tlo);
    uint32_t n_ab = 0u, n_in = 0u;  // this wave's counts (uniform)
    uint64_t nan_w = 0ull;          // lanes that read a NaN score
    uint32_t* kreg = store + wave * kRegion;
    uint32_t* preg = store + kCandMax + wave * kRegion;
    // Steps of kPB keys per thread, double-buffered: the next step's loads are
    // in flight while this step's keys are compared.
    constexpr int kPB = kLBatch / 2;
    constexpr int kStep = kLT * kPB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(srow), (short)0, (int)(nc * 4), kBufferFlags);
    const int nsteps = (int)((nc + kStep - 1) / kStep);
    auto load_step = [&](float (&v)[kPB], int sp) __attribute__((always_inline)) {
      const int64_t base = (int64_t)sp * kStep;
      if (base + kStep <= nc) {
#pragma unroll
        for (int j = 0; j < kPB; ++j)
          v[j] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
              rs, tid * 4, (int)(base + j * kLT) * 4, 0));
      } else {
#pragma unroll
        for (int j = 0; j < kPB; ++j) v[j] = srow[min(base + (int64_t)j * kLT + tid, nc - 1)];
      }
    };
    // FULL: every key of the step lies inside the row (a compile-time fact,
    // so full steps carry no per-key bounds test).
    auto use_step = [&](auto full_tag, const float (&v)[kPB], int sp) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
      const int64_t base = (int64_t)sp * kStep;
      // lane q of words_v holds bitmap word q of this step's 2 * kPB words of this
      // wave: keys base + (q / 2) * kLT + wave * 64 + 32 * (q % 2) .. + 31
      uint32_t words_v = 0u;
#pragma unroll
      for (int j = 0; j < kPB; ++j) {
        const int64_t i = base + (int64_t)j * kLT + tid;
        const bool valid = FULL || i < nc;
        const bool up = valid && v[j] >= f_above;
        const bool in = valid && v[j] >= f_lo && !(v[j] >= f_above);
        nan_w |= __ballot(v[j] != v[j]);  // a NaN compares false: the unit starts over below
        const uint64_t ab = __ballot(up);
        const uint64_t ib = __ballot(in);
        n_ab += (uint32_t)__popcll(ab);
        const uint32_t half = (lane & 1) ? (uint32_t)(ab >> 32) : (uint32_t)ab;
        if ((lane >> 1) == j) words_v = half;
        if (ib != 0ull) {
          if (in) {
            const uint32_t s = n_in + __builtin_amdgcn_mbcnt_hi((uint32_t)(ib >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)ib, 0u));
            if (s < (uint32_t)kRegion) {
              kreg[s] = __float_as_uint(v[j]);
              preg[s] = (uint32_t)i;
            }
          }
          n_in += (uint32_t)__popcll(ib);
        }
      }
      if (lane < 2 * kPB) {
        const int64_t w = base / 32 + (lane >> 1) * (kLT / 32) + wave * 2 + (lane & 1);
        if (w < words) gtb[w] = words_v;
      }
    };
    auto use_any = [&](const float (&v)[kPB], int sp) __attribute__((always_inline)) {
      if ((int64_t)(sp + 1) * kStep <= nc) use_step(std::true_type{}, v, sp);
      else use_step(std::false_type{}, v, sp);
    };
    float va[kPB], vb[kPB];
    load_step(va, 0);
    for (int sp = 0; sp < nsteps; sp += 2) {
      if (sp + 1 < nsteps) load_step(vb, sp + 1);
      use_any(va, sp);
      if (sp + 2 < nsteps) load_step(va, sp + 2);
      if (sp + 1 < nsteps) use_any(vb, sp + 1);
    }
    // raw score bits to keys
    for (uint32_t i = lane; i < min(n_in, (uint32_t)kRegion); i += 64) kreg[i] = order_key(__uint_as_float(kreg[i]));
    if (lane == 0) {
      cnt_s[wave] = n_ab;
      cnt_s[kLW + wave] = n_in;
      if (nan_w) st[7] = 1u;
    }
  }
  __syncthreads();
  {
    uint32_t above = 0u, inside = 0u;
#pragma unroll
    for (int w = 0; w < kLW; ++w) {
      above += cnt_s[w];
      inside += cnt_s[kLW + w];
      sampled = sampled && cnt_s[kLW + w] <= (uint32_t)kRegion;
    }
    sampled = sampled && st[7] == 0u;  // no NaN score (NaN keys order above +inf)
    sampled = sampled && above < (uint32_t)need && (uint64_t)above + inside >= (uint64_t)need;
    rem = (uint32_t)need - above;
  }

  if (sampled) {
    // bits shared by every key of [Tlo, Thi], in whole 8-bit digits
    const uint32_t common = (uint32_t)Tlo ^ (uint32_t)Thi;
    const int lead = common ? __builtin_clz(common) : 32;
    const int fixed = (lead / 8) * 8;
    mask = fixed ? (fixed == 32 ? 0xFFFFFFFFu : ~(0xFFFFFFFFu >> fixed)) : 0u;
    prefix = (uint32_t)Thi & mask;
    if (fixed < 32)
      resolve_regions(store, kRegion, cnt_s + kLW, 24 - fixed, prefix, mask, rem, h8, st);
    const uint32_t nw = cnt_s[kLW + wave];
    for (uint32_t i = lane; i < nw; i += 64) {
      const uint32_t x = store[wave * kRegion + i];
      const uint32_t pos = store[kCandMax + wave * kRegion + i];
      if (x > prefix) atomicOr(&gtb[pos >> 5], 1u << (pos & 31u));
      else if (x == prefix) atomicOr(&eqb[pos >> 5], 1u << (pos & 31u));
    }
    __syncthreads();
  } else {
    // ---- without the sample: histograms of [31:20], then [19:10], then [9:0]
    for (int64_t w = tid; w < words; w += kLT) gtb[w] = 0u;
    rem = (uint32_t)need;
    prefix = 0u;
    mask = 0u;
    uint32_t cnt = 0u;
    int shift = 20, bits = 12;
    for (;;) {
      const uint32_t nb = 1u << bits;
      for (uint32_t b = tid; b < nb; b += kLT) store[b] = 0u;
      __syncthreads();
      stream_scores(srow, nc, [&](int64_t, float v, bool valid) __attribute__((always_inline)) {
        const uint32_t x = order_key(v);
        wave_count(store, valid && (x & mask) == prefix, (x >> shift) & (nb - 1u), lane);
      });
      __syncthreads();
      find_bin(store, nb, rem, wsum, st);
      __syncthreads();
      const uint32_t bin = st[0];
      prefix |= bin << shift;
      mask |= (nb - 1u) << shift;
      rem -= st[1];
      cnt = store[bin];
      __syncthreads();  // st and store are rewritten below
      if (cnt <= (uint32_t)kCandMax || shift == 0) break;
      shift -= 10;
      bits = 10;
    }
    const bool resolved = shift == 0;  // prefix is tau itself
    if (tid == 0) st[3] = 0u;
    __syncthreads();
    stream_scores(srow, nc, [&](int64_t i, float v, bool valid) __attribute__((always_inline)) {
      const uint32_t x = order_key(v);
      const uint32_t hi = x & mask;
      const uint64_t above = __ballot(valid && hi > prefix);
      const bool in = valid && hi == prefix;
      const uint64_t inb = __ballot(in);
      const int64_t i0 = i - lane;
      if (lane < 2 && i0 + 32 * lane < nc) {
        const int64_t w = i0 / 32 + lane;
        gtb[w] = (uint32_t)(above >> (32 * lane));
        if (resolved) eqb[w] = (uint32_t)(inb >> (32 * lane));
      }
      if (!resolved && inb != 0ull) {
        uint32_t slot0 = 0u;
        if (lane == 0) slot0 = atomicAdd(&st[3], (uint32_t)__popcll(inb));
        slot0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot0);
        if (in) {
          const uint32_t s = slot0 + (uint32_t)__popcll(inb & ((1ull << lane) - 1ull));
          if (s < (uint32_t)kCandMax) {
            store[s] = x;
            store[kCandMax + s] = (uint32_t)i;
          }
        }
      }
    });
    __syncthreads();
    if (!resolved) {
      // the n stored keys as one region per wave of n / kLW (the last takes the rest)
      const uint32_t n = min(st[3], (uint32_t)kCandMax);  // equals cnt
      const uint32_t per = n / kLW;
      __syncthreads();  // st is rewritten by the radix select
      if (tid < kLW) cnt_s[kLW + tid] = tid == kLW - 1 ? n - per * (kLW - 1) : per;
      __syncthreads();
      resolve_regions(store, (int)per, cnt_s + kLW, shift - 8, prefix, mask, rem, h8, st);
      for (uint32_t i = tid; i < n; i += kLT) {
        const uint32_t x = store[i];
        const uint32_t pos = store[kCandMax + i];
        if (x > prefix) atomicOr(&gtb[pos >> 5], 1u << (pos & 31u));
        else if (x == prefix) atomicOr(&eqb[pos >> 5], 1u << (pos & 31u));
      }
      __syncthreads();
    }
  }
  const uint32_t e = rem;

  // ---- ordered sweep over the bitmaps ----------------------------------------
  // Wave w owns a contiguous range of words, taken 64 at a time, one per lane.
  {
    const int64_t wpw = ((words + kLW - 1) / kLW + 63) / 64 * 64;
    const int64_t wb = min((int64_t)wave * wpw, words), we = min(wb + wpw, words);
    uint32_t cg = 0u, ce = 0u;
    for (int64_t w = wb + lane; w < we; w += 64) {
      cg += (uint32_t)__popc(gtb[w]);
      ce += (uint32_t)__popc(eqb[w]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      cg += __shfl_xor(cg, off, 64);
      ce += __shfl_xor(ce, off, 64);
    }
    __syncthreads();  // cnt_s is rewritten
    if (lane == 0) {
      cnt_s[wave] = cg;
      cnt_s[kLW + wave] = ce;
    }
    __syncthreads();
    uint32_t gbase = 0u, ebase = 0u;
    for (int w = 0; w < wave; ++w) {
      gbase += cnt_s[w];
      ebase += cnt_s[kLW + w];
    }
    for (int64_t c0 = wb; c0 < we; c0 += 64) {
      const int64_t w = c0 + lane;
      const uint32_t G = w < we ? gtb[w] : 0u, E = w < we ? eqb[w] : 0u;
      const uint32_t packed = ((uint32_t)__popc(G) << 16) | (uint32_t)__popc(E);  // <= 2048 each per chunk
      uint32_t incl = packed;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint32_t excl = incl - packed;
      uint32_t gt_before = gbase + (excl >> 16);
      uint32_t eq_before = ebase + (excl & 0xFFFFu);
      uint32_t m = G | E;
      if (G == 0xFFFFFFFFu && E == 0u) {  // 32 consecutive kept positions, consecutive ranks
        const uint64_t r0 = (uint64_t)gt_before + min(eq_before, e);
        if (r0 + 32 <= (uint64_t)need) {
          int32_t* o = dst + r0;
          const int32_t p0 = (int32_t)(S + w * 32);
#pragma unroll
          for (int k = 0; k < 32; ++k) o[k] = p0 + k;
        }
        m = 0u;
      }
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1u;
        const int64_t pos = w * 32 + b;
        // ranks are < need by construction; the bound check only keeps a
        // counting error from ever writing outside this list
        if ((G >> b) & 1u) {
          const uint64_t rank = (uint64_t)gt_before + min(eq_before, e);
          if (rank < (uint64_t)need) dst[rank] = (int32_t)(S + pos);
          ++gt_before;
        } else {
          if (eq_before < e) {
            const uint64_t rank = (uint64_t)gt_before + eq_before;
            if (rank < (uint64_t)need) dst[rank] = (int32_t)(S + pos);
          }
          ++eq_before;
        }
      }
      gbase += tot >> 16;
      ebase += tot & 0xFFFFu;
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup radix select.
//
// Used when one (layer, KV head) has more candidates than the LDS key cache
// holds, and for the global eviction over every (layer, KV head) at once (KV²
// summary, "무엇과 다른가": the chunks' local scores gathered into one tensor,
// sinks pinned to the top and the lowest entries evicted down to the budget,
// so that each head ends with its own length, as "전제와 한계" notes).
//
// A segment is the candidate set one threshold is found for: one unit's
// positions [S, N), or (global) every unit's, in (unit, position) order.  Its
// candidates are cut into spans of kSpan, one 256-thread workgroup per (span,
// unit) (small workgroups keep many resident per CU, so one's load latency
// hides behind another's counting):
//   init       per segment: histogram cleared, (prefix, rem) = (0, need)
//   hist, pick four 8-bit digits, most significant first: each span counts
//              the candidates that match the prefix so far into per-wave LDS
//              histograms and adds its nonzero bins to the segment's
//              histogram with integer atomics; one workgroup per segment then
//              takes the digit where the count from the top reaches rem and
//              clears the histogram for the next digit.  Afterwards prefix is
//              tau, the key of the need-th best candidate, and rem is e, the
//              number of candidates equal to tau that are kept.
//   count      per span: candidates above tau and equal to tau
//   scan       per unit (one wave): exclusive prefix counts of its spans; in
//              global mode then one workgroup gives each unit its share of the
//              e tied candidates (lower units first, as the order (score
//              desc, unit, position) says), its kept count and the start of
//              its list
//   emit       per span: keys staged in LDS by coalesced loads, then an
//              ordered block scan over kItems consecutive keys per thread places
//              every kept candidate at its rank in the unit's ascending list
// Only integer atomics are used, so the result does not depend on scheduling.
constexpr int kMT = 256;          // threads per span workgroup
constexpr int kMW = kMT / 64;
constexpr int kSpan = kSelSpan;   // candidates per span workgroup
static_assert(kSpan == kMT * kItems, "one span is kItems candidates per thread");
// Each segment's histogram has one copy per XCD (workgroups are dispatched
// round-robin over the 8 XCDs), so the spans of a large segment do not all
// queue on the same 256 counters; the pick sums the copies.
constexpr int kCopies = 8;

struct MultiArgs {
  const float* scores;
  int32_t* kept;
  int64_t* offsets;   // global mode: [units + 1], start of each unit's list
  uint32_t* hist;     // [segments][kCopies][256]: one copy per XCD
  uint32_t* state;    // [segments][4]: prefix, rem, done, -
  uint32_t* cnt;      // [units][nch][2]: (above tau, equal to tau) of each span
  uint32_t* before;   // [units][nch][2]: the same, summed over the unit's earlier spans
  uint32_t* ekeep;    // global mode: [units], tau-equal candidates each unit keeps
  uint32_t* tot;      // global mode: [units][2], (above tau, equal to tau) of each unit
  int64_t N, S;       // S is min(n_sinks, N)
  int64_t nc;         // N - S candidates per unit
  int64_t need;       // global mode: non-sink entries kept over all units
  int32_t Hkv, units, nch, global;
  LayerTable t;
};

__device__ __forceinline__ int64_t segment_need(const MultiArgs& a, int64_t seg) {
  return a.global ? a.need : (int64_t)a.t.k[seg / a.Hkv] - a.S;
}

// Keys of the kItems candidates a thread owns in an order-free pass over a
// span of len >= 1 candidates at p: candidate j * 4 * kMT + 4 * tid + q is
// item 4j + q (idx), so every load instruction of a wave covers 1 KiB.  VEC:
// p is 16-byte aligned and len a multiple of 4, so each group of four is one
// 16-byte load.  Loads are clamped into the span; items with idx >= len are
// not candidates.
template <bool VEC>
__device__ __forceinline__ void keys_strided(const float* p, int64_t len, int tid,
                                             uint32_t (&x)[kItems], int64_t (&idx)[kItems]) {
#pragma unroll
  for (int j = 0; j < kItems / 4; ++j) {
    const int64_t b = (int64_t)j * 4 * kMT + 4 * tid;
    if (VEC) {
      const float4 v = *reinterpret_cast<const float4*>(p + min(b, len - 4));
      x[4 * j + 0] = order_key(v.x);
      x[4 * j + 1] = order_key(v.y);
      x[4 * j + 2] = order_key(v.z);
      x[4 * j + 3] = order_key(v.w);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) x[4 * j + q] = order_key(p[min(b + q, len - 1)]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) idx[4 * j + q] = b + q;
  }
}

__global__ __launch_bounds__(256) void ms_init(MultiArgs a) {
  const int64_t seg = blockIdx.x;
#pragma unroll
  for (int c = 0; c < kCopies; ++c) a.hist[(seg * kCopies + c) * 256 + threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    const int64_t count = a.global ? a.nc * a.units : a.nc;
    const int64_t need = segment_need(a, seg);
    uint32_t* st = a.state + seg * 4;
    if (need <= 0) {            // only sinks: no candidate reaches tau = ~0 with e = 0
      st[0] = 0xFFFFFFFFu;
      st[1] = 0u;
      st[2] = 1u;
    } else if (need >= count) { // every candidate: all keys are >= tau = 0
      st[0] = 0u;
      st[1] = (uint32_t)count;
      st[2] = 1u;
    } else {
      st[0] = 0u;
      st[1] = (uint32_t)need;
      st[2] = 0u;
    }
    st[3] = 0u;
  }
}

// Each wave counts into kSubHist LDS histograms, lane l into copy l % kSubHist,
// so that lanes whose keys share a bin (after wave_count's peel) queue on
// fewer same-address atomics: 252 -> 237 us per global select of the KV²
// 131K shape's 37.7M scores against one histogram per wave.
constexpr int kSubHist = 4;

template <bool VEC>
__global__ __launch_bounds__(kMT) void ms_hist(MultiArgs a, int shift) {
  __shared__ uint32_t hw[kMW * kSubHist * 256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t u = blockIdx.y;
  const int64_t seg = a.global ? 0 : u;
  const uint32_t* st = a.state + seg * 4;
  if (st[2]) return;  // the same for the whole workgroup
  const uint32_t prefix = st[0];
  const uint32_t mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
  for (int b = tid; b < kMW * kSubHist * 256; b += kMT) hw[b] = 0u;
  const int64_t c0 = (int64_t)blockIdx.x * kSpan;
  const int64_t len = min((int64_t)kSpan, a.nc - c0);
  uint32_t x[kItems];
  int64_t idx[kItems];
  keys_strided<VEC>(a.scores + u * a.N + a.S + c0, len, tid, x, idx);
  __syncthreads();
  uint32_t* mine = hw + (wave * kSubHist + lane % kSubHist) * 256;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    wave_count(mine, idx[j] < len && (x[j] & mask) == prefix, (x[j] >> shift) & 255u, lane);
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t c = 0u;
#pragma unroll
    for (int w = 0; w < kMW * kSubHist; ++w) c += hw[w * 256 + tid];
    const int64_t copy = (blockIdx.x + (int64_t)blockIdx.y * gridDim.x) % kCopies;
    if (c) atomicAdd(&a.hist[(seg * kCopies + copy) * 256 + tid], c);
  }
}

__global__ __launch_bounds__(kThreads) void ms_pick(MultiArgs a, int shift) {
  __shared__ uint32_t wsum[2 * kWaves];
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x;
  uint32_t* st = a.state + seg * 4;
  if (st[2]) return;
  const uint32_t prefix = st[0];
  const uint32_t rem = st[1];
  uint32_t c = 0u;
  if (tid < 256) {  // thread t holds bin 255 - t: the scan runs from the top bin down
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      uint32_t* h = a.hist + (seg * kCopies + k) * 256 + 255 - tid;
      c += *h;
      *h = 0u;      // cleared for the next digit
    }
  }
  uint32_t tot;
  const uint32_t cum = block_scan(c, wsum, &tot);
  if (tid < 256 && cum >= rem && cum - c < rem) {
    st[0] = prefix | ((255u - (uint32_t)tid) << shift);
    st[1] = rem - (cum - c);
    if (shift == 0) st[2] = 1u;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kMT) void ms_count(MultiArgs a) {
  __shared__ uint32_t wsum[2 * kMW];
  const int tid = threadIdx.x;
  const int64_t u = blockIdx.y;
  const uint32_t tau = a.state[(a.global ? 0 : u) * 4];
  const int64_t c0 = (int64_t)blockIdx.x * kSpan;
  const int64_t len = min((int64_t)kSpan, a.nc - c0);
  uint32_t x[kItems];
  int64_t idx[kItems];
  keys_strided<VEC>(a.scores + u * a.N + a.S + c0, len, tid, x, idx);
  uint32_t ngt = 0u, neq = 0u;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    ngt += idx[j] < len && x[j] > tau;
    neq += idx[j] < len && x[j] == tau;
  }
  uint32_t tot;
  block_scan<kMT>((ngt << 16) | neq, wsum, &tot);  // a span's counts fit 16 bits each
  if (tid == 0) {
    uint32_t* c = a.cnt + (u * a.nch + blockIdx.x) * 2;
    c[0] = tot >> 16;
    c[1] = tot & 0xFFFFu;
  }
}

// One wave per unit: exclusive prefix counts of the unit's spans (64 spans
// per step, carried), and in global mode the unit's totals.
__global__ __launch_bounds__(64) void ms_scan_units(MultiArgs a) {
  const int64_t u = blockIdx.x;
  const int lane = threadIdx.x;
  uint32_t cgt = 0u, ceq = 0u;
  for (int64_t c0 = 0; c0 < a.nch; c0 += 64) {
    const int64_t c = c0 + lane;
    const int64_t o = (u * a.nch + c) * 2;
    const uint32_t g = c < a.nch ? a.cnt[o] : 0u;
    const uint32_t e = c < a.nch ? a.cnt[o + 1] : 0u;
    uint32_t ig = g, ie = e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t yg = __shfl_up(ig, off, 64);
      const uint32_t ye = __shfl_up(ie, off, 64);
      if (lane >= off) {
        ig += yg;
        ie += ye;
      }
    }
    if (c < a.nch) {
      a.before[o] = cgt + ig - g;
      a.before[o + 1] = ceq + ie - e;
    }
    cgt += __shfl(ig, 63, 64);
    ceq += __shfl(ie, 63, 64);
  }
  if (a.global && lane == 0) {
    a.tot[u * 2] = cgt;
    a.tot[u * 2 + 1] = ceq;
  }
}

// Global mode: one workgroup walks the unit totals in order, giving each
// unit its share e_u of the tied candidates (lower units first), its kept
// count and the start of its list.
__global__ __launch_bounds__(kThreads) void ms_scan_global(MultiArgs a) {
  __shared__ uint32_t wsum[2 * kWaves];
  const int tid = threadIdx.x;
  const uint32_t e = a.state[1];
  uint64_t carry_eq = 0, carry_k = 0;
  for (int64_t base = 0; base < a.units; base += kThreads) {
    const int64_t u = base + tid;
    const uint32_t gt_u = u < a.units ? a.tot[u * 2] : 0u;
    const uint32_t eq_u = u < a.units ? a.tot[u * 2 + 1] : 0u;
    uint32_t tot_eq;
    const uint32_t inc_eq = block_scan(eq_u, wsum, &tot_eq);
    const uint64_t eq_before = carry_eq + (inc_eq - eq_u);
    const uint32_t e_u = eq_before >= e ? 0u : (uint32_t)min((uint64_t)eq_u, e - eq_before);
    const uint32_t k_u = u < a.units ? (uint32_t)a.S + gt_u + e_u : 0u;
    uint32_t tot_k;
    const uint32_t inc_k = block_scan(k_u, wsum, &tot_k);
    if (u < a.units) {
      a.offsets[u] = (int64_t)(carry_k + (inc_k - k_u));
      a.ekeep[u] = e_u;
    }
    carry_eq += tot_eq;
    carry_k += tot_k;
  }
  if (tid == 0) a.offsets[a.units] = (int64_t)carry_k;
}

template <bool VEC>
__global__ __launch_bounds__(kMT) void ms_emit(MultiArgs a) {
  __shared__ uint32_t wsum[2 * kMW];
  __shared__ uint32_t staged[kSpan];
  const int tid = threadIdx.x;
  const int64_t u = blockIdx.y, c = blockIdx.x;
  const uint32_t tau = a.state[(a.global ? 0 : u) * 4];
  uint32_t e_u;
  int32_t* out;
  int64_t need_u;
  if (a.global) {
    e_u = a.ekeep[u];
    const int64_t o0 = a.offsets[u];
    out = a.kept + o0;
    need_u = a.offsets[u + 1] - o0 - a.S;
  } else {
    e_u = a.state[u * 4 + 1];
    const int64_t l = u / a.Hkv, g = u % a.Hkv, kl = a.t.k[l];
    out = a.kept + a.t.off[l] + g * kl;
    need_u = kl - a.S;
  }
  if (c == 0)
    for (int64_t i = tid; i < a.S; i += kMT) out[i] = (int32_t)i;
  const int64_t c0 = c * kSpan;
  const int64_t len = min((int64_t)kSpan, a.nc - c0);
  if (len <= 0) return;  // no candidate at all (N <= S): only the sinks
  // coalesced loads into LDS, then each thread takes kItems consecutive keys
  {
    uint32_t xs[kItems];
    int64_t idx[kItems];
    keys_strided<VEC>(a.scores + u * a.N + a.S + c0, len, tid, xs, idx);
#pragma unroll
    for (int j = 0; j < kItems; ++j) staged[idx[j]] = xs[j];  // idx < kSpan
  }
  __syncthreads();
  const int64_t i0 = (int64_t)tid * kItems;
  uint32_t x[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) x[j] = staged[i0 + j];
  uint32_t ngt = 0u, neq = 0u;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    ngt += i0 + j < len && x[j] > tau;
    neq += i0 + j < len && x[j] == tau;
  }
  const uint32_t packed = (ngt << 16) | neq;
  uint32_t tot;
  const uint32_t excl = block_scan<kMT>(packed, wsum, &tot) - packed;
  const uint32_t* bf = a.before + (u * a.nch + c) * 2;
  uint64_t gt_before = bf[0] + (excl >> 16);
  uint64_t eq_before = bf[1] + (excl & 0xFFFFu);
  int32_t* dst = out + a.S;
  const int64_t val0 = a.S + c0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t i = i0 + j;
    // ranks are < need_u by construction; the bound check only keeps a
    // counting error from ever writing outside this unit's list
    if (i < len && x[j] > tau) {
      const uint64_t rank = gt_before + (eq_before < e_u ? eq_before : (uint64_t)e_u);
      if (rank < (uint64_t)need_u) dst[rank] = (int32_t)(val0 + i);
      ++gt_before;
    } else if (i < len && x[j] == tau) {
      const uint64_t rank = gt_before + eq_before;
      if (eq_before < e_u && rank < (uint64_t)need_u) dst[rank] = (int32_t)(val0 + i);
      ++eq_before;
    }
  }
}

template <bool VEC>
int multi_select(MultiArgs a, int64_t segments, hipStream_t st) {
  const dim3 spans((unsigned)a.nch, (unsigned)a.units);
  {
    TraceScope ts("select_init", st);
    hipLaunchKernelGGL(ms_init, dim3((unsigned)segments), dim3(256), 0, st, a);
  }
  if (a.nc > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      {
        TraceScope ts("select_hist", st);
        hipLaunchKernelGGL(ms_hist<VEC>, spans, dim3(kMT), 0, st, a, shift);
      }
      TraceScope ts("select_pick", st);
      hipLaunchKernelGGL(ms_pick, dim3((unsigned)segments), dim3(kThreads), 0, st, a, shift);
    }
    TraceScope ts("select_count", st);
    hipLaunchKernelGGL(ms_count<VEC>, spans, dim3(kMT), 0, st, a);
  }
  {
    TraceScope ts("select_scan", st);
    hipLaunchKernelGGL(ms_scan_units, dim3((unsigned)a.units), dim3(64), 0, st, a);
    if (a.global) hipLaunchKernelGGL(ms_scan_global, dim3(1), dim3(kThreads), 0, st, a);
  }
  TraceScope ts("select_emit", st);
  hipLaunchKernelGGL(ms_emit<VEC>, dim3((unsigned)std::max<int64_t>(a.nch, 1), (unsigned)a.units),
                     dim3(kMT), 0, st, a);
  return (int)hipGetLastError();
}

// Carves the select workspace (layout of select_workspace_bytes) and runs the
// multi-workgroup select in per-unit or global mode.
int run_multi(const kvs_problem& p, const float* scores, const LayerTable* t, int64_t need,
              int32_t* kept, int64_t* offsets, void* ws, hipStream_t st) {
  const int64_t N = p.n_cache, S = std::min(p.n_sinks, p.n_cache);
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  MultiArgs a;
  a.scores = scores;
  a.kept = kept;
  a.offsets = offsets;
  a.N = N;
  a.S = S;
  a.nc = N - S;
  a.need = need;
  a.Hkv = p.kv_heads;
  a.units = (int32_t)units;
  a.nch = (int32_t)ceil_div(a.nc, kSpan);
  a.global = t ? 0 : 1;
  if (t) a.t = *t;
  const SelectWs w = select_ws_layout(p);
  uint8_t* base = static_cast<uint8_t*>(ws);
  a.hist = reinterpret_cast<uint32_t*>(base + w.off_hist);
  a.state = reinterpret_cast<uint32_t*>(base + w.off_state);
  a.cnt = reinterpret_cast<uint32_t*>(base + w.off_cnt);
  a.before = reinterpret_cast<uint32_t*>(base + w.off_before);
  a.ekeep = reinterpret_cast<uint32_t*>(base + w.off_ekeep);
  a.tot = reinterpret_cast<uint32_t*>(base + w.off_tot);
  const int64_t segments = t ? units : 1;
  const bool vec = (N % 4 == 0) && (S % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  return vec ? multi_select<true>(a, segments, st) : multi_select<false>(a, segments, st);
}

}  // namespace

int launch_select(const kvs_problem& p, const float* scores, const LayerTable& t,
                  int32_t* kept, void* ws, void* stream) {
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  if (units <= 0 || p.n_cache <= 0) return 0;
  const int64_t nc = p.n_cache - std::min(p.n_sinks, p.n_cache);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (select_uses_multi(p)) return run_multi(p, scores, &t, 0, kept, nullptr, ws, st);
  SelArgs a;
  a.scores = scores;
  a.kept = kept;
  a.N = p.n_cache;
  a.S = p.n_sinks;
  a.Hkv = p.kv_heads;
  a.t = t;
  TraceScope ts("select", st);
  if (nc > kSelLongMin)
    hipLaunchKernelGGL(select_long_kernel, dim3((unsigned)units), dim3(kLT), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel<true>, dim3((unsigned)units), dim3(kThreads), 0, st, a);
  return (int)hipGetLastError();
}

int launch_select_global(const kvs_problem& p, const float* scores, int64_t total,
                         int32_t* kept, int64_t* offsets, void* ws, void* stream) {
  const int64_t units = (int64_t)p.layers * p.kv_heads;
  const int64_t S = std::min(p.n_sinks, p.n_cache);
  return run_multi(p, scores, nullptr, total - units * S, kept, offsets, ws,
                   static_cast<hipStream_t>(stream));
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
