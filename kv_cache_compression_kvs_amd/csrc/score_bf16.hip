// Attention scoring of appended queries over a bf16 cache, on bf16 MFMA.
//
// What is computed (KV² summary, "무엇과 다른가"): for every query row j of a
// query head h and every cached key i, z_ji = q_j . k_i / sqrt(d); the
// probability p_ji = exp(z_ji) / sum_i' exp(z_ji') is normalised over the whole
// cache; a position i of chunk C_r scores max over the heads sharing its KV
// head and over C_r's rows of p_ji.  Sinks score 1.
//
// Two passes, everything in base-2 units (c1 = log2(e) / sqrt(d)):
//   pass 1  c2_j = log2 sum_i 2^(z_ji c1): a running max and sum per row over
//           all N keys (optionally split along the keys and merged after).
//           The score matrix is formed transposed, keys x queries, so each
//           lane owns one query and its keys sit in its own registers: the row
//           reduction needs no cross-lane traffic inside the key loop.
//   pass 2  score_i = 2^(max_j (z_ji c1 - c2_j)), the max taken over the rows
//           of the chunk that owns i.  Formed queries x keys so each lane owns
//           one key; -c2_j / c1 is preloaded into the accumulator, so the hot
//           loop is MFMA plus one running max per element, and a single exp2
//           per position at the end (max of exp = exp of max).
//
// Pass 1 workgroup: W waves x 64 query rows (two 32-column MFMA blocks per
// wave, Q fragments resident in VGPRs); keys stream through a ring of LDS
// tiles filled by direct global->LDS loads.  Pass 2 workgroup: 64 keys per
// wave resident in VGPRs; the chunk's query rows (all heads of the group)
// stream through a ring of LDS tiles together with their -c2/c1 values.
#include <float.h>
#include <math.h>

#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_trace.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;

struct P1Args {
  const uint16_t* q;
  const uint8_t* kh;  // key rows [0, split) of each slab, slab stride kh_stride rows
  const uint8_t* kt;  // key rows [split, N): row kt_row0 + (i - split), slab stride kt_stride
  float* c2n;       // [total_rows] -c2 / c1, written when splits == 1
  float* part_m;    // [splits][total_rows]
  float* part_l;    // [splits][total_rows]
  int64_t Nq, N, rows_per_unit, row_blocks, splits, keys_per_split, total_rows;
  int64_t kh_stride, kt_stride, kt_row0, split;
  int64_t n_logical;
  int32_t Hq, Hkv, G;
  float c1, inv_c1;
};

// Two waves per SIMD whatever W is (8 / W workgroups per CU): about 200
// VGPRs per wave.
template <int D, int TK, int NBUF, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void pass1_bf16(P1Args a) {
  constexpr int NT = W * 64;                       // threads per workgroup
  constexpr int KS = D / 16;                       // MFMA steps along d
  constexpr int ROWB = D * 2;                      // bytes per key row
  constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row
  constexpr int NB = TK / 32;                      // 32-key blocks per tile
  constexpr int TILEB = TK * ROWB;                 // bytes per key tile
  constexpr int LPT = TILEB / (NT * 16);           // DMA instructions per wave per tile
  static_assert(NBUF >= 2 && NBUF <= 4 && TK % 32 == 0 && LPT >= 1, "ring shape");
  // NBUF key tiles in flight through a ring of LDS buffers filled by direct
  // global->LDS loads.  Separate arrays (indexed statically below) let the
  // compiler see that a DMA into one buffer never aliases reads of another.
  __shared__ __attribute__((aligned(16))) uint8_t r0[TILEB], r1[TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t r2[NBUF > 2 ? TILEB : 16], r3[NBUF > 3 ? TILEB : 16];
  auto ring = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return i == 0 ? r0 : i == 1 ? r1 : i == 2 ? r2 : r3;
  };

  const int64_t tau = xcd_remap(blockIdx.x, gridDim.x);
  if (tau >= a.n_logical) return;
  const int64_t rb = tau % a.row_blocks;
  const int64_t t2 = tau / a.row_blocks;
  const int64_t split = t2 % a.splits;
  const int64_t unit = t2 / a.splits;
  const int64_t l = unit / a.Hkv, g = unit % a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps DMA operands scalar
  const int col = lane & 31, half = lane >> 5;

  const int64_t unit_row0 = (l * a.Hq + g * a.G) * a.Nq;
  const uint16_t* qunit = a.q + unit_row0 * D;
  const int64_t slab = l * a.Hkv + g;
  const uint8_t* khead = a.kh + slab * a.kh_stride * ROWB;
  const uint8_t* ktail = a.kt + (slab * a.kt_stride + a.kt_row0) * ROWB;
  const int64_t row_w = rb * NT + wave * 64;

  bf16x8 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int64_t r = row_w + qb * 32 + col;
    if (r > a.rows_per_unit - 1) r = a.rows_per_unit - 1;
    const uint16_t* src = qunit + r * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *(const bf16x8*)(src + ks * 16);
  }

  const int64_t kbeg = split * a.keys_per_split;
  const int64_t kend = min(kbeg + a.keys_per_split, a.N);
  const int64_t nkeys = kend - kbeg;
  const int64_t nfull = nkeys / TK;
  const int64_t ntiles = ceil_div(nkeys, TK);
  const int64_t ngroups = nfull / NBUF;

  // Running max (base-2 units) and sum of 2^(z c1 - m) per query block.  The
  // start value is finite so that the pipeline's empty first stage (all -inf)
  // adds exactly zero; the first real block moves m off it.
  float m[2] = {-FLT_MAX, -FLT_MAX};
  float ls[2] = {0.f, 0.f};
  const float c1 = a.c1;

  // Tile layout in LDS: row r (a key), 16-byte chunk c at r*ROWB + ((c ^ (r % CPR)) * 16).
  // The XOR swizzle makes the fragment reads (32 rows, same chunk) hit
  // distinct banks.  Wave w's i-th DMA fills LDS chunks [(Wi+w)*64, +64),
  // that is RPI whole rows starting at row (Wi+w)*RPI, lane by lane, so each
  // lane fetches the global chunk that lands there.  The lane's part of the
  // byte offset (its row within those RPI rows and its swizzled chunk) is the
  // same for every i, because W*RPI is a multiple of CPR (asserted below), so
  // the rows (Wi+w)*RPI of one wave share their residue mod CPR; the
  // instruction's first row rides in the scalar offset.  That row also picks
  // the buffer (head or tail segment: every segment boundary is a multiple of
  // RPI), and each buffer resource covers exactly its segment's rows, so rows
  // past the end read as zero instead of leaving the slab.
  constexpr int RPI = 64 / CPR;
  static_assert((W * RPI) % CPR == 0, "one swizzle residue per wave across its DMAs");
  const __amdgpu_buffer_rsrc_t rs_head = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(khead), (short)0, (int)(uint32_t)(a.split * ROWB), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_tail = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(ktail), (short)0, (int)(uint32_t)((a.N - a.split) * ROWB), kBufferFlags);
  const int lrow = (wave * 64 + lane) / CPR;
  const uint32_t voff = (uint32_t)((lane / CPR) * ROWB + (((wave * 64 + lane) % CPR) ^ (lrow & (CPR - 1))) * 16);
  auto dma = [&](uint8_t* buf, int64_t tile) __attribute__((always_inline)) {
    const int64_t row0 = kbeg + tile * TK;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int64_t rf = row0 + (i * W + wave) * RPI;
      auto* dst = lds_ptr(buf + (i * W + wave) * 1024);
      if (rf < a.split)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_head, dst, 16, (int)voff, (int)(uint32_t)(rf * ROWB), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_tail, dst, 16, (int)voff,
                                                 (int)(uint32_t)((rf - a.split) * ROWB), 0, 0);
    }
  };
  // Fragment (kb, ks) of a tile: row kb*32 + col, chunk 2ks + half.  As
  // 32 % CPR == 0 the row's swizzle is col % CPR, and the chunk's byte offset
  // (2ks ^ half ^ (col % CPR)) * 16 splits into (16 (half ^ (col % CPR))) ^ 32ks
  // below ROWB: one per-lane base XORed with a constant per ks, so the
  // fragment addresses take no registers of their own.
  static_assert(32 % CPR == 0, "a 32-row block starts on a swizzle period");
  const uint32_t fbase = (uint32_t)(col * ROWB + ((half ^ (col & (CPR - 1))) * 16));
  auto afrag = [&](const uint8_t* buf, int kb, int ks) __attribute__((always_inline)) -> bf16x8 {
    return *(const bf16x8*)(buf + kb * 32 * ROWB + (fbase ^ (uint32_t)(32 * ks)));
  };

  // Exact update by one block: move m to the block's max if larger, rescale
  // the sum, add the block's terms.
  auto update = [&](int qb, const f32x16& z) __attribute__((always_inline)) {
    float mx = max3f(max3f(z[0], z[1], z[2]), max3f(z[3], z[4], z[5]), max3f(z[6], z[7], z[8]));
    mx = max3f(mx, max3f(z[9], z[10], z[11]), max3f(z[12], z[13], z[14]));
    mx = fmaxf(mx, z[15]);
    const float mn = fmaxf(m[qb], mx * c1);
    float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 16; ++e) t4[e & 3] += exp2_hw(fmaf(z[e], c1, -mn));
    ls[qb] = ls[qb] * exp2_hw(m[qb] - mn) + ((t4[0] + t4[1]) + (t4[2] + t4[3]));
    m[qb] = mn;
  };

  // Software pipeline over 32-key blocks: the MFMAs of block j and the
  // softmax update of block j-1 sit in one basic block; after each MFMA one
  // slice of the update follows and a scheduling fence keeps that order, so
  // the vector ALU works while the MFMA occupies the matrix pipe.
  //
  // The update in the pipeline takes a block's terms against the current m
  // without first reducing the block's max: one fma, one exp2 and one add per
  // element.  A block sum below 2^16 proves that no term overflowed, and
  // terms up to that size lose nothing in fp32; a block that fails the test
  // (its max lies more than 16 above m, or it is the first block) takes a
  // wave-uniform branch that redoes it exactly against its max.
  // c2 = m + log2(l) is exact for any m, so this changes nothing but rounding.
  constexpr float kSumLimit = 65536.f;
  f32x16 p0, p1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p0[i] = -INFINITY;
    p1[i] = -INFINITY;
  }
  auto compute_tile = [&](const uint8_t* buf) __attribute__((always_inline)) {
    constexpr int NS = 2 * KS;      // MFMAs (and update slices) per block
    static_assert(NS >= 4, "at least two slices take the previous block's terms");
    bf16x8 af[2][KS];               // fragments of the current and the next key block
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[0][ks] = afrag(buf, 0, ks);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const int cur = kb & 1;
      f32x16 n0 = {}, n1 = {};
      float t0 = 0.f, t1 = 0.f;
      const float m0 = m[0], m1 = m[1];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if ((i & 1) == 0) {
          n0 = mfma32x32x16(af[cur][i >> 1], qf[0][i >> 1], n0);
        } else {
          n1 = mfma32x32x16(af[cur][i >> 1], qf[1][i >> 1], n1);
          // fragment ks of this block is dead after its second MFMA: fetch the
          // next block's fragment ks now, so that block starts without an LDS wait
          if (kb + 1 < NB) af[cur ^ 1][i >> 1] = afrag(buf, kb + 1, i >> 1);
        }
        // The previous block's 32 terms go to slices 2 .. NS-1 (p0's first):
        // its last MFMAs (slices NS-2, NS-1) may still be writing them during
        // slices 0 and 1, and a read there would wait for them.
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          if (2 + (e * (NS - 2)) / 32 == i) {
            if (e < 16) t0 += exp2_hw(fmaf(p0[e], c1, -m0));
            else t1 += exp2_hw(fmaf(p1[e - 16], c1, -m1));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (__any(!(t0 < kSumLimit) || !(t1 < kSumLimit))) {
        update(0, p0);
        update(1, p1);
      } else {
        ls[0] += t0;
        ls[1] += t1;
      }
      p0 = n0;
      p1 = n1;
    }
  };
  // Tile u lives in buffer u % NBUF.  Before computing it: wait until at
  // most the younger tiles' DMAs are outstanding, meet at the barrier (every
  // wave's share of tile u has landed and every wave is done with tile u-1),
  // then start the DMA of tile u + NBUF - 1 into tile u-1's buffer.
  auto step = [&](int b, int64_t u) __attribute__((always_inline)) {
    wait_vmcnt<(NBUF - 2) * LPT>();
    __builtin_amdgcn_s_barrier();
    dma(ring((b + NBUF - 1) % NBUF), u + NBUF - 1);
    compute_tile(ring(b));
  };

#pragma unroll
  for (int b = 0; b + 1 < NBUF; ++b) dma(ring(b), b);
  for (int64_t gi = 0; gi < ngroups; ++gi) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) step(b, gi * NBUF + b);
  }
  update(0, p0);
  update(1, p1);

  // Remaining tiles (fewer than NBUF full tiles and a ragged tail), one at a
  // time with masking.  Tiles below `issued` already have their DMA in flight.
  int64_t issued = ngroups * NBUF + NBUF - 1;
  for (int64_t u = ngroups * NBUF; u < ntiles; ++u) {
    uint8_t* buf = ring((int)(u % NBUF));
    if (u >= issued) {
      __builtin_amdgcn_s_barrier();  // every wave is done with the buffer's previous tile
      dma(buf, u);
      ++issued;
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const int valid = (int)min(nkeys - u * TK, (int64_t)TK);  // keys of this tile
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      if (kb * 32 < valid) {
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 av = afrag(buf, kb, ks);
          acc0 = mfma32x32x16(av, qf[0][ks], acc0);
          acc1 = mfma32x32x16(av, qf[1][ks], acc1);
        }
        if (valid < TK) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (kb * 32 + acc_row(i, lane) >= valid) {
              acc0[i] = -INFINITY;
              acc1[i] = -INFINITY;
            }
          }
        }
        update(0, acc0);
        update(1, acc1);
      }
    }
  }
  wait_vmcnt<0>();  // no DMA may still target LDS when the workgroup exits

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = ls[qb];
    const float mo = swap_halves(m[qb]);
    const float lo = swap_halves(lsum);
    const float M = fmaxf(m[qb], mo);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float L = lsum * exp2_hw(m[qb] - Ms) + lo * exp2_hw(mo - Ms);
    const int64_t r = row_w + qb * 32 + col;
    if (half == 0 && r < a.rows_per_unit) {
      const int64_t grow = unit_row0 + r;
      if (a.splits == 1) {
        a.c2n[grow] = -(M + log2f(L)) * a.inv_c1;
      } else {
        a.part_m[split * a.total_rows + grow] = M;
        a.part_l[split * a.total_rows + grow] = L;
      }
    }
  }
}

// Fixed-order log-sum-exp merge of the per-split partials of pass 1; writes
// -c2 / c1 per row, the accumulator start value pass 2 takes.
__global__ __launch_bounds__(kThreads) void merge_splits(const float* pm, const float* pl,
                                                        float* c2n, int64_t total_rows,
                                                        int64_t splits, float inv_c1) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total_rows) return;
  float M = -INFINITY;
  for (int64_t s = 0; s < splits; ++s) M = fmaxf(M, pm[s * total_rows + i]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  for (int64_t s = 0; s < splits; ++s) L += pl[s * total_rows + i] * exp2_hw(pm[s * total_rows + i] - Ms);
  c2n[i] = -(M + log2f(L)) * inv_c1;
}

struct P2Args {
  const uint16_t* q;
  const uint16_t* kh;  // as in P1Args
  const uint16_t* kt;
  const float* c2n;     // [total_rows] -c2 / c1 per query row
  float* scores;
  int64_t Nq, N, S, m, nq, R, tiles, n_logical;
  int64_t kh_stride, kt_stride, kt_row0, split;
  int32_t Hq, Hkv, G;
  uint32_t nq_mul, nq_shift;  // rho / nq as (umulhi(rho, nq_mul) + rho) >> nq_shift
  float c1;
};

// Pass-2 workgroup: W waves x 64 keys, the keys' fragments resident in VGPRs.
// The chunk's query rows (all heads of the group, gathered) stream through a
// ring of NBUF LDS tiles of 64 rows filled by direct global->LDS loads, each
// tile with its rows' -c2/c1 (one private copy per wave).  A tile is two
// stages of 32 rows; a stage is 16 MFMAs whose accumulators start at the
// rows' -c2/c1, and the running max over the previous stage's accumulators
// is interleaved with them.  Rows past the chunk's last one repeat it, which
// leaves every max unchanged, so the row loop needs no masking or tail.
template <int D, int W, int NBUF>
__global__ __launch_bounds__(W * 64, 8 / W) void pass2_bf16(P2Args a) {
  constexpr int KS = D / 16;
  constexpr int ROWB = D * 2;                 // bytes per query row
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int ROWS = 64;                    // query rows per tile
  constexpr int TILEB = ROWS * ROWB;
  constexpr int LPT = TILEB / (W * 64 * 16);  // Q DMA instructions per wave per tile
  constexpr int CB = W * ROWS * 4;            // -c2/c1 copies, one per wave
  static_assert(NBUF >= 3 && NBUF <= 4 && LPT >= 1, "ring shape");
  __shared__ __attribute__((aligned(16))) uint8_t q0[TILEB], q1[TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t q2[NBUF > 2 ? TILEB : 16], q3[NBUF > 3 ? TILEB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t cs0[CB], cs1[CB];
  __shared__ __attribute__((aligned(16))) uint8_t cs2[NBUF > 2 ? CB : 16], cs3[NBUF > 3 ? CB : 16];
  auto qring = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return i == 0 ? q0 : i == 1 ? q1 : i == 2 ? q2 : q3;
  };
  auto cring = [&](int i) __attribute__((always_inline)) -> uint8_t* {
    return i == 0 ? cs0 : i == 1 ? cs1 : i == 2 ? cs2 : cs3;
  };

  const int64_t tau = xcd_remap(blockIdx.x, gridDim.x);
  if (tau >= a.n_logical) return;
  const int64_t tile = tau % a.tiles;
  const int64_t t2 = tau / a.tiles;
  const int64_t r = t2 % a.R;
  // Units in reverse order: pass 1 streams the keys unit by unit in forward
  // order just before, so the last units' keys are the ones still in the
  // memory-side cache when this pass starts.
  const int64_t unit = a.n_logical / (a.R * a.tiles) - 1 - t2 / a.R;
  const int64_t l = unit / a.Hkv, g = unit % a.Hkv;
  const int64_t cb0 = a.S + r * a.m;
  const int64_t cb1 = min(cb0 + a.m, a.N);
  const int64_t kt0 = cb0 + tile * (W * 64);
  if (kt0 >= cb1) return;  // uniform over the workgroup, before any barrier

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int64_t kw = kt0 + wave * 64;
  const uint16_t* khead = a.kh + unit * a.kh_stride * D;
  const uint16_t* ktail = a.kt + (unit * a.kt_stride + a.kt_row0) * D;
  float* srow = a.scores + unit * a.N;

  if (r == 0 && tile == 0) {
    const int64_t ns = min(a.S, a.N);
    for (int64_t i = tid; i < ns; i += W * 64) srow[i] = 1.0f;
  }

  bf16x8 kf[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int64_t key = kw + kb * 32 + col;
    if (key > a.N - 1) key = a.N - 1;
    const uint16_t* src = (key < a.split ? khead + key * D : ktail + (key - a.split) * D) + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = *(const bf16x8*)(src + ks * 16);
  }

  const int64_t unit_row0 = (l * a.Hq + g * a.G) * a.Nq;
  const int64_t rows_per_unit = (int64_t)a.G * a.Nq;
  const uint32_t nrows = (uint32_t)(a.G * a.nq);
  const int64_t ntiles = ceil_div(nrows, ROWS);
  const int64_t ngroups = ceil_div(ntiles, NBUF);

  // Buffer resources over the unit's query rows and their -c2/c1 values.
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.q + unit_row0 * D), (short)0, (int)(uint32_t)(rows_per_unit * ROWB),
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.c2n + unit_row0), (short)0, (int)(uint32_t)(rows_per_unit * 4),
      kBufferFlags);
  // Unit row of chunk row rho (clamped to the chunk's last row): head rho / nq
  // of the group, query rho % nq of chunk r.
  const uint32_t nq32 = (uint32_t)a.nq;
  const uint32_t rbase = (uint32_t)(r * a.nq);
  auto urow = [&](uint32_t rho) __attribute__((always_inline)) -> uint32_t {
    rho = min(rho, nrows - 1);
    const uint32_t t = (__umulhi(rho, a.nq_mul) + rho) >> a.nq_shift;
    return t * (uint32_t)a.Nq + rbase + (rho - t * nq32);
  };
  // Tile layout in LDS as in pass 1: row rr, 16-byte chunk c at
  // rr*ROWB + ((c ^ (rr % CPR)) * 16).  Wave w's i-th DMA fills LDS chunks
  // [(i*W + w)*64, +64) lane by lane; each lane fetches the chunk landing there.
  auto dma = [&](uint8_t* qb, uint8_t* cb, int64_t tl) __attribute__((always_inline)) {
    const uint32_t row0 = (uint32_t)(tl * ROWS);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int L = (i * W + wave) * 64 + lane;
      const int rr = L / CPR;
      const int cc = (L % CPR) ^ (rr & (CPR - 1));
      const uint32_t off = urow(row0 + rr) * ROWB + cc * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, lds_ptr(qb + (i * W + wave) * 1024), 16, (int)off,
                                               0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, lds_ptr(cb + wave * ROWS * 4), 4,
                                             (int)(urow(row0 + lane) * 4), 0, 0, 0);
  };
  auto afrag = [&](const uint8_t* qb, int rb, int ks) __attribute__((always_inline)) -> bf16x8 {
    const int row = rb * 32 + col;
    const int c = 2 * ks + half;
    return *(const bf16x8*)(qb + row * ROWB + ((c ^ (row & (CPR - 1))) * 16));
  };
  // -c2/c1 of the accumulator rows of stage rb: rows rb*32 + (i/4)*8 + half*4 + i%4.
  auto cinit = [&](const uint8_t* cb, int rb) __attribute__((always_inline)) -> f32x16 {
    const float* cw = reinterpret_cast<const float*>(cb + wave * ROWS * 4) + rb * 32 + half * 4;
    f32x16 v;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = *(const float4*)(cw + q4 * 8);
      v[q4 * 4 + 0] = x.x;
      v[q4 * 4 + 1] = x.y;
      v[q4 * 4 + 2] = x.z;
      v[q4 * 4 + 3] = x.w;
    }
    return v;
  };

  float cm[2] = {-INFINITY, -INFINITY};
  f32x16 p0, p1;  // accumulators of the previous stage
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p0[i] = -INFINITY;
    p1[i] = -INFINITY;
  }
  // One stage: 16 MFMAs on the fragments `av` with accumulators starting at
  // `ci`, the running max over the previous stage interleaved, and the next
  // stage's fragments fetched (`next(ks)` after fragment ks is dead, `cnext`
  // after the first MFMA) so that stage starts without an LDS wait.
  auto stage = [&](const bf16x8 (&av)[KS], const f32x16& ci, auto&& next, auto&& cnext)
      __attribute__((always_inline)) {
    f32x16 x0 = ci, x1 = ci;
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      const int ks = i >> 1;
      if ((i & 1) == 0) {
        x0 = mfma32x32x16(av[ks], kf[0][ks], x0);
      } else {
        x1 = mfma32x32x16(av[ks], kf[1][ks], x1);
        next(ks);
      }
      if (i == 0) cnext();
      constexpr int PER = 32 / (2 * KS);
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const int j = i * PER + e;
        if (j < 16) cm[0] = max3f(cm[0], p0[j], p0[j + 1]);
        else cm[1] = max3f(cm[1], p1[j - 16], p1[j - 15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    p0 = x0;
    p1 = x1;
  };

  // Tile u lives in ring slot u % NBUF and is two stages (rows 0-31, 32-63).
  // The barrier sits between the stages of tile u: after it every wave's
  // loads of tile u+1 have landed (they were issued a tile earlier) and every
  // wave is done with tile u-1, whose slot then takes the loads of tile
  // u + NBUF - 1.  Stage 1 of tile u fetches stage 0 of tile u+1.  Rows past
  // the last tile repeat the chunk's last row, so the tile count is padded to
  // a multiple of NBUF.
  bf16x8 avA[KS], avB[KS];
  f32x16 ciA, ciB;
#pragma unroll
  for (int b = 0; b + 1 < NBUF; ++b) dma(qring(b), cring(b), b);
  wait_vmcnt<(NBUF - 2) * (LPT + 1)>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) avA[ks] = afrag(q0, 0, ks);
  ciA = cinit(cs0, 0);
  for (int64_t gi = 0; gi < ngroups; ++gi) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const uint8_t* qb = qring(b);
      const uint8_t* cb = cring(b);
      const uint8_t* qn = qring((b + 1) % NBUF);
      const uint8_t* cn = cring((b + 1) % NBUF);
      stage(avA, ciA, [&](int ks) __attribute__((always_inline)) { avB[ks] = afrag(qb, 1, ks); },
            [&]() __attribute__((always_inline)) { ciB = cinit(cb, 1); });
      wait_vmcnt<(NBUF - 3) * (LPT + 1)>();
      __builtin_amdgcn_s_barrier();
      dma(qring((b + NBUF - 1) % NBUF), cring((b + NBUF - 1) % NBUF), gi * NBUF + b + NBUF - 1);
      stage(avB, ciB, [&](int ks) __attribute__((always_inline)) { avA[ks] = afrag(qn, 0, ks); },
            [&]() __attribute__((always_inline)) { ciA = cinit(cn, 0); });
    }
  }
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    cm[0] = max3f(cm[0], p0[j], p0[j + 1]);
    cm[1] = max3f(cm[1], p1[j], p1[j + 1]);
  }
  wait_vmcnt<0>();  // no DMA may still target LDS when the workgroup exits

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const float v = fmaxf(cm[kb], swap_halves(cm[kb]));
    const int64_t key = kw + kb * 32 + col;
    if (half == 0 && key < cb1) srow[key] = fminf(exp2_hw(v * a.c1), 1.0f);
  }
}

// Exact unsigned division by a runtime divisor through a multiply-high:
// n / d == (umulhi(n, mul) + n) >> shift for every n < 2^31.
inline void fast_div(uint32_t d, uint32_t* mul, uint32_t* shift) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  *shift = s;
  *mul = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
}

inline int64_t pad8(int64_t n) { return (n + 7) & ~int64_t(7); }

template <int D>
int run(const kvs_problem& p, const ScorePlan& pl, const void* q, const KvSrc& kv, float* scores,
        void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  float* c2 = reinterpret_cast<float*>(w + pl.off_c2);
  float* pm = reinterpret_cast<float*>(w + pl.off_pm);
  float* plw = reinterpret_cast<float*>(w + pl.off_pl);
  const int64_t N = p.n_cache;
  const float c1 = (float)(1.4426950408889634 / sqrt((double)D));
  const float inv_c1 = (float)(sqrt((double)D) / 1.4426950408889634);

  P1Args a1;
  a1.q = static_cast<const uint16_t*>(q);
  a1.kh = static_cast<const uint8_t*>(kv.k_head);
  a1.kt = static_cast<const uint8_t*>(kv.k_tail);
  a1.kh_stride = kv.head_stride;
  a1.kt_stride = kv.tail_stride;
  a1.kt_row0 = kv.tail_row0;
  a1.split = kv.split;
  a1.c2n = c2;
  a1.part_m = pm;
  a1.part_l = plw;
  a1.Nq = pl.n_queries;
  a1.N = N;
  a1.rows_per_unit = pl.rows_per_unit;
  a1.row_blocks = pl.row_blocks;
  a1.splits = pl.splits;
  a1.keys_per_split = pl.keys_per_split;
  a1.total_rows = pl.total_rows;
  a1.n_logical = pl.units * pl.splits * pl.row_blocks;
  a1.Hq = p.q_heads;
  a1.Hkv = p.kv_heads;
  a1.G = p.q_heads / p.kv_heads;
  a1.c1 = c1;
  a1.inv_c1 = inv_c1;
  {
    TraceScope ts("score_pass1_bf16", st);
    static_assert(kP1Waves * 64 == kP1Rows, "planner and kernel agree on the rows per workgroup");
    hipLaunchKernelGGL((pass1_bf16<D, kP1Keys, kP1Ring, kP1Waves>), dim3((unsigned)pad8(a1.n_logical)),
                       dim3(kP1Waves * 64), 0, st, a1);
  }
  if (hipError_t e = hipGetLastError()) return (int)e;
  if (pl.splits > 1) {
    TraceScope ts("score_merge_splits", st);
    hipLaunchKernelGGL(merge_splits, dim3((unsigned)ceil_div(pl.total_rows, kThreads)),
                       dim3(kThreads), 0, st, pm, plw, c2, pl.total_rows, pl.splits, inv_c1);
    if (hipError_t e = hipGetLastError()) return (int)e;
  }

  P2Args a2;
  a2.q = a1.q;
  a2.kh = static_cast<const uint16_t*>(kv.k_head);
  a2.kt = static_cast<const uint16_t*>(kv.k_tail);
  a2.kh_stride = kv.head_stride;
  a2.kt_stride = kv.tail_stride;
  a2.kt_row0 = kv.tail_row0;
  a2.split = kv.split;
  a2.c2n = c2;
  a2.scores = scores;
  a2.Nq = pl.n_queries;
  a2.N = N;
  a2.S = p.n_sinks;
  a2.m = p.chunk_size;
  a2.nq = p.q_per_chunk;
  a2.R = pl.n_chunks;
  a2.tiles = pl.p2_tiles;
  a2.n_logical = pl.units * pl.n_chunks * pl.p2_tiles;
  a2.Hq = p.q_heads;
  a2.Hkv = p.kv_heads;
  a2.G = a1.G;
  a2.c1 = c1;
  fast_div((uint32_t)p.q_per_chunk, &a2.nq_mul, &a2.nq_shift);
  {
    TraceScope ts("score_pass2_bf16", st);
    hipLaunchKernelGGL((pass2_bf16<D, kP2Waves, kP2Ring>), dim3((unsigned)pad8(a2.n_logical)),
                       dim3(kP2Waves * 64), 0, st, a2);
  }
  if (hipError_t e = hipGetLastError()) return (int)e;
  return 0;
}

}  // namespace

int launch_score_bf16(const kvs_problem& p, const ScorePlan& pl, const void* q, const KvSrc& kv,
                      float* scores, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p.head_dim == 128) return run<128>(p, pl, q, kv, scores, ws, st);
  return run<64>(p, pl, q, kv, scores, ws, st);
}

}  // namespace kvs
