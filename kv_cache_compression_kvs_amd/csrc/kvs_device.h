// Device-side helpers for the gfx950 kernels: vector types, the bf16 MFMA
// wrapper, exp2, cross-lane moves and the XCD-aware block remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// D = A * B + C on a 32x32 output tile with a 16-deep bf16 contraction.
// Register layout (per lane l of the wave64):
//   A: row l % 32 of the 32x16 operand, 8 consecutive k starting at (l / 32) * 8
//   B: column l % 32 of the 16x32 operand, the same 8 k
//   C/D: column l % 32, rows (i / 4) * 8 + (l / 32) * 4 + (i % 4) for i = 0..15
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within the 32-row tile) held in accumulator slot i by lane l.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

// Value of `x` held by lane (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Remapping b so that consecutive logical tiles land on the same XCD
// keeps tiles that share operands inside one L2.  The grid is padded to a
// multiple of 8; a logical index >= n_logical means "no work".
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t grid) {
  const int64_t per = grid >> 3;  // grid is a multiple of 8
  return (b & 7) * per + (b >> 3);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Third dword of a raw (offset-mode) buffer resource on gfx9-family parts:
// 32-bit data format, no swizzle.  Loads at or past num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// Generic LDS pointer as the address-space-3 pointer the LDS DMA builtin takes.
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)(p);
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 family
// encoding: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace kvs
