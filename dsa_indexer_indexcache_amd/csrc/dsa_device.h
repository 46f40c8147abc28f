// Device-side helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/dsa.h"

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The lane id recomputed where it is used (volatile asm is not hoisted out of loops): for
// loop-invariant per-lane values that would otherwise stay live across a loop and be
// spilled under register pressure; two VALU ops instead of a scratch reload.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ReLU of a finite float as a signed-integer max of its bit pattern: negative
// values (sign bit set) and -0.0 become +0.0.  One v_max_i32, where fmaxf would
// first canonicalise its input under IEEE mode.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Total order on fp32 scores as unsigned keys; -0.0 is first mapped to +0.0 so
// the two zeros tie (the selection then falls back to position order).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const i32x4& a, const i32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// fp8 e4m3 x fp8 e4m3, K = 128 (format code 0 for both operands, no block scaling).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 64-lane global->LDS copy of 16 (or 4) bytes per lane to lds_base + lane * size,
// issued from asm so that the compiler does not attach waits for it to unrelated
// LDS reads; completion is awaited by an s_waitcnt vmcnt before the next workgroup
// barrier.  M0 is saved and restored.  An SALU write of M0 needs one wait state
// before an LDS-DMA load reads it (the compiler inserts it for its own copies, not
// inside asm): without the s_nop the copy may land at the previous M0.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}
// Compile-time loop: f(std::integral_constant<int, M>) for M = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// dma16 with a wave-uniform base address (SGPR pair) and a per-lane 32-bit byte offset plus
// an immediate offset (the copy's scalar-base form): no 64-bit address arithmetic per lane.
// The instruction's immediate offset moves the LDS destination as well as the global
// address, so M0 is set IMM bytes below the intended LDS base.
template <int IMM>
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds_base) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 offset:%4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base) - (uint32_t)IMM), "i"(IMM)
      : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt), not for outstanding global->LDS copies (vmcnt).  The "memory"
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48), all lanes get it
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48), all lanes get it.
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Last key row visible to packed query row i of sequence b (sequence-local): its token
// position t in token mode (s <= t), floor(t / block) - 1 with a compression ratio
// block > 1 (compressed block s is visible iff s < floor(t / block); -1: none).
__device__ __forceinline__ int64_t row_last(const dsa_seqs& s, int b, int64_t i) {
  const int64_t t = s.q_pos0[b] + (i - s.q_start[b]);
  return s.block > 1 ? t / s.block - 1 : t;
}

// Locate the sequence that owns packed query row i (wave-uniform; the table is
// a kernel argument, so this is a short scalar loop).
__device__ __forceinline__ int seq_of_row(const dsa_seqs& s, int64_t i) {
  int b = 0;
  while (b + 1 < s.B && i >= s.q_start[b + 1]) ++b;
  return b;
}

}  // namespace dsa
