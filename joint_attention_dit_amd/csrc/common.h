// Shared device types and helpers for the gfx950 kernels of the DiT block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3dit {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// log2(e) / sqrt(128): turns a q.k dot product into a base-2 softmax exponent.
constexpr float kLog2eOverSqrt128 = (float)(1.4426950408889634 / 11.313708498984761);

// Round-to-nearest-even conversions (gfx950 converts f32 pairs in hardware;
// the f64 path rounds to odd first, so it is a single correct rounding).
__device__ __forceinline__ bf16 to_bf16(float v) { return (bf16)v; }
__device__ __forceinline__ bf16 to_bf16(double v) { return (bf16)v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

__device__ __forceinline__ bf16x2 pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ float bf16_round_f32(float v) { return (float)(bf16)v; }

// Load of data that one kernel reads once (weights of a GEMV, rows of a
// normalisation): the nontemporal hint lets the caches drop the line instead of
// keeping it over data that is reused.
template <typename T>
__device__ __forceinline__ T load_once(const T *p) {
  return __builtin_nontemporal_load(p);
}

// 32x32x16 bf16 matrix-core product with fp32 accumulation.
// Lane l supplies A[l % 32][8 * (l / 32) .. +7] and B[8 * (l / 32) .. +7][l % 32];
// it receives C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32] in element i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product with fp32 accumulation.
// Lane l supplies A[l % 16][8 * (l / 16) .. +7] and B[8 * (l / 16) .. +7][l % 16];
// it receives C[4 * (l / 16) + i][l % 16] in element i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte global -> LDS copy per lane (gfx950's global-load-to-LDS): lane
// l reads base + voff (bytes; base wave-uniform) and writes LDS bytes
// lds_addr + 16 l (lds_addr wave-uniform). It is issued as an instruction the
// compiler does not model: with such a copy in flight the compiler otherwise
// waits for every outstanding LDS read at each use. Callers therefore await
// completion themselves (s_waitcnt vmcnt before the barrier that publishes
// the tile).
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_addr) {
  // m0 (the LDS destination) is an input constraint, so the compiler knows the
  // block reads it; the s_nop covers the m0 -> LDS-DMA hazard
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "{m0}"(lds_addr)
               : "memory");
}

// Byte address of an LDS object, as the wave-uniform value dma16 takes.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace h3dit
