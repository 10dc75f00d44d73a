// Device helpers of MXFP8 quantisation (OCP 8-bit floating point E4M3
// elements, one E8M0 scale per 32 consecutive elements along K; the MXFP8
// linears of the vLLM blog "H3-Image Day-0 Support", section Inference
// Optimizations), shared by the quantisation kernel and the producers that
// quantise their own output (the normalisation and the GELU epilogue).
//
// Scale: X = floor(log2(max |v|)) - 8 for a block with largest magnitude
// max |v| > 0, X = -127 for an all-zero block, stored as the byte X + 127.
// Elements: E4M3 code of v * 2^-X, rounded to nearest, ties to even,
// magnitudes of 448 and above saturating to 448, sign kept on zero.
//
// The element conversion is gfx950's v_cvt_pk_fp8_f32 (OCP E4M3, round to
// nearest even) of v * 2^-X clamped to [-448, 448]; the product is exact (a
// power of two times a bf16 value, never below the fp32 normal range that
// matters: results under 2^-10 become a signed zero either way). It agrees
// with an integer reference conversion on every finite bf16 value at every
// scale byte 0..246 (checked exhaustively on the GPU).
#pragma once

#include "common.h"

namespace h3dit {

// Scale byte X + 127 of a block whose largest magnitude has the bf16 bit
// pattern amax (sign cleared): floor(log2) is the exponent field minus 127,
// so the byte is the exponent field minus 8, at least 0.
__device__ __forceinline__ int mx_scale_byte(uint32_t amax_bits) {
  const int ex = (int)(amax_bits >> 7);
  return ex > 8 ? ex - 8 : 0;
}

// 2^-X = 2^(127 - byte) as an fp32 value (byte <= 246 for finite bf16 input).
__device__ __forceinline__ float mx_inv_scale(int sbyte) {
  return __uint_as_float((uint32_t)(254 - sbyte) << 23);
}

// Four values (already bf16-exact) to four E4M3 codes, byte i = value i.
__device__ __forceinline__ uint32_t mx_code4(float a, float b, float c, float d, float inv) {
  const float lo = -448.0f, hi = 448.0f;
  a = __builtin_amdgcn_fmed3f(a * inv, lo, hi);
  b = __builtin_amdgcn_fmed3f(b * inv, lo, hi);
  c = __builtin_amdgcn_fmed3f(c * inv, lo, hi);
  d = __builtin_amdgcn_fmed3f(d * inv, lo, hi);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// Value of a bf16 bit pattern (16 low bits) as fp32.
__device__ __forceinline__ float mx_bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// Byte offset of the scale of row `row` and 32-element block `kblk` (along K)
// in the 1 KB block layout: block (row / 256, kblk / 4) at
// ((row / 256) * (K / 128) + kblk / 4) * 1024, then byte
// ((kblk % 4) * 16 + row % 16) * 16 + (row % 256) / 16.
__device__ __forceinline__ int64_t mx_scale_offset(int row, int kblk, int K) {
  return ((int64_t)(row >> 8) * (K >> 7) + (kblk >> 2)) * 1024 +
         (((kblk & 3) * 16 + (row & 15)) * 16 + ((row & 255) >> 4));
}

}  // namespace h3dit
