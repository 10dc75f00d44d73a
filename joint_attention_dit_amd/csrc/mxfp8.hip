// MXFP8 quantisation of bf16 rows along K, the operand format of the MXFP8
// linears (vLLM blog "H3-Image Day-0 Support", section Inference
// Optimizations, runs the DiT's linears in MXFP8; the element and block
// formats are the OCP 8-bit floating point and Microscaling definitions).
//
// Each run of 32 consecutive elements of a row shares the scale 2^X with
// X = floor(log2(max |v|)) - 8 (8 is E4M3's largest exponent), stored as the
// E8M0 byte X + 127; an all-zero block takes X = -127 (byte 0). Each element
// becomes the E4M3 code of v * 2^-X rounded to nearest, ties to even, with
// magnitudes of 448 and above saturating to 448 and the sign kept when the
// value rounds to zero.
//
// Layouts: codes [rows, K] bytes, row-major. Scales in 1 KB blocks, one per
// (panel of 256 rows, K tile of 128); block (panel p, K tile t) starts at
// byte (p * K / 128 + t) * 1024, and the scale of panel row 16 b + r
// (b, r < 16) and 32-element block kb (< 4) of the K tile is its byte
// (kb * 16 + r) * 16 + b. That is the order in which the MXFP8 GEMM's lanes
// read them (gemm_mx.hip). Rows of the last panel past `rows` get byte 0.
#include "common.h"
#include "kernels.h"
#include "mxfp8_device.h"

namespace h3dit {

namespace {

// One workgroup per (panel of 256 rows, K tile of 128). Each pass of a wave
// covers 4 rows of 256 bytes (16 lanes per row, 8 elements per lane); the 4
// lanes of a 32-element block find its maximum with two exchanges.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const bf16 *__restrict__ x, int rows,
                                                             int K, uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t sc[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int panel = blockIdx.x, kt = blockIdx.y;
  const int chunk = lane & 15, kb = chunk >> 2;
  const int64_t k0 = (int64_t)kt * 128 + chunk * 8;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int rl = it * 16 + wave * 4 + (lane >> 4);  // row within the panel
    const int row = panel * 256 + rl;
    const bool live = row < rows;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4 *>(x + (int64_t)row * K + k0);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = w[i] & 0xFFFFu;
      h[2 * i + 1] = w[i] >> 16;
    }
    // largest magnitude of the block: magnitudes of finite bf16 values order
    // like their bit patterns without the sign
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, h[i] & 0x7FFFu);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const int sbyte = mx_scale_byte(amax);
    const float inv = mx_inv_scale(sbyte);
    const uint32_t lo = mx_code4(mx_bf16_value(h[0]), mx_bf16_value(h[1]), mx_bf16_value(h[2]),
                                 mx_bf16_value(h[3]), inv);
    const uint32_t hi = mx_code4(mx_bf16_value(h[4]), mx_bf16_value(h[5]), mx_bf16_value(h[6]),
                                 mx_bf16_value(h[7]), inv);
    if (live) *reinterpret_cast<u32x2 *>(codes + (int64_t)row * K + k0) = u32x2{lo, hi};
    if ((lane & 3) == 0) sc[(kb * 16 + (rl & 15)) * 16 + (rl >> 4)] = (uint8_t)(live ? sbyte : 0);
  }
  __syncthreads();
  if (tid < 64)
    *reinterpret_cast<u32x4 *>(scales + ((int64_t)panel * (K / 128) + kt) * 1024 + tid * 16) =
        *reinterpret_cast<const u32x4 *>(sc + tid * 16);
}

}  // namespace

hipError_t launch_mxfp8_quantize(const void *x, int rows, int K, uint8_t *codes, uint8_t *scales,
                                 hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rows, 256), (unsigned)(K / 128));
  hipLaunchKernelGGL(mxfp8_quantize_kernel, grid, dim3(256), 0, s, static_cast<const bf16 *>(x),
                     rows, K, codes, scales);
  return hipGetLastError();
}

}  // namespace h3dit
