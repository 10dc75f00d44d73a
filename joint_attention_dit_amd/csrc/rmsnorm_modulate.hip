// RMSNorm + AdaLN modulation (apxml.com spec page: RMS normalisation, scaled
// and shifted by the AdaLN modulation). One wavefront per token row:
//   pass 1: sum of squares in fp64 (squares of bf16 / fp32 values are exact);
//   pass 2: h = x * r * (1 + scale) + shift in fp64, one rounding to bf16.
// The second pass re-reads the row (an L2 hit), so HBM traffic is one read
// of x and one write of h.
#include "common.h"
#include "kernels.h"

namespace h3dit {

template <typename XT>
struct Chunk8;

template <>
struct Chunk8<bf16> {
  static __device__ __forceinline__ void load(const bf16 *p, float v[8]) {
    const bf16x8 t = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)t[j];
  }
};

template <>
struct Chunk8<float> {
  static __device__ __forceinline__ void load(const float *p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
};

template <typename XT>
__global__ __launch_bounds__(256) void rmsnorm_modulate_kernel(const XT *__restrict__ x,
                                                               const double *__restrict__ shift,
                                                               const double *__restrict__ scale,
                                                               bf16 *__restrict__ h, int T, int D,
                                                               double eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const XT *xr = x + (int64_t)row * D;
  bf16 *hr = h + (int64_t)row * D;
  const int chunks = D >> 3;

  double ss = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    Chunk8<XT>::load(xr + c * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += (double)v[j] * (double)v[j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double r = 1.0 / sqrt(ss / (double)D + eps);

  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    Chunk8<XT>::load(xr + c * 8, v);
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = c * 8 + j;
      o[j] = to_bf16((double)v[j] * r * (1.0 + scale[col]) + shift[col]);
    }
    *reinterpret_cast<bf16x8 *>(hr + c * 8) = o;
  }
}

hipError_t launch_rmsnorm_modulate(const void *x, bool x_is_f32, const double *shift,
                                   const double *scale, void *h, int T, int D, float eps,
                                   hipStream_t s) {
  const int blocks = (int)ceil_div(T, 4);
  if (x_is_f32)
    hipLaunchKernelGGL(rmsnorm_modulate_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float *>(x), shift, scale, static_cast<bf16 *>(h), T, D,
                       (double)eps);
  else
    hipLaunchKernelGGL(rmsnorm_modulate_kernel<bf16>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const bf16 *>(x), shift, scale, static_cast<bf16 *>(h), T, D,
                       (double)eps);
  return hipGetLastError();
}

}  // namespace h3dit
