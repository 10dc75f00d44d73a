// AdaLN modulation: mod = W_ada . cond (apxml.com spec page, "Architecture
// Diagram": the AdaLN modulation turns the timestep conditioning into
// per-channel shift / scale / gate). One wavefront per output row; each lane
// streams 16-byte chunks of the bf16 row and accumulates in fp64 (the
// bf16 x fp32 products are exact in fp64). HBM-bound: every weight byte is
// read once.
#include "common.h"
#include "kernels.h"

namespace h3dit {

__global__ __launch_bounds__(256) void modulation_kernel(const bf16 *__restrict__ w,
                                                         const float *__restrict__ cond,
                                                         double *__restrict__ mod, int rows,
                                                         int cols) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bf16 *wr = w + (int64_t)row * cols;
  const int chunks = cols >> 3;
  double acc = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    const bf16x8 wv = *reinterpret_cast<const bf16x8 *>(wr + c * 8);
    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cond + c * 8);
    const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cond + c * 8 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += (double)(float)wv[j] * (double)c0[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += (double)(float)wv[4 + j] * (double)c1[j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) mod[row] = acc;
}

hipError_t launch_modulation(const void *w, const float *cond, double *mod, int rows, int cols,
                             hipStream_t s) {
  const int blocks = (int)ceil_div(rows, 4);
  hipLaunchKernelGGL(modulation_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const bf16 *>(w), cond, mod, rows, cols);
  return hipGetLastError();
}

}  // namespace h3dit
