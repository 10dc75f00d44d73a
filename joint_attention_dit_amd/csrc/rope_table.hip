// 2D axial RoPE table (model card: multimodal RoPE; read here as a 2D axial
// rotation): entry (t, j) holds cos and sin of position[t][j / 32] times
// base^(-(j % 32) / 32), i.e. pair i = j % 32 of half j / 32 (half 0 = row,
// half 1 = column). Angles are formed and evaluated in fp64, stored as fp32.
#include "common.h"
#include "kernels.h"

namespace h3dit {

__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t *__restrict__ pos,
                                                         float *__restrict__ table, int T,
                                                         double log2_base) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * 64) return;
  const int t = (int)(idx >> 6);
  const int j = (int)(idx & 63);
  const double theta = exp2(-(double)(j & 31) / 32.0 * log2_base);
  const double ang = (double)pos[2 * t + (j >> 5)] * theta;
  double sn, cs;
  sincos(ang, &sn, &cs);
  f32x2 v = {(float)cs, (float)sn};
  *reinterpret_cast<f32x2 *>(table + 2 * idx) = v;
}

hipError_t launch_rope_table(const int32_t *pos, float *table, int T, float base, hipStream_t s) {
  const int64_t n = (int64_t)T * 64;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, pos,
                     table, T, log2((double)base));
  return hipGetLastError();
}

}  // namespace h3dit
