// The pieces of the DiT stack around the blocks (model card, "Model
// Architecture": latents are cut into patches that become image tokens of the
// packed sequence; the DiT's output is projected back to latent patches). A
// latent [C, H, W] with patch size p becomes gh * gw = (H / p) * (W / p) image
// tokens of C * p * p values; an fp32 linear embeds them into the hidden width
// and, after the blocks, a modulated RMSNorm plus an fp32 linear map the image
// tokens back to C * p * p values per token.
#include "common.h"
#include "kernels.h"

namespace h3dit {

namespace {

// one thread per patch value: coalesced writes along the token row
__global__ __launch_bounds__(256) void patchify_kernel(const float *__restrict__ latent,
                                                       float *__restrict__ patches, int C, int p,
                                                       int gh, int gw) {
  const int pp = p * p, F = C * pp;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)gh * gw * F) return;
  const int t = (int)(i / F), f = (int)(i % F);
  const int gy = t / gw, gx = t % gw;
  const int c = f / pp, dy = (f % pp) / p, dx = f % p;
  const int W = gw * p;
  patches[i] = latent[((int64_t)c * gh * p + gy * p + dy) * W + gx * p + dx];
}

// one thread per latent value: coalesced writes along the latent row
__global__ __launch_bounds__(256) void unpatchify_kernel(const float *__restrict__ vt,
                                                         float *__restrict__ v, int C, int p,
                                                         int gh, int gw) {
  const int H = gh * p, W = gw * p, pp = p * p;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)C * H * W) return;
  const int c = (int)(i / ((int64_t)H * W));
  const int rem = (int)(i % ((int64_t)H * W));
  const int yy = rem / W, xx = rem % W;
  const int t = (yy / p) * gw + xx / p;
  const int f = c * pp + (yy % p) * p + xx % p;
  v[i] = vt[(int64_t)t * C * pp + f];
}

// fp32 GEMM, y = a . b^T: 64 x 64 output tile per workgroup, k chunks of 16
// staged in LDS (k-major, so each thread's 4 x 4 outputs read broadcast
// fragments), 256 threads of 4 x 4 outputs each.
constexpr int GT = 64, GK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ a,
                                                       const float *__restrict__ b,
                                                       float *__restrict__ y, int M, int N, int K,
                                                       int ldy) {
  __shared__ float as[GK][GT + 4];
  __shared__ float bs[GK][GT + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int tr = tid >> 4, tc = tid & 15;  // 16 x 16 threads, 4 x 4 outputs each
  // loader: thread -> (row lr, 4 consecutive k at lk)
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += GK) {
    const int k = k0 + lk;
    f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
    if (m0 + lr < M && k < K) va = *reinterpret_cast<const f32x4 *>(a + (int64_t)(m0 + lr) * K + k);
    if (n0 + lr < N && k < K) vb = *reinterpret_cast<const f32x4 *>(b + (int64_t)(n0 + lr) * K + k);
    __syncthreads();  // the previous chunk has been consumed
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      as[lk + j][lr] = va[j];
      bs[lk + j][lr] = vb[j];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      const f32x4 fa = *reinterpret_cast<const f32x4 *>(&as[kk][tr * 4]);
      const f32x4 fb = *reinterpret_cast<const f32x4 *>(&bs[kk][tc * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(fa[i], fb[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tr * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tc * 4 + j;
      if (n < N) y[(int64_t)m * ldy + n] = acc[i][j];
    }
  }
}

__global__ __launch_bounds__(256) void latent_step_kernel(float *__restrict__ latent,
                                                          const float *__restrict__ v, float dt,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) latent[i] = fmaf(dt, v[i], latent[i]);
}

}  // namespace

hipError_t launch_patchify(const float *latent, float *patches, int C, int p, int gh, int gw,
                           hipStream_t s) {
  const int64_t n = (int64_t)gh * gw * C * p * p;
  hipLaunchKernelGGL(patchify_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, latent,
                     patches, C, p, gh, gw);
  return hipGetLastError();
}

hipError_t launch_unpatchify(const float *vt, float *v, int C, int p, int gh, int gw,
                             hipStream_t s) {
  const int64_t n = (int64_t)gh * gw * C * p * p;
  hipLaunchKernelGGL(unpatchify_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, vt, v,
                     C, p, gh, gw);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float *a, const float *b, float *y, int M, int N, int K, int ldy,
                           hipStream_t s) {
  dim3 grid((unsigned)ceil_div(N, GT), (unsigned)ceil_div(M, GT));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, a, b, y, M, N, K, ldy);
  return hipGetLastError();
}

hipError_t launch_latent_step(float *latent, const float *v, float dt, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(latent_step_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, latent,
                     v, dt, n);
  return hipGetLastError();
}

}  // namespace h3dit
