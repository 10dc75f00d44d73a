// bf16 matrix-core GEMM with fused epilogues for the DiT block's linears
// (QKV, output projection, MLP up, MLP down; model card, "Model
// Architecture", and the spec page's block diagram).
//
//   C[t, n] = sum_k X[t, k] * W[n, k]      X: activations [M, K], W: weights [N, K]
//
// Both operands are K-contiguous, so both feed the 32x32x16 bf16 MFMA
// directly. The weight rows are the MFMA "A" rows and the token rows the
// "B" columns, which leaves every lane holding four consecutive output
// features of one token: RoPE pairs (2i, 2i+1) sit in one lane and stores are
// 8- or 16-byte vectors.
//
// Tiling: 256 features x 256 tokens per workgroup, K step 64, four waves in a
// 2 x 2 arrangement, each owning 128 x 128 outputs (4 x 4 MFMA blocks, 256
// fp32 accumulators per lane). Tiles are staged through LDS, double
// buffered (2 stages x 2 operands x 32 KB), with a register prefetch of the
// next K step while the current one is multiplied. LDS rows are 128 bytes;
// 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7) so that the
// 32 rows read by one fragment load spread over all banks.
//
// Workgroup order: the dispatcher hands workgroup i to XCD i % 8. The
// linear id is remapped so that each XCD receives a contiguous range of
// tiles, and tiles are walked in groups of 8 token tiles so that the tiles
// in flight on one XCD share weight and activation panels in its L2.
#include "common.h"
#include "kernels.h"

namespace h3dit {

namespace {

constexpr int BN = 256;   // weight rows (output features) per tile
constexpr int BT = 256;   // activation rows (tokens) per tile
constexpr int BK = 64;    // K per LDS stage
constexpr int TILE_ELEMS = 256 * BK;  // one operand tile, bf16 elements
constexpr int GROUP_T = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_n, int tiles_t,
                                            int &tn, int &tt) {
  // XCD-contiguous remap (bijective for any nblocks)
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
  // grouped walk: GROUP_T token tiles per group, features outer within the group
  const int per_group = GROUP_T * tiles_n;
  const int g = L / per_group;
  const int first_t = g * GROUP_T;
  const int gt = min(tiles_t - first_t, GROUP_T);
  const int in = L - g * per_group;
  tt = first_t + in % gt;
  tn = in / gt;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  // 0.5 z (1 + tanh(y)) == z / (1 + exp(-2y)),  y = sqrt(2/pi) (z + 0.044715 z^3)
  const float y = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  return z / (1.0f + expf(-2.0f * y));
}

template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const f32x16 (&acc)[4][4], int n_base,
                                         int t_base, int lane) {
  const int G = lane >> 5, c = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t_base + j * 32 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n_base + i * 32 + 8 * g + 4 * G;
        if (n >= a.N) continue;
        const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if constexpr (EPI == EPI_QKV_ROPE) {
          const int A2 = 2 * a.A;
          if (n < A2) {
            if (t >= a.M) continue;
            // q or k: round, rotate the two adjacent pairs, round again
            const float u0 = bf16_round_f32(v0), w0 = bf16_round_f32(v1);
            const float u1 = bf16_round_f32(v2), w1 = bf16_round_f32(v3);
            const int p = (n & 127) >> 1;  // pair index within the head (0..63)
            const f32x4 cs = *reinterpret_cast<const f32x4 *>(a.table + ((int64_t)t * 64 + p) * 2);
            bf16x4 r;
            r[0] = to_bf16(u0 * cs[0] - w0 * cs[1]);
            r[1] = to_bf16(u0 * cs[1] + w0 * cs[0]);
            r[2] = to_bf16(u1 * cs[2] - w1 * cs[3]);
            r[3] = to_bf16(u1 * cs[3] + w1 * cs[2]);
            *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(a.out) + (int64_t)t * A2 + n) = r;
          } else {
            if (t >= a.Mp) continue;
            const int hv = n - A2;  // head * 128 + dim
            bf16 *vt = static_cast<bf16 *>(a.out2) + (int64_t)hv * a.Mp + t;
            const bool live = t < a.M;
            vt[0] = to_bf16(live ? v0 : 0.0f);
            vt[a.Mp] = to_bf16(live ? v1 : 0.0f);
            vt[2 * (int64_t)a.Mp] = to_bf16(live ? v2 : 0.0f);
            vt[3 * (int64_t)a.Mp] = to_bf16(live ? v3 : 0.0f);
          }
        } else if constexpr (EPI == EPI_RESID_BF16 || EPI == EPI_RESID_F32) {
          if (t >= a.M) continue;
          const int64_t off = (int64_t)t * a.N + n;
          f32x4 rv;
          if constexpr (EPI == EPI_RESID_BF16) {
            const bf16x4 rb = *reinterpret_cast<const bf16x4 *>(static_cast<const bf16 *>(a.resid) + off);
            rv = f32x4{(float)rb[0], (float)rb[1], (float)rb[2], (float)rb[3]};
          } else {
            rv = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.resid) + off);
          }
          f32x4 ov;
          ov[0] = rv[0] + (float)a.gate[n + 0] * v0;
          ov[1] = rv[1] + (float)a.gate[n + 1] * v1;
          ov[2] = rv[2] + (float)a.gate[n + 2] * v2;
          ov[3] = rv[3] + (float)a.gate[n + 3] * v3;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + off) = ov;
        } else if constexpr (EPI == EPI_F32) {
          if (t >= a.M) continue;
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (int64_t)t * a.N + n) =
              f32x4{v0, v1, v2, v3};
        } else {  // EPI_GELU
          if (t >= a.M) continue;
          bf16x4 r;
          r[0] = to_bf16(gelu_tanh(v0));
          r[1] = to_bf16(gelu_tanh(v1));
          r[2] = to_bf16(gelu_tanh(v2));
          r[3] = to_bf16(gelu_tanh(v3));
          *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(a.out) + (int64_t)t * a.N + n) = r;
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * 2 * TILE_ELEMS];  // 128 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wt = wave >> 1;
  const int tiles_n = (int)ceil_div(a.N, BN), tiles_t = (int)ceil_div(a.M, BT);
  int tn, tt;
  tile_coords(blockIdx.x, gridDim.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BN, t0 = tt * BT;

  // global -> LDS assignment: chunk (tid & 7) of rows (tid >> 3) + 32 j
  const int lrow = tid >> 3, lchunk = tid & 7;
  const bf16 *wsrc = static_cast<const bf16 *>(a.w);
  const bf16 *xsrc = static_cast<const bf16 *>(a.x);
  int64_t woff[8], xoff[8];
  int soff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = lrow + 32 * j;
    woff[j] = (int64_t)min(n0 + row, a.N - 1) * a.K + lchunk * 8;
    xoff[j] = (int64_t)min(t0 + row, a.M - 1) * a.K + lchunk * 8;
    soff[j] = row * BK + swz(row, lchunk) * 8;
  }

  u32x4 wreg[8], xreg[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      wreg[j] = *reinterpret_cast<const u32x4 *>(wsrc + woff[j] + k0);
      xreg[j] = *reinterpret_cast<const u32x4 *>(xsrc + xoff[j] + k0);
    }
  };
  auto sstore = [&](int stage) {
    bf16 *sw = lds + stage * 2 * TILE_ELEMS;
    bf16 *sx = sw + TILE_ELEMS;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<u32x4 *>(sw + soff[j]) = wreg[j];
      *reinterpret_cast<u32x4 *>(sx + soff[j]) = xreg[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment read offsets (rows of this wave, lane's row within a 32-block)
  const int c = lane & 31, G = lane >> 5;
  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = wn * 128 + i * 32 + c;
    brow[i] = wt * 128 + i * 32 + c;
  }

  const int ktiles = a.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ktiles) gload((kt + 1) * BK);
    const bf16 *sw = lds + cur * 2 * TILE_ELEMS;
    const bf16 *sx = sw + TILE_ELEMS;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = 2 * s + G;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8 *>(sw + arow[i] * BK + swz(arow[i], ch) * 8);
        bfr[i] = *reinterpret_cast<const bf16x8 *>(sx + brow[i] * BK + swz(brow[i], ch) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < ktiles) sstore(cur ^ 1);
    __syncthreads();
  }

  epilogue<EPI>(a, acc, n0 + wn * 128, t0 + wt * 128, lane);
}

}  // namespace

hipError_t launch_gemm(GemmEpilogue epi, const GemmArgs &a, hipStream_t s) {
  const int tiles = (int)(ceil_div(a.N, BN) * ceil_div(a.M, BT));
  switch (epi) {
    case EPI_QKV_ROPE:
      hipLaunchKernelGGL(gemm_kernel<EPI_QKV_ROPE>, dim3(tiles), dim3(256), 0, s, a);
      break;
    case EPI_RESID_BF16:
      hipLaunchKernelGGL(gemm_kernel<EPI_RESID_BF16>, dim3(tiles), dim3(256), 0, s, a);
      break;
    case EPI_RESID_F32:
      hipLaunchKernelGGL(gemm_kernel<EPI_RESID_F32>, dim3(tiles), dim3(256), 0, s, a);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL(gemm_kernel<EPI_GELU>, dim3(tiles), dim3(256), 0, s, a);
      break;
    case EPI_F32:
      hipLaunchKernelGGL(gemm_kernel<EPI_F32>, dim3(tiles), dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace h3dit
