// Joint bidirectional attention over the packed text + image sequence
// (model card, "Model Architecture": every token sits in one packed sequence
// of a single-stream transformer; spec page: 56 query and 56 key-value heads
// of dimension 128). Flash-style: keys and values are visited in tiles of 64
// with an online softmax, so no T x T matrix is ever stored.
//
// Layout of the work: a workgroup owns 128 queries of one head (four waves of
// 32). Each wave computes the transposed score tile S^T = K Q^T with the
// 32x32x16 bf16 MFMA, so a lane holds 32 of the 64 scores of ONE query (the
// other 32 sit in lane l ^ 32): row maxima and sums need one cross-lane
// exchange. The output is accumulated transposed as well, O^T += V^T P^T;
// the MFMA's K slots of that product are assigned to keys in the order in
// which the score registers hold them, and the V^T fragments are read from
// LDS in that same order.
//
// Softmax weights: s = q.k * log2(e) / sqrt(128); the running maximum is
// rounded up to an integer m, and P = bf16(2^(s - m)). Because rescaling
// between tiles is by an exact power of two, the bf16 weights do not depend
// on the order of the key tiles; o = bf16(sum P v / sum P), where the sum
// runs over the rounded weights.
//
// K tiles ([64 keys][128 dims], 256-byte rows, chunk swizzle c ^ (row & 15))
// and V^T tiles ([128 dims][64 keys], 128-byte rows, swizzle c ^ ((row>>1) & 7))
// are double buffered in LDS (64 KB per workgroup) with a register prefetch.
#include "common.h"
#include "kernels.h"

namespace h3dit {

namespace {

constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile
constexpr int K_ELEMS = KT * 128;
constexpr int V_ELEMS = 128 * KT;

__global__ __launch_bounds__(256, 2) void attention_kernel(const bf16 *__restrict__ qk,
                                                           const bf16 *__restrict__ vt,
                                                           bf16 *__restrict__ o, int T, int H,
                                                           int Tp) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * (K_ELEMS + V_ELEMS)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5, c = lane & 31;
  const int h = blockIdx.y;
  const int A = H * 128;
  const int64_t ldqk = 2 * (int64_t)A;
  const int q0 = blockIdx.x * QT + wave * 32;

  // this lane's query fragments: Q[q0 + c][16 s + 8 G .. +7], s = 0..7
  bf16x8 qf[8];
  {
    const int qrow = min(q0 + c, T - 1);
    const bf16 *qp = qk + (int64_t)qrow * ldqk + h * 128 + 8 * G;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
  }

  // tile load assignment
  const int kc = tid & 15, kr = tid >> 4;  // K: chunk kc of key rows kr + 16 j
  const int vc = tid & 7, vr = tid >> 3;   // V^T: chunk vc of dim rows vr + 32 j
  const bf16 *kbase = qk + A + h * 128 + kc * 8;
  const bf16 *vbase = vt + (int64_t)(h * 128 + vr) * Tp + vc * 8;
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int kv0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(kv0 + kr + 16 * j, T - 1);
      kreg[j] = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)key * ldqk);
      vreg[j] = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)(32 * j) * Tp + kv0);
    }
  };
  auto sstore = [&](int stage) {
    bf16 *sk = lds + stage * (K_ELEMS + V_ELEMS);
    bf16 *sv = sk + K_ELEMS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = kr + 16 * j;
      *reinterpret_cast<u32x4 *>(sk + r * 128 + ((kc ^ (r & 15)) * 8)) = kreg[j];
      const int d = vr + 32 * j;
      *reinterpret_cast<u32x4 *>(sv + d * 64 + ((vc ^ ((d >> 1) & 7)) * 8)) = vreg[j];
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  const int ntiles = (int)ceil_div(T, KT);
  gload(0);
  sstore(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kv0 = it * KT;
    if (it + 1 < ntiles) gload(kv0 + KT);
    const bf16 *sk = lds + cur * (K_ELEMS + V_ELEMS);
    const bf16 *sv = sk + K_ELEMS;

    // S^T[key][query] for keys kv0 + 32 b + (8 (v/4) + 4 G + v%4), query q0 + c
    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[b][v] = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int r = 32 * b + c;
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8 *>(sk + r * 128 + (((2 * s + G) ^ (r & 15)) * 8));
        sacc[b] = mfma32(kf, qf[s], sacc[b]);
      }
    }

    if (kv0 + KT > T) {  // ragged last tile: keys past T get zero weight
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kv0 + 32 * b + 8 * (v >> 2) + 4 * G + (v & 3);
          if (key >= T) sacc[b][v] = -INFINITY;
        }
    }

    float mx = sacc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[b][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, ceilf(mx * kLog2eOverSqrt128));
    if (__ballot(m_new > m_run)) {
      const float f = __builtin_amdgcn_exp2f(m_run - m_new);  // exact power of two (0 at start)
      l_run *= f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d][v] *= f;
    }
    m_run = m_new;

    // P = bf16(2^(s - m)), packed in pairs; row sum over the rounded weights
    bf16x2 pk[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[b][2 * u], kLog2eOverSqrt128, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[b][2 * u + 1], kLog2eOverSqrt128, -m_new));
        pk[b][u] = pack2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[b][u], ones, l_run, false);
      }

    // O^T[dim][query] += V^T[dim][keys] P^T[keys][query]; K step j covers
    // score block b = j / 2, registers 8 (j % 2) .. +7, i.e. the keys
    // 32 b + 16 (j % 2) + 4 G + {0..3} and the same + 8.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = j >> 1, half = j & 1;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[2 * e] = pk[b][4 * half + e][0];
        pf[2 * e + 1] = pk[b][4 * half + e][1];
      }
      const int ch0 = 4 * b + 2 * half;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + c;
        const int sw = (d >> 1) & 7;
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(sv + d * 64 + ((ch0 ^ sw) * 8) + 4 * G);
        const bf16x4 hi =
            *reinterpret_cast<const bf16x4 *>(sv + d * 64 + (((ch0 + 1) ^ sw) * 8) + 4 * G);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = mfma32(vf, pf, oacc[db]);
      }
    }

    if (it + 1 < ntiles) sstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int q = q0 + c;
  if (q < T) {
    bf16 *op = o + (int64_t)q * A + h * 128 + 4 * G;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = to_bf16(oacc[db][4 * g + e] / l_tot);
        *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * g) = r;
      }
  }
}

}  // namespace

hipError_t launch_attention(const void *qk, const void *vt, void *o, int T, int H, int Tp,
                            hipStream_t s) {
  dim3 grid((unsigned)ceil_div(T, QT), (unsigned)H);
  hipLaunchKernelGGL(attention_kernel, grid, dim3(256), 0, s, static_cast<const bf16 *>(qk),
                     static_cast<const bf16 *>(vt), static_cast<bf16 *>(o), T, H, Tp);
  return hipGetLastError();
}

}  // namespace h3dit
