// Joint bidirectional attention over the packed text + image sequence
// (model card, "Model Architecture": every token sits in one packed sequence
// of a single-stream transformer; spec page: 56 query and 56 key-value heads
// of dimension 128). Flash-style: keys and values are visited in tiles of 64
// with an online softmax, so no T x T matrix is ever stored.
//
// Work split: a workgroup owns 256 queries of one head (eight waves of 32, two
// waves per SIMD so that one wave's softmax overlaps the other's matrix-core
// work). Each wave computes the transposed score tile S^T = K Q^T with the
// 32x32x16 bf16 MFMA, so a lane holds 32 of the 64 scores of ONE query (the
// other 32 sit in lane l ^ 32): row maxima and sums need one cross-lane
// exchange. The output is accumulated transposed as well, O^T += V^T P^T;
// the MFMA's K slots of that product are assigned to keys in the order in
// which the score registers hold them (lane half G holds keys 4G..4G+3 and
// 8+4G..8+4G+3 of every 16), and V^T is stored in global memory with bits 2
// and 3 of the key index exchanged, so each such fragment is one 16-byte read.
//
// Softmax weights: s = q.k * log2(e) / sqrt(128); the running maximum is
// rounded up to an integer m, and P = bf16(2^(s - m)). Because rescaling
// between tiles is by an exact power of two, the bf16 weights do not depend
// on the order of the key tiles; o = bf16(sum P v / sum P), where the sum
// runs over the rounded weights.
//
// K tiles ([64 keys][128 dims], 256-byte rows, 16-byte chunk c stored at
// c ^ (row & 15)) and V^T tiles ([128 dims][64 keys], 128-byte rows, chunk c at
// c ^ ((row >> 1) & 7)) stream straight from global memory into a 3-stage LDS
// ring (gfx950's global-load-to-LDS), two tiles ahead, one barrier per tile.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace h3dit {

namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int QT = 32 * NW;        // queries per workgroup
constexpr int NTHREADS = 64 * NW;  // threads per workgroup
constexpr int KT = 64;             // keys per tile
constexpr int NST = 3;             // LDS stages
constexpr int K_ELEMS = KT * 128;  // bf16 elements of one K tile (16 KB)
constexpr int V_ELEMS = 128 * KT;  // bf16 elements of one V^T tile (16 KB)
constexpr int STAGE_ELEMS = K_ELEMS + V_ELEMS;

typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N of this wave's tile loads are in flight (they complete
// in issue order), then meet the other waves.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  constexpr int enc = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(enc);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

__global__ __launch_bounds__(NTHREADS, 2) void attention_kernel(const bf16 *__restrict__ qk,
                                                          const bf16 *__restrict__ vt,
                                                          bf16 *__restrict__ o, int T, int H,
                                                          int Tp) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[NST * STAGE_ELEMS];  // 96 KB

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Tile loads: wave w fills 1 KB blocks 2w, 2w+1 of the K tile (4 rows of 256 B
  // each) and of the V^T tile (8 rows of 128 B each). Lane l lands at byte 16 l
  // of its block, so it fetches the logical chunk that the swizzle puts there.
  const bf16 *ksrc[2];
  const bf16 *vsrc[2];
  int krow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = (2 * wave + j) * 4 + (lane >> 4);  // key row within the tile
    const int kc = (lane & 15) ^ (kr & 15);
    krow[j] = kr;
    ksrc[j] = qk + A + h * 128 + kc * 8;
    const int vr = (2 * wave + j) * 8 + (lane >> 3);  // dim row of V^T
    const int vc = (lane & 7) ^ ((vr >> 1) & 7);
    vsrc[j] = vt + (int64_t)(h * 128 + vr) * Tp + vc * 8;
  }
  auto tload = [&](int stage, int kv0) {
    bf16 *sk = lds + stage * STAGE_ELEMS + wave * 2 * 512;
    bf16 *sv = lds + stage * STAGE_ELEMS + K_ELEMS + wave * 2 * 512;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = min(kv0 + krow[j], T - 1);
      __builtin_amdgcn_global_load_lds(ksrc[j] + (int64_t)key * ldqk, (lds_void *)(sk + j * 512),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(vsrc[j] + kv0, (lds_void *)(sv + j * 512), 16, 0, 0);
    }
  };

  // fragment read offsets within a stage (elements)
  int koff[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = 32 * b + c;
      koff[b][s] = r * 128 + (((2 * s + G) ^ (r & 15)) * 8);
    }
  int voff[4][4];  // [db][chunk pair index p = 2 b + half]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int d = db * 32 + c;
      voff[db][p] = K_ELEMS + d * 64 + (((2 * p + G) ^ ((d >> 1) & 7)) * 8);
    }

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  const int ntiles = (int)ceil_div(T, KT);
  tload(0, 0);
  if (ntiles > 1) tload(1, KT);

  for (int it = 0; it < ntiles; ++it) {
    const int stage = it % NST;
    const int kv0 = it * KT;
    // tile it has landed for every wave, and tile it-1's stage is free
    if (it + 1 < ntiles) tile_barrier<4>();
    else tile_barrier<0>();
    if (it + 2 < ntiles) tload((it + 2) % NST, (it + 2) * KT);
    const bf16 *sb = lds + stage * STAGE_ELEMS;

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
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(sb + koff[b][s]);
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

    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(sacc[0][v], sacc[1][v]));
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
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(sacc[b][2 * u + 1], kLog2eOverSqrt128, -m_new));
        pk[b][u] = pack2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[b][u], ones, l_run, false);
      }

    // O^T[dim][query] += V^T[dim][keys] P^T[keys][query]; K step j covers
    // score block b = j / 2, registers 8 (j % 2) .. +7.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = j >> 1, half = j & 1;
      const bf16x8 pf = as_bf16x8(pk[b][4 * half], pk[b][4 * half + 1], pk[b][4 * half + 2],
                                  pk[b][4 * half + 3]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(sb + voff[db][j]);
        oacc[db] = mfma32(vf, pf, oacc[db]);
      }
    }
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
  hipLaunchKernelGGL(attention_kernel, grid, dim3(NTHREADS), 0, s, static_cast<const bf16 *>(qk),
                     static_cast<const bf16 *>(vt), static_cast<bf16 *>(o), T, H, Tp);
  return hipGetLastError();
}

}  // namespace h3dit
