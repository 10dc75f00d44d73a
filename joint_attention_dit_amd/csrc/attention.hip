// Joint bidirectional attention over the packed text + image sequence
// (model card, "Model Architecture": every token sits in one packed sequence
// of a single-stream transformer; spec page: 56 query and 56 key-value heads
// of dimension 128). Flash-style: keys and values are visited in tiles of 64
// with an online softmax, so no T x T matrix is ever stored.
//
// Work split: a workgroup owns 256 queries of one head (eight waves of 32, two
// waves per SIMD). Each wave computes the transposed score tile S^T = K Q^T
// with the 32x32x16 bf16 MFMA, so a lane holds 32 of the 64 scores of ONE
// query (the other 32 sit in lane l ^ 32). The output is accumulated
// transposed as well, O^T += V^T P^T; the MFMA's K slots of that product are
// assigned to keys in the order in which the score registers hold them (lane
// half G holds keys 4G..4G+3 and 8+4G..8+4G+3 of every 16), and V^T is stored
// in global memory with bits 2 and 3 of the key index exchanged, so each such
// fragment is one 16-byte read.
//
// Pipeline: after the barrier of key tile i, a wave multiplies the scores of
// tile i+1 on the matrix cores while its vector ALUs turn the scores of tile i
// into weights, then accumulates P(i) V(i). K and V^T tiles are double
// buffered in LDS and stream in one tile ahead through gfx950's global-to-LDS
// loads; there is one barrier per tile.
//
// Softmax weights. The stored queries already carry the factor log2(e)/sqrt(128)
// (the QKV epilogue applies it before rounding q to bf16), so a score
// s = q.k is in base-2 units, and P = bf16(2^(s - m)) for an integer shift m
// per query. The score MFMAs start their accumulation from -m, so the matrix
// cores deliver s - m and each weight costs one exp2. m is not raised tile by
// tile: it is set from the first tile's maximum, and afterwards only when
// some lane's sum of its 32 new weights exceeds 2^32 is the tile's maximum
// taken, m raised to its rounded-up value, the running output and sum
// rescaled by the exact power of two 2^(m_old - m_new), and the tile's weights
// formed again. Every weight is therefore at most 2^32. Because rescaling by
// a power of two commutes with bf16 rounding, the result equals that of the
// single shift ceil(max over all keys): o = bf16(sum P v / sum P), the sum
// taken over the rounded weights.
//
// LDS layouts: K tile [64 keys][128 dims], 256-byte rows, 16-byte chunk c
// stored at c ^ (row & 15); V^T tile [128 dims][64 keys], 128-byte rows,
// chunk c at c ^ ((row >> 1) & 7). Both make the fragment reads conflict-free.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace h3dit {

namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int QT = 32 * NW;        // queries per workgroup
constexpr int NTHREADS = 64 * NW;  // threads per workgroup
constexpr int KT = 64;             // keys per tile
constexpr int K_ELEMS = KT * 128;  // bf16 elements of one K tile (16 KB)
constexpr int V_ELEMS = 128 * KT;  // bf16 elements of one V^T tile (16 KB)
constexpr int KSTAGE0 = 0, VSTAGE0 = 2 * K_ELEMS;  // [K0 | K1 | V0 | V1], 64 KB
// A lane's weight sum per tile that forces a new shift. Weights up to 2^32
// keep every fp32 sum (at most 2^20 keys) far below overflow.
constexpr float SUM_LIMIT = 4294967296.0f;

// Wait for all of this wave's tile copies, then meet the other waves.
__device__ __forceinline__ void tile_barrier() {
  constexpr int enc = (0x7 << 4) | (0xF << 8);  // vmcnt(0)
  __builtin_amdgcn_s_waitcnt(enc);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(NTHREADS, 2) void attention_kernel(const bf16 *__restrict__ qk,
                                                                const bf16 *__restrict__ vt,
                                                                bf16 *__restrict__ o, int T,
                                                                int H, int Tp) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * K_ELEMS + 2 * V_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5, c = lane & 31;
  // Work order: the dispatcher hands workgroup i to XCD i % 8. The linear id
  // is remapped so that each XCD receives a contiguous range of (head, query
  // tile) items, head-major: the workgroups in flight on one XCD then work on
  // the same one or two heads and stream the same K and V tiles through its L2.
  const int qtiles = (int)ceil_div(T, QT);
  int h, qt;
  {
    const int n = (int)gridDim.x, bid = (int)blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3, q = n >> 3, r = n & 7;
    const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
    h = L / qtiles;
    qt = L - h * qtiles;
  }
  const int A = H * 128;
  const int ldqk = 2 * A;
  const int q0 = qt * QT + wave * 32;
  const int ntiles = (int)ceil_div(T, KT);

  // this lane's query fragments: Q[q0 + c][16 s + 8 G .. +7], s = 0..7
  bf16x8 qf[8];
  {
    const int qrow = min(q0 + c, T - 1);
    const bf16 *qp = qk + (int64_t)qrow * ldqk + h * 128 + 8 * G;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
  }

  // Tile copies: wave w fills 1 KB blocks 2w, 2w+1 of a K tile (4 rows of 256 B
  // each) and of a V^T tile (8 rows of 128 B each). Lane l lands at byte 16 l
  // of its block, so it fetches the logical chunk that the swizzle puts there.
  // Byte offsets are relative to the tile's first row (K) or the head's first
  // dim row and the tile's first key (V^T).
  const bf16 *khead = qk + A + h * 128;
  const bf16 *vhead = vt + (int64_t)h * 128 * Tp;
  int krow[2], kcol[2];
  uint32_t kofs[2], vofs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = (2 * wave + j) * 4 + (lane >> 4);  // key row within the tile
    krow[j] = kr;
    kcol[j] = ((lane & 15) ^ (kr & 15)) * 8;
    kofs[j] = (uint32_t)(kr * ldqk + kcol[j]) * 2u;
    const int vr = (2 * wave + j) * 8 + (lane >> 3);  // dim row of V^T
    vofs[j] = (uint32_t)(vr * Tp + ((lane & 7) ^ ((vr >> 1) & 7)) * 8) * 2u;
  }
  const uint32_t lds0 = lds_address(lds);
  auto kload = [&](int stage, int tile) {
    const uint32_t dst = lds0 + (uint32_t)(KSTAGE0 + stage * K_ELEMS + wave * 2 * 512) * 2u;
    const bf16 *base = khead + (int64_t)tile * KT * ldqk;
    const int rows = T - tile * KT;  // keys present in this tile
    if (rows >= KT) {
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(base, kofs[j], dst + j * 1024);
    } else {  // ragged last tile: rows past T repeat row T - 1
#pragma unroll
      for (int j = 0; j < 2; ++j)
        dma16(base, (uint32_t)(min(krow[j], rows - 1) * ldqk + kcol[j]) * 2u, dst + j * 1024);
    }
  };
  auto vload = [&](int stage, int tile) {
    const uint32_t dst = lds0 + (uint32_t)(VSTAGE0 + stage * V_ELEMS + wave * 2 * 512) * 2u;
    const bf16 *base = vhead + tile * KT;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(base, vofs[j], dst + j * 1024);
  };

  // Fragment read offsets (elements) within stage 0. The swizzles depend only
  // on the lane's row within a 16-row (K) or 32-row (V^T) group, so the other
  // key block, the other dim blocks and the other stage are immediate offsets.
  int koff[8];  // K row c, 16-byte chunk 2 s + G
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = KSTAGE0 + c * 128 + (((2 * s + G) ^ (c & 15)) * 8);
  int voff[4];  // V^T row c, 16-byte chunk 2 j + G
#pragma unroll
  for (int j = 0; j < 4; ++j) voff[j] = VSTAGE0 + c * 64 + (((2 * j + G) ^ ((c >> 1) & 7)) * 8);

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.0f;
  float m_run = 0.0f, l_run = 0.0f;
  f32x16 negm;  // -m_run in every element: the score MFMAs start from it
#pragma unroll
  for (int v = 0; v < 16; ++v) negm[v] = 0.0f;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  f32x16 sacc[2][2];  // [parity][key block]: s - m of one tile
  u32x4 pf[4];        // P^T fragments of the four k-steps of P V

  // S^T(tile) - m from K stage KS into sacc[KS]
  auto scores = [&](auto ks_c) {
    constexpr int KS = decltype(ks_c)::value;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8 *>(lds + koff[s] + b * 32 * 128 + KS * K_ELEMS);
        sacc[KS][b] = mfma32(kf, qf[s], s == 0 ? negm : sacc[KS][b]);
      }
  };

  // P = bf16(2^(sacc - dm)) straight into the P^T fragments (fragment j holds
  // registers 8 (j % 2) .. +7 of score block j / 2); returns this lane's sum
  // of its 32 weights.
  auto weights = [&](auto p_c, float dm) -> float {
    constexpr int P = decltype(p_c)::value;
    float t[2] = {0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[P][b][2 * u] - dm);
        const float p1 = __builtin_amdgcn_exp2f(sacc[P][b][2 * u + 1] - dm);
        const bf16x2 pr = pack2(p0, p1);
        pf[2 * b + (u >> 2)][u & 3] = __builtin_bit_cast(uint32_t, pr);
        t[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, t[u & 1], false);
      }
    return t[0] + t[1];
  };

  // O^T[dim][query] += V^T[dim][keys] P^T[keys][query] from V stage VS
  auto pv = [&](auto vs_c) {
    constexpr int VS = decltype(vs_c)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 pj = __builtin_bit_cast(bf16x8, pf[j]);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8 *>(lds + voff[j] + VS * V_ELEMS + db * 32 * 64);
        oacc[db] = mfma32(vf, pj, oacc[db]);
      }
    }
    // fragment reads run four MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 12; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // One tile: copies of K(it + 2) and V(it + 1), S(it + 1) (when NEXT_S)
  // overlapped with the weights of tile it, the shift check, then P V.
  auto step = [&](auto p_c, auto next_s_c, int it) {
    constexpr int P = decltype(p_c)::value;
    constexpr bool NEXT_S = decltype(next_s_c)::value;
    using KN = std::integral_constant<int, P ^ 1>;
    tile_barrier();  // V(it) and K(it + 1) are in LDS everywhere
    if (it + 2 < ntiles) kload(P, it + 2);
    if (it + 1 < ntiles) vload(P ^ 1, it + 1);

    const int kv0 = it * KT;
    if (kv0 + KT > T) {  // ragged last tile: keys past T get zero weight
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kv0 + 32 * b + 8 * (v >> 2) + 4 * G + (v & 3);
          if (key >= T) sacc[P][b][v] = -INFINITY;
        }
    }

    if constexpr (NEXT_S) scores(KN());
    float ts = weights(p_c, 0.0f);
    if constexpr (NEXT_S) {
      // score MFMAs interleaved with the weight computation, K fragment reads
      // running four MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }

    // First tile: take the shift from its maximum. Later tiles: only when the
    // weights grew past 2^32 (or overflowed).
    if (__ballot((ts > SUM_LIMIT) | (it == 0))) {
      float mx = fmaxf(sacc[P][0][0], sacc[P][1][0]);
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(sacc[P][0][v], sacc[P][1][v]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float dm = ceilf(mx);  // integer step of the shift
      if (it > 0) {
        dm = fmaxf(dm, 0.0f);
        const float fct = __builtin_amdgcn_exp2f(-dm);  // exact power of two
        l_run *= fct;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[d][v] *= fct;
      }
      m_run += dm;
#pragma unroll
      for (int v = 0; v < 16; ++v) negm[v] = -m_run;
      if constexpr (NEXT_S) {  // the next tile's scores were taken with the old shift
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[P ^ 1][b][v] -= dm;
      }
      ts = weights(p_c, dm);
    }
    l_run += ts;
    pv(p_c);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using Y = std::true_type;
  using N = std::false_type;

  // prologue: K(0), K(1), V(0) in flight; S(0) once they land
  kload(0, 0);
  if (ntiles > 1) kload(1, 1);
  vload(0, 0);
  tile_barrier();
  scores(I0());

  int it = 0;
  for (; it + 2 < ntiles; it += 2) {
    step(I0(), Y(), it);
    step(I1(), Y(), it + 1);
  }
  if (ntiles - it == 2) {
    step(I0(), Y(), it);
    step(I1(), N(), it + 1);
  } else {
    step(I0(), N(), it);
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
  dim3 grid((unsigned)(ceil_div(T, QT) * H));
  hipLaunchKernelGGL(attention_kernel, grid, dim3(NTHREADS), 0, s, static_cast<const bf16 *>(qk),
                     static_cast<const bf16 *>(vt), static_cast<bf16 *>(o), T, H, Tp);
  return hipGetLastError();
}

}  // namespace h3dit
