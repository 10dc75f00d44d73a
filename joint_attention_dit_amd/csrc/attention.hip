// Joint bidirectional attention over the packed text + image sequence
// (model card, "Model Architecture": every token sits in one packed sequence
// of a single-stream transformer; spec page: 56 query and 56 key-value heads
// of dimension 128). Flash-style: keys and values are visited in tiles of 64
// and the weights are accumulated as they are formed (one integer shift per
// row, below), so no T x T matrix is ever stored.
//
// Work split: a workgroup owns 256 queries of one head (eight waves of 32, two
// waves per SIMD). Each wave computes the transposed score tile S^T = K Q^T
// with the 16x16x32 bf16 MFMA: on random operands the chip runs into its power
// limit, and this product moves half the accumulator data per flop of the
// 32x32x16 one. Lane l = 16 g + r holds, for each of its two queries (r and
// 16 + r of the wave), the scores of keys 16 b + 4 g .. +3 of every 16-key
// block b: 16 of the tile's 64 keys; the other 48 sit in lanes l ^ 16, l ^ 32,
// l ^ 48. The output is accumulated transposed as well, O^T += V^T P^T; the
// MFMA's K slots of that product are assigned to keys in the order in which
// the score registers hold them (lane group g holds keys 4g..4g+3 and
// 16+4g..16+4g+3 of every 32), and V^T is stored in global memory in that
// order (bits 4, 3, 2 of the key index moved to bits 2, 4, 3 within each
// group of 32 keys), so each such fragment is one 16-byte read.
//
// Pipeline: after the barrier of key tile i, a wave multiplies the scores of
// tile i+1 on the matrix cores while its vector ALUs turn the scores of tile i
// into weights, then accumulates P(i) V(i). K and V^T tiles are double
// buffered in LDS and stream in through gfx950's global-to-LDS loads (K two
// tiles ahead, V one), with one barrier per tile.
//
// Softmax weights. The stored queries already carry the factor log2(e)/sqrt(128)
// (the QKV epilogue applies it before rounding q to bf16), so a score
// s = q.k is in base-2 units, and P = bf16(2^(s - m)) for an integer shift m
// per query. The score MFMAs start their accumulation from -m, so the matrix
// cores deliver s - m and each weight costs one exp2. m is not raised tile by
// tile: it is set to the first tile's rounded-up maximum plus 32, and the
// running output is never rescaled. The loop only notes (in a wave-wide flag,
// without a branch) whether some lane's sum of its 16 weights of a query in
// some tile exceeded 2^76, i.e. a score more than about 104 above the first
// tile's maximum. After the pass the workgroup then computes the exact maxima
// of its rows (a scores-only pass, K streamed through LDS) and runs the whole
// key loop a second time, its shifts raised to at least the rounded-up row
// maxima. Every weight of the kept pass is at most 2^76. On scores that rise
// along the sequence (every workgroup repeats) attention takes about 2.3x its
// ordinary time.
// Nothing in the common path touches the accumulated output outside the
// matrix cores (a rescale of it inside the loop would not fit the registers).
// Because scaling by a power of two commutes with bf16 rounding, the result
// equals that of the single shift ceil(max over all keys) (up to weights more
// than 2^94 below the largest, which may underflow): o = bf16(sum P v / sum P),
// the sum taken over the rounded weights.
//
// LDS layouts: K tile [64 keys][128 dims], 256-byte rows, 16-byte chunk c
// stored at c ^ (row & 15); V^T tile [128 dims][64 keys], 128-byte rows,
// chunk c at c ^ ((row >> 1) & 7). Both make the fragment reads conflict-free.
#include "common.h"
#include "kernels.h"
#include "mxfp8_device.h"

#include <type_traits>

namespace h3dit {

namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int QT = 32 * NW;        // queries per workgroup
constexpr int NTHREADS = 64 * NW;  // threads per workgroup
constexpr int KT = 64;             // keys per tile
constexpr int K_ELEMS = KT * 128;  // bf16 elements of one K tile (16 KB)
constexpr int V_ELEMS = 128 * KT;  // bf16 elements of one V^T tile (16 KB)
constexpr int VSTAGE0 = 2 * K_ELEMS;  // [K0 | K1 | V0 | V1], 64 KB
// one key-range piece of an item: O^T-unnormalised [256 queries][128 dims],
// the weight sums [256] and the shifts [256], fp32
constexpr int PIECE_FLOATS = QT * 130;
// The first shift lies SHIFT_BIAS above the first tile's maximum, and a
// lane's weight sum per query and tile above SUM_LIMIT forces the second pass:
// a score more than about 104 (base 2) above the first tile's maximum. The
// largest score of a row then has a weight in [2^-32, 2^76]; sums over up to
// 2^20 keys stay below 2^96, and the output accumulators neither overflow nor
// underflow for values between 2^-94 and 2^32 in size. The bias is kept small
// because the score MFMAs accumulate s - m in fp32: the nearer s - m stays to
// zero for the largest scores, the finer the argument of their exp2.
constexpr float SHIFT_BIAS = 32.0f;
constexpr float SUM_LIMIT = 75557863725914323419136.0f;  // 2^76

// Wait for all of this wave's tile copies, then meet the other waves.
__device__ __forceinline__ void tile_barrier() {
  constexpr int enc = (0x7 << 4) | (0xF << 8);  // vmcnt(0)
  __builtin_amdgcn_s_waitcnt(enc);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// With MX, o is also written as MXFP8 codes [T, A] and scales (the layout of
// mxfp8_quantize_kernel), the operand of the MXFP8 output projection.
template <bool MX>
__global__ __launch_bounds__(NTHREADS, 2) void attention_kernel(const bf16 *__restrict__ qk,
                                                                const bf16 *__restrict__ vt,
                                                                bf16 *__restrict__ o,
                                                                uint8_t *__restrict__ o_codes,
                                                                uint8_t *__restrict__ o_scales,
                                                                int T, int H, int Tp,
                                                                float *__restrict__ part,
                                                                int full, int split) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * K_ELEMS + 2 * V_ELEMS];
  __shared__ int rerun;  // some wave of the workgroup needs pass 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  if (tid == 0) rerun = 0;
  __syncthreads();
  // Work order: the dispatcher hands workgroup i to XCD i % 8. The linear id
  // is remapped so that each XCD receives a contiguous range of (head, query
  // tile) items, head-major: the workgroups in flight on one XCD then work on
  // the same one or two heads and stream the same K and V tiles through its L2.
  // With split > 1, workgroups full, full + 1, ... each take one key range
  // (piece) of the items full, full + 1, ... (the last, partial round of
  // items): piece p of an item covers key tiles [p per, min((p + 1) per, all)).
  // Their unnormalised outputs, weight sums and shifts go to `part`, and
  // attention_merge_kernel combines the pieces.
  const int qtiles = (int)ceil_div(T, QT);
  const int all_tiles = (int)ceil_div(T, KT);
  int h, qt, L, piece = -1, kt0 = 0, kt1 = all_tiles;
  {
    const int bid = (int)blockIdx.x;
    if (split <= 1 || bid < full) {
      const int n = split <= 1 ? (int)gridDim.x : full;
      const int xcd = bid & 7, idx = bid >> 3, q = n >> 3, rem = n & 7;
      L = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + idx;
    } else {
      const int u = bid - full;
      L = full + u / split;
      piece = u - (u / split) * split;
      const int per = (int)ceil_div(all_tiles, split);
      kt0 = piece * per;
      kt1 = min(kt0 + per, all_tiles);
    }
    h = L / qtiles;
    qt = L - h * qtiles;
  }
  const int A = H * 128;
  const int ldqk = 2 * A;
  const int q0 = qt * QT + wave * 32;
  const int ntiles = kt1 - kt0;  // key tiles of this workgroup; `tile` below counts from kt0

  // this lane's query fragments: Q[q0 + 16 qb + r][32 s + 8 g .. +7], s = 0..3
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = min(q0 + 16 * qb + r, T - 1);
    const bf16 *qp = qk + (int64_t)qrow * ldqk + h * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[qb][s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
  }

  // Tile copies: wave w fills 1 KB blocks 2w, 2w+1 of a K tile (4 rows of 256 B
  // each) and of a V^T tile (8 rows of 128 B each). Lane l lands at byte 16 l
  // of its block, so it fetches the logical chunk that the swizzle puts there.
  // Byte offsets are relative to the tile's first row (K) or the head's first
  // dim row and the tile's first key (V^T).
  const bf16 *khead = qk + A + h * 128;
  const bf16 *vhead = vt + (int64_t)h * 128 * Tp;
  const uint32_t lds0 = lds_address(lds);
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
  auto kload = [&](int stage, int tile) {
    const uint32_t dst = lds0 + (uint32_t)(stage * K_ELEMS + wave * 2 * 512) * 2u;
    const bf16 *base = khead + (int64_t)(kt0 + tile) * KT * ldqk;
    const int rows = T - (kt0 + tile) * KT;  // keys present in this tile
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
    const bf16 *base = vhead + (kt0 + tile) * KT;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(base, vofs[j], dst + j * 1024);
  };

  // Fragment read offsets (elements) within stage 0. The swizzles depend only
  // on the lane's row within a 16-row group, so the other key blocks, the other
  // dim blocks and the other stage are immediate offsets. K: row r, 16-byte
  // chunk (4 s + g) ^ r; V^T: row r, chunk (4 ks + g) ^ ((r >> 1) & 7) (key
  // slots 32 ks + 8 g ..).
  int koff[4], voff[2];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = r * 128 + (((4 * s + g) ^ r) * 8);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) voff[ks] = VSTAGE0 + r * 64 + (((4 * ks + g) ^ ((r >> 1) & 7)) * 8);

  f32x4 oacc[8][2];  // [dim block][query block]
  float l_run[2];
  f32x4 negm[2];  // -m (the shift) of each query block in every element: the score MFMAs start from it
  float mrow[2] = {-INFINITY, -INFINITY};  // rounded-up row maxima (pass 1 of a flagged wave)
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  f32x4 sacc[2][4][2];  // [parity][key block][query block]: s - m of one tile
  u32x4 pf[2][2];       // P^T fragments [32-key slab][query block] of P V

  // S^T(tile) - m from K stage KS into sacc[D]
  auto scores = [&](auto ks_c, auto d_c) {
    constexpr int KS = decltype(ks_c)::value, D = decltype(d_c)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8 *>(lds + KS * K_ELEMS + koff[s] + b * 16 * 128);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[D][b][qb] = mfma16(kf, qf[qb][s], s == 0 ? negm[qb] : sacc[D][b][qb]);
      }
  };

  // keys past T of tile `tile` get zero weight
  auto mask = [&](auto d_c, int tile) {
    constexpr int D = decltype(d_c)::value;
    const int kv0 = (kt0 + tile) * KT;
    if (kv0 + KT > T) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (kv0 + 16 * b + 4 * g + v >= T) sacc[D][b][qb][v] = -INFINITY;
    }
  };

  // Largest score of each query in sacc[D] (over the whole tile: xor 16, 32
  // reach the other three lanes of the query), rounded up.
  auto tile_max = [&](auto d_c, int qb) -> float {
    constexpr int D = decltype(d_c)::value;
    float mx = sacc[D][0][qb][0];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sacc[D][b][qb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    return ceilf(mx);
  };

  // P = bf16(2^sacc[P]) straight into the P^T fragments (fragment [ks][qb]
  // holds key blocks 2 ks and 2 ks + 1 of query block qb); t[qb] receives this
  // lane's sum of its 16 weights of query block qb.
  auto weights = [&](auto p_c, float t[2]) {
    constexpr int P = decltype(p_c)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float tq[2] = {0.0f, 0.0f};
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[P][b][qb][2 * u]);
          const float p1 = __builtin_amdgcn_exp2f(sacc[P][b][qb][2 * u + 1]);
          const bf16x2 pr = pack2(p0, p1);
          pf[b >> 1][qb][2 * (b & 1) + u] = __builtin_bit_cast(uint32_t, pr);
          tq[u] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, tq[u], false);
        }
      t[qb] = tq[0] + tq[1];
    }
  };

  // O^T[dim][query] += V^T[dim][keys] P^T[keys][query] from V stage VS
  auto pv = [&](auto vs_c) {
    constexpr int VS = decltype(vs_c)::value;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8 *>(lds + voff[ks] + VS * V_ELEMS + db * 16 * 64);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = mfma16(vf, __builtin_bit_cast(bf16x8, pf[ks][qb]), oacc[db][qb]);
      }
    // fragment reads run four reads (eight MFMAs) ahead of their use, two
    // reads after every four products
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // One tile (stages P = it % 2): copies of K(it + 2) into the K stage of
  // tile it (its scores were multiplied in the previous step) and of V(it + 1)
  // into the V stage of tile it - 1 (last read before this barrier), S(it + 1)
  // (when NEXT_S) overlapped with the weights of tile it, the shift check,
  // then P V.
  auto step = [&](auto p_c, auto next_s_c, int it, bool &again) {
    constexpr int P = decltype(p_c)::value;
    constexpr bool NEXT_S = decltype(next_s_c)::value;
    using DC = std::integral_constant<int, P>;
    using DN = std::integral_constant<int, P ^ 1>;
    tile_barrier();  // V(it) and K(it + 1) are in LDS everywhere
    if (it + 2 < ntiles) kload(P, it + 2);
    if (it + 1 < ntiles) vload(P ^ 1, it + 1);

    mask(DC(), it);
    if constexpr (NEXT_S) scores(DN(), DN());
    float ts[2];
    weights(p_c, ts);
    if constexpr (NEXT_S) {
      // score MFMAs interleaved with the weight computation, three and then
      // two vector instructions after each product; K fragment reads run four
      // ahead. The scheduler's vector class (0x002) leaves out transcendental
      // instructions: the pattern places the packing and summing, and the
      // scheduler puts the exp2s among the first products itself. Placing the
      // exp2s too (class 0x400) ran at the same speed; one vector instruction
      // after each of the tile's 64 products ran 5 % slower.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }

    // Weights grew past 2^76 (or overflowed): the row maxima are found after
    // this pass and the pass is run again (rare; no branch here).
    again |= __ballot((ts[0] > SUM_LIMIT) | (ts[1] > SUM_LIMIT)) != 0;
    l_run[0] += ts[0];
    l_run[1] += ts[1];
    pv(p_c);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using Y = std::true_type;
  using N = std::false_type;

  // Pass 0 takes the shift from the first tile's maximum (plus SHIFT_BIAS).
  // If some tile's weights outgrow 2^76, the wave finds the exact maxima of
  // its rows and pass 1 runs the whole key loop again with the shift at
  // least ceil(row maximum): no weight exceeds 1 and nothing fires.
  for (int pass = 0;; ++pass) {
    bool again = false;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int v = 0; v < 4; ++v) oacc[d][qb][v] = 0.0f;
    l_run[0] = l_run[1] = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int v = 0; v < 4; ++v) negm[qb][v] = 0.0f;

    // prologue: K(0), K(1), V(0) in flight; S(0) once they land, and the
    // shift from its maximum
    kload(0, 0);
    if (ntiles > 1) kload(1, 1);
    vload(0, 0);
    tile_barrier();
    scores(I0(), I0());
    mask(I0(), 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m = fmaxf(tile_max(I0(), qb) + SHIFT_BIAS, mrow[qb]);
#pragma unroll
      for (int v = 0; v < 4; ++v) negm[qb][v] = -m;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) sacc[0][b][qb][v] -= m;
    }

    int it = 0;
    for (; it + 2 < ntiles; it += 2) {
      step(I0(), Y(), it, again);
      step(I1(), Y(), it + 1, again);
    }
    if (ntiles - it == 2) {
      step(I0(), Y(), it, again);
      step(I1(), N(), it + 1, again);
    } else {
      step(I0(), N(), it, again);
    }
    if (pass == 1) break;
    // the workgroup runs pass 1 if any of its waves needs it (every wave
    // takes part in the tile copies and barriers)
    if (again && lane == 0) rerun = 1;
    __syncthreads();
    if (!rerun) break;
    // Exact row maxima of every wave's queries for pass 1: a scores-only pass
    // over the key tiles, streamed through the two K stages of LDS like the
    // main loop (each tile copied once per workgroup; no weights, no P V).
    // At the barrier of tile t, K(t) has landed and every wave is done with
    // tile t - 1, whose stage then takes K(t + 1).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int v = 0; v < 4; ++v) negm[qb][v] = 0.0f;
    kload(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      tile_barrier();
      if (t + 1 < ntiles) kload((t + 1) & 1, t + 1);
      if (t & 1)
        scores(I1(), I0());
      else
        scores(I0(), I0());
      mask(I0(), t);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) mrow[qb] = fmaxf(mrow[qb], tile_max(I0(), qb));
    }
    __syncthreads();  // every wave is done with the K stages before pass 1 refills them
  }

  if (piece >= 0) {  // unnormalised output, weight sum and shift of each query row
    float *pp = part + ((int64_t)(L - full) * split + piece) * PIECE_FLOATS;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const int ql = wave * 32 + 16 * qb + r;  // query row within the item
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<f32x4 *>(pp + ql * 128 + 16 * db + 4 * g) = oacc[db][qb];
      if (g == 0) {
        pp[QT * 128 + ql] = l_tot;
        pp[QT * 129 + ql] = -negm[qb][0];
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const float inv_l = 1.0f / l_tot;  // one division per row, 64 products
    const int q = q0 + 16 * qb + r;
    bf16x4 rv[8];  // dims 16 db + 4 g .. +3 of query q
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) rv[db][e] = to_bf16(oacc[db][qb][e] * inv_l);
    if (q < T && (!MX || o)) {  // with MX, o may be left out (only its codes consumed)
      bf16 *op = o + (int64_t)q * A + h * 128 + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) *reinterpret_cast<bf16x4 *>(op + db * 16) = rv[db];
    }
    if constexpr (MX) {
      // MX block j = dims 32 j .. 32 j + 31 of the head: dim blocks 2 j and
      // 2 j + 1 of the four lanes l ^ 16, l ^ 32 that hold query q
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 w0 = __builtin_bit_cast(u32x2, rv[2 * j]);
        const u32x2 w1 = __builtin_bit_cast(u32x2, rv[2 * j + 1]);
        uint32_t amax = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          amax = max(amax, max(w0[e] & 0x7FFFu, (w0[e] >> 16) & 0x7FFFu));
          amax = max(amax, max(w1[e] & 0x7FFFu, (w1[e] >> 16) & 0x7FFFu));
        }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16, 64));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32, 64));
        const int sbyte = mx_scale_byte(amax);
        const float inv = mx_inv_scale(sbyte);
        if (q < T) {
          uint8_t *cp = o_codes + (int64_t)q * A + h * 128 + 32 * j + 4 * g;
          *reinterpret_cast<uint32_t *>(cp) =
              mx_code4(mx_bf16_value(w0[0] & 0xFFFFu), mx_bf16_value(w0[0] >> 16),
                       mx_bf16_value(w0[1] & 0xFFFFu), mx_bf16_value(w0[1] >> 16), inv);
          *reinterpret_cast<uint32_t *>(cp + 16) =
              mx_code4(mx_bf16_value(w1[0] & 0xFFFFu), mx_bf16_value(w1[0] >> 16),
                       mx_bf16_value(w1[1] & 0xFFFFu), mx_bf16_value(w1[1] >> 16), inv);
        }
        // rows past T of the last 256-row panel get scale byte 0
        if (g == 0) o_scales[mx_scale_offset(q, 4 * h + j, A)] = (uint8_t)(q < T ? sbyte : 0);
      }
    }
  }
}

}  // namespace

// Sum of the key-range pieces of split item full + blockIdx.x: with M the
// largest of the pieces' shifts, O = sum_p O_p 2^(m_p - M) and
// l = sum_p l_p 2^(m_p - M) (power-of-two scalings, exact in fp32), then
// o = bf16(O * (1 / l)) as in the unsplit kernel. Because a power-of-two
// scaling commutes with the bf16 rounding of the weights, this equals the
// single-shift result up to the fp32 summation order. Workgroup (x, y) takes
// query rows 64 y .. 64 y + 63 of the item (four workgroups per item, so that
// enough waves are in flight); thread u handles dims 8 c .. 8 c + 7 of query
// row ql.
__global__ __launch_bounds__(256) void attention_merge_kernel(const float *__restrict__ part,
                                                              bf16 *__restrict__ o, int T, int H,
                                                              int full, int split) {
  const int L = full + (int)blockIdx.x;
  const int qtiles = (int)ceil_div(T, QT);
  const int h = L / qtiles, qt = L - h * qtiles;
  const float *base = part + (int64_t)blockIdx.x * split * PIECE_FLOATS;
  const int A = H * 128;
  for (int u = (int)blockIdx.y * 64 * 16 + threadIdx.x; u < ((int)blockIdx.y + 1) * 64 * 16;
       u += 256) {
    const int ql = u >> 4, c = u & 15;
    const int q = qt * QT + ql;
    if (q >= T) continue;
    float M = -INFINITY;
    for (int p = 0; p < split; ++p) M = fmaxf(M, base[p * PIECE_FLOATS + QT * 129 + ql]);
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    float l = 0.0f;
    for (int p = 0; p < split; ++p) {
      const float *pp = base + p * PIECE_FLOATS;
      const float sc = ldexpf(1.0f, (int)(pp[QT * 129 + ql] - M));
      const f32x4 v0 = *reinterpret_cast<const f32x4 *>(pp + ql * 128 + 8 * c);
      const f32x4 v1 = *reinterpret_cast<const f32x4 *>(pp + ql * 128 + 8 * c + 4);
      a0 += v0 * sc;
      a1 += v1 * sc;
      l += pp[QT * 128 + ql] * sc;
    }
    const float inv_l = 1.0f / l;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = to_bf16(a0[e] * inv_l);
      out[4 + e] = to_bf16(a1[e] * inv_l);
    }
    *reinterpret_cast<bf16x8 *>(o + (int64_t)q * A + h * 128 + 8 * c) = out;
  }
}

// Whole items first, then the last, partial round of items cut along the keys
// into `split` pieces when that shortens it enough to pay for the pieces'
// partial sums: cut into s, the rem items of the last round take
// ceil(rem s / cus) rounds of 1/s of an item, and merging moves 266 KB per
// piece through memory after the kernel (at about 5 TB/s, against an item's
// time of about 26 ns per key: rem s 2.06 / T rounds); s = 1 unless the cut
// saves a tenth of a round. (4096x4096 block: 112 items left, two pieces:
// 0.53 instead of 1 round; 2048x2048: 184 left, no cut pays.)
static int attention_split_plan(int T, int H, int *full, int *pieces_per_item) {
  constexpr int cus = 256;  // MI355X compute units; one workgroup per CU
  const int items = (int)ceil_div(T, QT) * H;
  const int all_tiles = (int)ceil_div(T, KT);
  const int rem = items % cus;
  *full = items;
  *pieces_per_item = 1;
  if (rem == 0 || items < cus) return items;
  double best = 1.0;
  int bs = 1;
  for (int sl = 2; sl <= 4 && 2 * sl <= all_tiles; ++sl) {
    const double c = (double)ceil_div((int64_t)rem * sl, cus) / sl + (double)rem * sl * 2.06 / T;
    if (c < best - 0.1) {
      best = c;
      bs = sl;
    }
  }
  if (bs == 1) return items;
  const int per = (int)ceil_div(all_tiles, bs);
  bs = (int)ceil_div(all_tiles, per);  // every piece non-empty
  *full = items - rem;
  *pieces_per_item = bs;
  return *full + rem * bs;
}

size_t attention_split_scratch_bytes(int T, int H) {
  int full = 0, sl = 1;
  attention_split_plan(T, H, &full, &sl);
  const int items = (int)ceil_div(T, QT) * H;
  return sl > 1 ? (size_t)(items - full) * sl * PIECE_FLOATS * sizeof(float) : 0;
}

hipError_t launch_attention(const void *qk, const void *vt, void *o, int T, int H, int Tp,
                            hipStream_t s, float *part, size_t part_bytes) {
  int full = 0, sl = 1;
  int grid = attention_split_plan(T, H, &full, &sl);
  const int items = (int)ceil_div(T, QT) * H;
  if (sl > 1 && (!part || part_bytes < (size_t)(items - full) * sl * PIECE_FLOATS * sizeof(float))) {
    sl = 1;  // no scratch for the pieces: whole items only
    full = items;
    grid = items;
  }
  hipLaunchKernelGGL(attention_kernel<false>, dim3((unsigned)grid), dim3(NTHREADS), 0, s,
                     static_cast<const bf16 *>(qk), static_cast<const bf16 *>(vt),
                     static_cast<bf16 *>(o), nullptr, nullptr, T, H, Tp, part, full, sl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sl <= 1) return e;
  hipLaunchKernelGGL(attention_merge_kernel, dim3((unsigned)(items - full), QT / 64), dim3(256), 0, s,
                     part, static_cast<bf16 *>(o), T, H, full, sl);
  return hipGetLastError();
}

hipError_t launch_attention_mx(const void *qk, const void *vt, void *o, uint8_t *o_codes,
                               uint8_t *o_scales, int T, int H, int Tp, hipStream_t s) {
  dim3 grid((unsigned)(ceil_div(T, QT) * H));
  hipLaunchKernelGGL(attention_kernel<true>, grid, dim3(NTHREADS), 0, s,
                     static_cast<const bf16 *>(qk), static_cast<const bf16 *>(vt),
                     static_cast<bf16 *>(o), o_codes, o_scales, T, H, Tp, nullptr, 0, 1);
  return hipGetLastError();
}

}  // namespace h3dit
