// bf16 matrix-core GEMM with fused epilogues for the DiT block's linears
// (QKV, output projection, MLP up, MLP down; model card, "Model
// Architecture", and the spec page's block diagram).
//
//   C[t, n] = sum_k X[t, k] * W[n, k]      X: activations [M, K], W: weights [N, K]
//
// Both operands are K-contiguous, so both feed the 16x16x32 bf16 MFMA
// directly. The weight rows are the MFMA "A" rows and the token rows the
// "B" columns, which leaves every lane holding four consecutive output
// features of one token: RoPE pairs (2i, 2i+1) sit in one lane and stores are
// 8- or 16-byte vectors.
//
// Tiling: 256 features x 256 tokens per workgroup, K step 64 (two MFMA
// k-steps of 32), eight waves (two per SIMD) in a 2 x 4 arrangement, each
// owning 128 features x 64 tokens (8 x 4 blocks of 16 x 16, 128 fp32
// accumulators per lane). The 16x16x32 product is used rather than 32x32x16:
// on random operands the chip runs into its power limit, and the smaller
// product (half the accumulator traffic per flop) sustains about a quarter
// more throughput there. With two waves per SIMD one wave's matrix cores keep
// running while the other waits at the barrier or issues its copies.
// Global tiles go straight into LDS (gfx950's 16-byte global-load-to-LDS).
// Every tile row is one 128-byte segment of a K-contiguous matrix row: copies
// of 64-byte segments reach only about half the global-to-LDS rate per CU that
// this tile needs. The weight tile has two LDS stages and the activation tile
// three (5 x 32 KB = 160 KB): activation panels are shared by fewer concurrent
// workgroups than weight panels, miss L2 more often and so get copies issued
// two K steps ahead instead of one. One barrier per K step, after the first
// products of the second k-step: by then every wave has read its last
// fragments of the current tile (so its stages take weight tile kt + 2 and
// activation tile kt + 3, copied right after the barrier) and the next tile
// has landed (so its first fragments are read during the second k-step). A
// fragments are re-read in place as soon as their four products have issued,
// B fragments are double buffered. LDS rows are 128 bytes; 16-byte chunk c of
// row r is stored at chunk c ^ ((r >> 1) & 7), so the 16 rows read by a
// quarter-wave fragment load cover all 64 banks.
//
// Workgroup order: the dispatcher hands workgroup i to XCD i % 8. The
// linear id is remapped so that each XCD receives a contiguous range of
// tiles, and tiles are walked in groups of 8 token tiles so that the tiles
// in flight on one XCD share weight and activation panels in its L2.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace h3dit {

namespace {

constexpr int BN = 256;   // weight rows (output features) per tile
constexpr int BT = 256;   // activation rows (tokens) per tile
constexpr int BK = 64;    // K per LDS stage (128-byte rows)
constexpr int TILE_ELEMS = 256 * BK;  // one operand tile, bf16 elements (32 KB)
constexpr int GROUP_T = 8;

// LDS rows are 128 bytes (8 chunks of 16 B); 2 rows share one 256-byte bank line,
// so chunk c of row r is stored at chunk c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Tile L of the grouped walk: GROUP_T token tiles per group, features outer
// within the group.
__device__ __forceinline__ void walk_coords(int L, int tiles_n, int tiles_t, int &tn, int &tt) {
  const int per_group = GROUP_T * tiles_n;
  const int g = L / per_group;
  const int first_t = g * GROUP_T;
  const int gt = min(tiles_t - first_t, GROUP_T);
  const int in = L - g * per_group;
  tt = first_t + in % gt;
  tn = in / gt;
}

__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_n, int tiles_t,
                                            int &tn, int &tt) {
  // XCD-contiguous remap (bijective for any nblocks)
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
  walk_coords(L, tiles_n, tiles_t, tn, tt);
}

// Split tiles: K slices of one tile are workgroups full_tiles + t * split + s;
// slice s covers K tiles [s * per, min((s + 1) * per, ktiles)).
__device__ __forceinline__ int slice_ktiles(int ktiles, int split) {
  return (ktiles + split - 1) / split;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  // 0.5 z (1 + tanh(y)) == z / (1 + exp(-2y)),  y = sqrt(2/pi) (z + 0.044715 z^3)
  const float y = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  return z / (1.0f + expf(-2.0f * y));
}

// q or k: rotate the two adjacent pairs of the fp32 products, then round once;
// q also takes the softmax factor log2(e)/sqrt(128) before its rounding, so that
// attention scores leave the matrix cores in base-2 units.
__device__ __forceinline__ bf16x4 qk_rope4(const GemmArgs &a, int t, int n, float v0, float v1,
                                           float v2, float v3) {
  const float u0 = v0, w0 = v1, u1 = v2, w1 = v3;
  const int p = (n & 127) >> 1;  // pair index within the head (0..63)
  const f32x4 cs = *reinterpret_cast<const f32x4 *>(a.table + ((int64_t)t * 64 + p) * 2);
  const float sc = n < a.A ? kLog2eOverSqrt128 : 1.0f;
  bf16x4 r;
  r[0] = to_bf16((u0 * cs[0] - w0 * cs[1]) * sc);
  r[1] = to_bf16((u0 * cs[1] + w0 * cs[0]) * sc);
  r[2] = to_bf16((u1 * cs[2] - w1 * cs[3]) * sc);
  r[3] = to_bf16((u1 * cs[3] + w1 * cs[2]) * sc);
  return r;
}

__device__ __forceinline__ bf16x4 gelu4(float v0, float v1, float v2, float v3) {
  bf16x4 r;
  r[0] = to_bf16(gelu_tanh(v0));
  r[1] = to_bf16(gelu_tanh(v1));
  r[2] = to_bf16(gelu_tanh(v2));
  r[3] = to_bf16(gelu_tanh(v3));
  return r;
}

// token t of a V tile is stored at column t with bits 2 and 3 exchanged (the key
// order of the attention kernel's P V fragments)
__device__ __forceinline__ int vt_col(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Four consecutive outputs (features n .. n+3 of token t) through the epilogue.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs &a, int t, int n, float v0, float v1,
                                       float v2, float v3) {
  if (n >= a.N) return;
  if constexpr (EPI == EPI_QKV_ROPE) {
    const int A2 = 2 * a.A;
    if (n < A2) {
      if (t >= a.M) return;
      *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(a.out) + (int64_t)t * A2 + n) =
          qk_rope4(a, t, n, v0, v1, v2, v3);
    } else {
      if (t >= a.Mp) return;
      const int hv = n - A2;  // head * 128 + dim
      const int col = vt_col(t);
      bf16 *vt = static_cast<bf16 *>(a.out2) + (int64_t)hv * a.Mp + col;
      const bool live = t < a.M;
      vt[0] = to_bf16(live ? v0 : 0.0f);
      vt[a.Mp] = to_bf16(live ? v1 : 0.0f);
      vt[2 * (int64_t)a.Mp] = to_bf16(live ? v2 : 0.0f);
      vt[3 * (int64_t)a.Mp] = to_bf16(live ? v3 : 0.0f);
    }
  } else if constexpr (EPI == EPI_RESID_BF16 || EPI == EPI_RESID_F32) {
    if (t >= a.M) return;
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
    if (t >= a.M) return;
    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (int64_t)t * a.N + n) =
        f32x4{v0, v1, v2, v3};
  } else {  // EPI_GELU
    if (t >= a.M) return;
    *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(a.out) + (int64_t)t * a.N + n) =
        gelu4(v0, v1, v2, v3);
  }
}

// bf16 staging of a 256 x 256 output tile in LDS (element offset): 16-byte chunk
// c of row r sits at chunk c ^ (2 (r & 15)), so the 16 rows written by a fragment
// block and the whole rows read back both spread over all banks.
__device__ __forceinline__ int stage_off(int row, int col) {
  return row * 256 + ((((col >> 3) ^ ((row & 15) << 1))) << 3) + (col & 7);
}

// bf16 epilogue through LDS: the wave's results go to the staged tile (tokens x
// features for q/k; features x tokens, columns in the attention's key order, for
// V), then every thread stores whole 16-byte chunks of rows, so each store
// instruction writes two contiguous 512-byte rows (instead of 2-byte scattered
// stores for V). Used for the QKV epilogue (about 1.5 % faster there); the
// GELU epilogue's direct 8-byte stores are as fast.
template <int EPI>
__device__ __forceinline__ void staged_bf16_epilogue(const GemmArgs &a, bf16 *lds, const f32x4 (&acc)[8][4],
                                                     int n0, int t0, int wn, int wt, int r16, int kq) {
  const int tid = threadIdx.x;
  bool vtile = false;
  if constexpr (EPI == EPI_QKV_ROPE) vtile = n0 >= 2 * a.A;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tl = wt * 64 + 16 * j + r16, fl = wn * 128 + 16 * i + 4 * kq;
      const int t = t0 + tl, n = n0 + fl;
      const f32x4 v = acc[i][j];
      if constexpr (EPI == EPI_QKV_ROPE) {
        if (vtile) {
          const bool live = t < a.M;
          const int col = vt_col(tl);
#pragma unroll
          for (int e = 0; e < 4; ++e) lds[stage_off(fl + e, col)] = to_bf16(live ? v[e] : 0.0f);
          continue;
        }
        const bf16x4 r = t < a.M ? qk_rope4(a, t, n, v[0], v[1], v[2], v[3]) : bf16x4{};
        *reinterpret_cast<bf16x4 *>(lds + stage_off(tl, fl)) = r;
      } else {
        *reinterpret_cast<bf16x4 *>(lds + stage_off(tl, fl)) = gelu4(v[0], v[1], v[2], v[3]);
      }
    }
  __syncthreads();
#pragma unroll 4
  for (int q = tid; q < 256 * 32; q += 512) {
    const int row = q >> 5, c = q & 31;
    const bf16x8 val = *reinterpret_cast<const bf16x8 *>(lds + stage_off(row, 8 * c));
    if (vtile) {  // row = feature of the V tile, 8 tokens per chunk
      const int hv = n0 - 2 * a.A + row, t = t0 + 8 * c;
      if (hv < a.A && t < a.Mp)
        *reinterpret_cast<bf16x8 *>(static_cast<bf16 *>(a.out2) + (int64_t)hv * a.Mp + t) = val;
    } else {  // row = token, 8 features per chunk
      const int t = t0 + row, n = n0 + 8 * c;
      const int ld = EPI == EPI_QKV_ROPE ? 2 * a.A : a.N;
      const int nend = EPI == EPI_QKV_ROPE ? 2 * a.A : a.N;
      if (t < a.M && n < nend)
        *reinterpret_cast<bf16x8 *>(static_cast<bf16 *>(a.out) + (int64_t)t * ld + n) = val;
    }
  }
}

// Wait until at most N of this wave's global-to-LDS copies are still in
// flight (they complete in issue order), then meet the other waves: afterwards
// every wave's earlier copies have landed in LDS. Instructions are not moved
// across it in either direction.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  // s_waitcnt vmcnt(N) (lgkmcnt and expcnt fields left at their maximum)
  constexpr int enc = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(enc);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GemmArgs a) {
  // weight tiles: 2 stages of 32 KB; activation tiles: 3 stages of 32 KB (160 KB)
  __shared__ __attribute__((aligned(1024))) bf16 lds[5 * TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;  // 2 x 4 waves of 128 features x 64 tokens
  const int tiles_n = (int)ceil_div(a.N, BN), tiles_t = (int)ceil_div(a.M, BT);
  // whole tile, or K slice `piece` of one of the split tiles of the last wave
  int tn, tt, piece = -1, kb0 = 0, ktiles = a.K / BK;
  if (a.split <= 1) {
    tile_coords(blockIdx.x, gridDim.x, tiles_n, tiles_t, tn, tt);
  } else if ((int)blockIdx.x < a.full_tiles) {
    tile_coords(blockIdx.x, a.full_tiles, tiles_n, tiles_t, tn, tt);
  } else {
    piece = (int)blockIdx.x - a.full_tiles;
    walk_coords(a.full_tiles + piece / a.split, tiles_n, tiles_t, tn, tt);
    const int per = slice_ktiles(ktiles, a.split);
    kb0 = (piece % a.split) * per;
    ktiles = min(per, ktiles - kb0);
  }
  const int n0 = tn * BN, t0 = tt * BT;

  // global -> LDS without registers: each wave fills 4 blocks of 1 KB (8 rows of
  // 128 bytes) per operand tile; lane l lands at byte 16 l of its block, i.e. at
  // row 8 b + l / 8, physical chunk l % 8, so it fetches logical chunk
  // (l % 8) ^ swz(row). Rows past the matrix edge repeat the last row.
  const char *wpanel = static_cast<const char *>(a.w) + ((int64_t)n0 * a.K + kb0 * BK) * 2;
  const char *xpanel = static_cast<const char *>(a.x) + ((int64_t)t0 * a.K + kb0 * BK) * 2;
  uint32_t woff[4], xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 8 + (lane >> 3);
    const int lc = swz(row, lane & 7);
    woff[j] = (uint32_t)(min(n0 + row, a.N - 1) - n0) * (uint32_t)a.K * 2u + lc * 16u;
    xoff[j] = (uint32_t)(min(t0 + row, a.M - 1) - t0) * (uint32_t)a.K * 2u + lc * 16u;
  }
  const uint32_t lds0 = lds_address(lds);
  // copies j0 .. j1-1 of the weight (activation) tile at k0 into weight stage
  // wst (activation stage xst)
  auto wload = [&](int wst, int k0, int j0, int j1) {
    const char *wp = wpanel + (int64_t)k0 * 2;
    const uint32_t sw = lds0 + (uint32_t)(wst * TILE_ELEMS + wave * 4 * 512) * 2u;
#pragma unroll
    for (int j = j0; j < j1; ++j) dma16(wp, woff[j], sw + j * 1024);
  };
  auto xload = [&](int xst, int k0, int j0, int j1) {
    const char *xp = xpanel + (int64_t)k0 * 2;
    const uint32_t sx = lds0 + (uint32_t)((2 + xst) * TILE_ELEMS + wave * 4 * 512) * 2u;
#pragma unroll
    for (int j = j0; j < j1; ++j) dma16(xp, xoff[j], sx + j * 1024);
  };

  // fragment reads: lane row r16 of each 16-row block, k chunk 4 s + kq of the
  // K tile (k-step s of 32); the swizzle depends on r16 only, so block b sits at
  // a fixed offset of b * 16 rows
  const int r16 = lane & 15, kq = lane >> 4;
  int fa_base[2], fb_base[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    fa_base[s] = (wn * 128 + r16) * BK + (swz(r16, 4 * s + kq) * 8);
    fb_base[s] = (wt * 64 + r16) * BK + (swz(r16, 4 * s + kq) * 8);
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // A fragments are re-read in place once their four products have issued; B
  // fragments are double buffered
  bf16x8 fa[8], fb[2][4];
  auto fload_all = [&](int wst, int xst, int s, int buf) {
    const bf16 *sw = lds + wst * TILE_ELEMS;
    const bf16 *sx = lds + (2 + xst) * TILE_ELEMS;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = *reinterpret_cast<const bf16x8 *>(sx + fb_base[s] + j * 16 * BK);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[i] = *reinterpret_cast<const bf16x8 *>(sw + fa_base[s] + i * 16 * BK);
  };
  // One k-step (32 of K) of 32 products on B buffer BCUR; the fragments of
  // k-step ns of weight stage wst_n and activation stage xst_n are fetched
  // meanwhile. When SYNC, the wave first settles its fragment reads, then
  // meets the others after its first 4 products (waiting for its own copies of
  // tile kt + 1; with vm4 the last four copies, activation tile kt + 2, may
  // still be in flight) and afterwards issues the copies of weight tile kt + 2
  // (wref) and activation tile kt + 3 (xref). With RT the three flags are
  // taken at run time, otherwise all of them hold.
  auto kstep = [&](auto bcur_c, auto sync_c, auto rt_c, bool wref, bool xref, bool vm4, int wst_n,
                   int xst_n, int ns, int kt, int xs) {
    constexpr int BCUR = decltype(bcur_c)::value;
    constexpr bool SYNC = decltype(sync_c)::value, RT = decltype(rt_c)::value;
    const bf16 *sw = lds + wst_n * TILE_ELEMS;
    const bf16 *sx = lds + (2 + xst_n) * TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[BCUR][j], acc[i][j]);
      if constexpr (SYNC) {
        if (i == 0) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
          if (!RT || vm4) tile_barrier<4>();
          else tile_barrier<0>();
        }
        if (i == 1 && (!RT || wref)) wload(kt & 1, (kt + 2) * BK, 0, 2);
        if (i == 2 && (!RT || wref)) wload(kt & 1, (kt + 2) * BK, 2, 4);
        if (i == 3 && (!RT || xref)) xload(xs, (kt + 3) * BK, 0, 2);
        if (i == 4 && (!RT || xref)) xload(xs, (kt + 3) * BK, 2, 4);
      }
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fb[BCUR ^ 1][j] = *reinterpret_cast<const bf16x8 *>(sx + fb_base[ns] + j * 16 * BK);
      }
      fa[i] = *reinterpret_cast<const bf16x8 *>(sw + fa_base[ns] + i * 16 * BK);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using Y = std::true_type;
  using N = std::false_type;

  // K step kt: weight tile kt in stage kt & 1, activation tile kt in stage
  // xs = kt % 3. The copies of each K step are issued in the order weight tile
  // kt + 2, activation tile kt + 3, so at the barrier of K step kt + 1 exactly
  // the four copies of activation tile kt + 3 are younger than everything tile
  // kt + 2 needs. The last K step still reads (stale) fragments of the next
  // stages and meets the other waves once more, which is harmless.
  auto ktile = [&](auto rt_c, int kt, int xs) {
    const int xn = xs == 2 ? 0 : xs + 1;
    kstep(I0(), N(), rt_c, false, false, false, kt & 1, xs, 1, kt, xs);
    kstep(I1(), Y(), rt_c, kt + 2 < ktiles, kt + 3 < ktiles, kt + 2 < ktiles, (kt + 1) & 1, xn, 0,
          kt, xs);
  };

  wload(0, 0, 0, 4);
  xload(0, 0, 0, 4);
  if (ktiles > 1) {
    wload(1, BK, 0, 4);
    xload(1, BK, 0, 4);
  }
  if (ktiles > 2) {
    xload(2, 2 * BK, 0, 4);
    tile_barrier<12>();
  } else if (ktiles > 1) {
    tile_barrier<8>();
  } else {
    tile_barrier<0>();
  }
  fload_all(0, 0, 0, 0);
  // settle the scalar loads once (pending ones would make the compiler wait for
  // all LDS reads at each k-step); copies stay in flight
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  ktile(Y(), 0, 0);
  int kt = 1, xs = 1;
  for (; kt + 3 < ktiles; ++kt) {
    ktile(N(), kt, xs);
    xs = xs == 2 ? 0 : xs + 1;
  }
  for (; kt < ktiles; ++kt) {
    ktile(Y(), kt, xs);
    xs = xs == 2 ? 0 : xs + 1;
  }

  if (piece >= 0) {  // a K slice: raw sums to the scratch, [register block][thread]
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.partial) + (int64_t)piece * (32 * 512) + tid;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(i * 4 + j) * 512] = acc[i][j];
    return;
  }
  if constexpr (EPI == EPI_QKV_ROPE) {
    // every copy has landed and every wave has read its last fragments
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    staged_bf16_epilogue<EPI>(a, lds, acc, n0, t0, wn, wt, r16, kq);
    return;
  }
  const int nb = n0 + wn * 128 + 4 * kq, tb = t0 + wt * 64 + r16;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      store4<EPI>(a, tb + 16 * j, nb + 16 * i, acc[i][j][0], acc[i][j][1], acc[i][j][2],
                  acc[i][j][3]);
}

// Sum of the K slices of split tile full_tiles + blockIdx.x (in slice order),
// then the epilogue, with the thread -> output mapping of gemm_kernel;
// workgroup blockIdx.y takes feature blocks 2 y and 2 y + 1 of every wave.
template <int EPI>
__global__ __launch_bounds__(512) void gemm_fixup_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wt = wave >> 1;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tiles_n = (int)ceil_div(a.N, BN), tiles_t = (int)ceil_div(a.M, BT);
  int tn, tt;
  walk_coords(a.full_tiles + blockIdx.x, tiles_n, tiles_t, tn, tt);
  const f32x4 *src =
      reinterpret_cast<const f32x4 *>(a.partial) + (int64_t)blockIdx.x * a.split * (32 * 512) + tid;
  const int nb = tn * BN + wn * 128 + 4 * kq, tb = tt * BT + wt * 64 + r16;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * (int)blockIdx.y + ii;
      const int64_t o = (i * 4 + j) * 512;
      f32x4 v = src[o];
      for (int sl = 1; sl < a.split; ++sl) v += src[(int64_t)sl * (32 * 512) + o];
      store4<EPI>(a, tb + 16 * j, nb + 16 * i, v[0], v[1], v[2], v[3]);
    }
}

}  // namespace

// Compute units of the current device (cached per device).
constexpr int kPlanCus = 256;  // MI355X; scratch is sized for it, larger devices split less
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// One workgroup per CU at a time: when the last wave of tiles is at most half
// full, its tiles are split along K into as many slices as fill the CUs (and
// fit the scratch); a second kernel adds the slices. Returns the number of
// slices per split tile (1: no split) and the number of split tiles.
static int plan_split(int64_t M, int64_t N, int64_t K, int cus, size_t scratch_bytes, int *rem_out) {
  const int tiles = (int)(ceil_div(N, BN) * ceil_div(M, BT));
  const int ktiles = (int)(K / BK);
  const int rem = tiles % cus;
  *rem_out = 0;
  if (rem == 0 || 2 * rem > cus || ktiles < 2) return 1;
  const size_t piece_bytes = (size_t)BN * BT * 4;
  const size_t fit = scratch_bytes / (piece_bytes * (size_t)rem);
  const int split = (int)std::min<size_t>((size_t)std::min(cus / rem, ktiles), fit);
  if (split < 2) return 1;
  const int per = (ktiles + split - 1) / split;
  *rem_out = rem;
  return (ktiles + per - 1) / per;  // every slice non-empty
}

size_t gemm_split_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  int rem = 0;
  const int split = plan_split(M, N, K, kPlanCus, (size_t)-1, &rem);
  return split > 1 ? (size_t)rem * split * BN * BT * 4 : 0;
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  const int tiles = (int)(ceil_div(a.N, BN) * ceil_div(a.M, BT));
  int rem = 0;
  a.split = a.partial ? plan_split(a.M, a.N, a.K, device_cus(), a.partial_bytes, &rem) : 1;
  a.full_tiles = tiles - (a.split > 1 ? rem : 0);
  const int grid = a.split > 1 ? a.full_tiles + rem * a.split : tiles;
  hipLaunchKernelGGL(gemm_kernel<EPI>, dim3(grid), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split <= 1) return e;
  hipLaunchKernelGGL(gemm_fixup_kernel<EPI>, dim3(rem, 4), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmEpilogue epi, const GemmArgs &a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV_ROPE: return launch_epi<EPI_QKV_ROPE>(a, s);
    case EPI_RESID_BF16: return launch_epi<EPI_RESID_BF16>(a, s);
    case EPI_RESID_F32: return launch_epi<EPI_RESID_F32>(a, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(a, s);
    case EPI_F32: return launch_epi<EPI_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace h3dit
