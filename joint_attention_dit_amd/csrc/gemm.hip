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
#include "gemm_common.h"

#include <type_traits>

namespace h3dit {

namespace {

constexpr int BK = 64;    // K per LDS stage (128-byte rows)
constexpr int TILE_ELEMS = 256 * BK;  // one operand tile, bf16 elements (32 KB)
constexpr int NW = 8;     // waves per workgroup (two per SIMD) of 128 features x 64 tokens
constexpr int JB = 4;     // token blocks of 16 per wave
constexpr int CP = 4;     // 1 KB copy blocks per wave per operand tile
constexpr int NT = 64 * NW;

template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmArgs a) {
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
  uint32_t woff[CP], xoff[CP];
#pragma unroll
  for (int j = 0; j < CP; ++j) {
    const int row = (wave * CP + j) * 8 + (lane >> 3);
    const int lc = swz(row, lane & 7);
    woff[j] = (uint32_t)(min(n0 + row, a.N - 1) - n0) * (uint32_t)a.K * 2u + lc * 16u;
    xoff[j] = (uint32_t)(min(t0 + row, a.M - 1) - t0) * (uint32_t)a.K * 2u + lc * 16u;
  }
  const uint32_t lds0 = lds_address(lds);
  // copies j0 .. j1-1 of the weight (activation) tile at k0 into weight stage
  // wst (activation stage xst)
  auto wload = [&](int wst, int k0, int j0, int j1) {
    const char *wp = wpanel + (int64_t)k0 * 2;
    const uint32_t sw = lds0 + (uint32_t)(wst * TILE_ELEMS + wave * CP * 512) * 2u;
#pragma unroll
    for (int j = j0; j < j1; ++j) dma16(wp, woff[j], sw + j * 1024);
  };
  auto xload = [&](int xst, int k0, int j0, int j1) {
    const char *xp = xpanel + (int64_t)k0 * 2;
    const uint32_t sx = lds0 + (uint32_t)((2 + xst) * TILE_ELEMS + wave * CP * 512) * 2u;
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
    fb_base[s] = (wt * 16 * JB + r16) * BK + (swz(r16, 4 * s + kq) * 8);
  }

  f32x4 acc[8][JB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // A fragments are re-read in place once their four products have issued; B
  // fragments are double buffered
  bf16x8 fa[8], fb[2][JB];
  auto fload_all = [&](int wst, int xst, int s, int buf) {
    const bf16 *sw = lds + wst * TILE_ELEMS;
    const bf16 *sx = lds + (2 + xst) * TILE_ELEMS;
#pragma unroll
    for (int j = 0; j < JB; ++j)
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
      for (int j = 0; j < JB; ++j) acc[i][j] = mfma16(fa[i], fb[BCUR][j], acc[i][j]);
      if constexpr (SYNC) {
        if (i == 0) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
          if (!RT || vm4) tile_barrier<CP>();
          else tile_barrier<0>();
        }
        if (i == 1 && (!RT || wref)) wload(kt & 1, (kt + 2) * BK, 0, CP / 2);
        if (i == 2 && (!RT || wref)) wload(kt & 1, (kt + 2) * BK, CP / 2, CP);
        if (i == 3 && (!RT || xref)) xload(xs, (kt + 3) * BK, 0, CP / 2);
        if (i == 4 && (!RT || xref)) xload(xs, (kt + 3) * BK, CP / 2, CP);
      }
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < JB; ++j)
          fb[BCUR ^ 1][j] = *reinterpret_cast<const bf16x8 *>(sx + fb_base[ns] + j * 16 * BK);
      }
      fa[i] = *reinterpret_cast<const bf16x8 *>(sw + fa_base[ns] + i * 16 * BK);
      // the next k-step's B fragments two reads per two products, then one A
      // fragment read per four products (measured: the fastest of the
      // groupings tried)
      if (i == 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
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

  wload(0, 0, 0, CP);
  xload(0, 0, 0, CP);
  if (ktiles > 1) {
    wload(1, BK, 0, CP);
    xload(1, BK, 0, CP);
  }
  if (ktiles > 2) {
    xload(2, 2 * BK, 0, CP);
    tile_barrier<3 * CP>();
  } else if (ktiles > 1) {
    tile_barrier<2 * CP>();
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
      for (int j = 0; j < JB; ++j) dst[(i * JB + j) * NT] = acc[i][j];
    return;
  }
  if constexpr (EPI == EPI_QKV_ROPE) {
    // every copy has landed and every wave has read its last fragments
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    staged_bf16_epilogue<EPI, JB, NT>(a, lds, acc, n0, t0, wn, wt, r16, kq);
    return;
  }
  direct_epilogue<EPI, JB>(a, acc, n0 + wn * 128 + 4 * kq, t0 + wt * 16 * JB + r16);
}

}  // namespace


size_t gemm_split_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  int rem = 0;
  const int split = plan_split(M, N, (int)(K / BK), kPlanCus, (size_t)-1, &rem);
  return split > 1 ? (size_t)rem * split * BN * BT * 4 : 0;
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  const int tiles = (int)(ceil_div(a.N, BN) * ceil_div(a.M, BT));
  int rem = 0;
  a.split = a.partial ? plan_split(a.M, a.N, a.K / BK, kPlanCus, a.partial_bytes, &rem) : 1;
  a.full_tiles = tiles - (a.split > 1 ? rem : 0);
  const int grid = a.split > 1 ? a.full_tiles + rem * a.split : tiles;
  hipLaunchKernelGGL((gemm_kernel<EPI>), dim3(grid), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split <= 1) return e;
  hipLaunchKernelGGL((gemm_fixup_kernel<EPI, NW>), dim3(rem, 4), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmEpilogue epi, const GemmArgs &a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV_ROPE: return launch_epi<EPI_QKV_ROPE>(a, s);
    case EPI_RESID_BF16: return launch_epi<EPI_RESID_BF16>(a, s);
    case EPI_RESID_F32: return launch_epi<EPI_RESID_F32>(a, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(a, s);
    case EPI_F32: return launch_epi<EPI_F32>(a, s);
    case EPI_GELU_MX: return hipErrorInvalidValue;  // MXFP8 GEMM only
  }
  return hipErrorInvalidValue;
}

}  // namespace h3dit
