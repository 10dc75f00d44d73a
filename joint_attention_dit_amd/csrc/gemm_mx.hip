// MXFP8 matrix-core GEMM for the DiT block's linears (vLLM blog "H3-Image
// Day-0 Support", section Inference Optimizations: the linears run in
// MXFP8). Both operands are E4M3 codes, K-contiguous, with one E8M0 scale
// per 32 consecutive K (OCP Microscaling), in the layout mxfp8.hip writes:
//
//   C[t, n] = sum_k (x[t, k] 2^(sx[t, k / 32] - 127)) (w[n, k] 2^(sw[n, k / 32] - 127))
//
// gfx950's scaled 16x16x128 product takes the codes and the per-row, per-32
// scales of both operands and accumulates in fp32. Lane l supplies 32 bytes
// of row l % 16: K chunks (16 bytes) l / 16 and 4 + l / 16 of the 128-wide K
// step, and the scale of 32-block l / 16 of that row; it receives the same
// output layout as the bf16 16x16x32 product, so the tile walk, the split of
// the last wave, the fixup and the epilogues are those of the bf16 GEMM.
//
// Tiling: 256 features x 256 tokens per workgroup, eight waves of 128 x 64,
// one K tile of 128 per LDS stage: a tile row is one 128-byte segment (the
// same copy shape as the bf16 kernel's 64-wide bf16 tiles) and one scaled
// product per 16 x 16 block. Operand tiles have two stages each (4 x 32 KB),
// followed by two 1 KB scale stages per operand (each wave copies 1/8 of a
// scale tile with 8 lanes enabled inside the copy's own asm block).
//
// Per K tile a wave runs its 8 feature blocks against its 4 token blocks,
// feature block by feature block. The fragments are twice as wide as bf16 ones
// (8 VGPRs), so the feature fragments live in a ring of 4 slots (block i in
// slot i mod 4): once block i's four products have issued, its slot is
// refilled with block i + 4 of the same tile or, from block 4 on, with block
// i - 4 of the next tile; the token fragments are re-read in place during the
// last feature block. The barrier sits after feature block 4, when every wave
// has read all its fragments of the current tile (its stages then take tile
// kt + 2) and every copy of tile kt + 1 has landed. The K-tile body has no
// branch (a conditional copy splits it into basic blocks, across which LLVM
// moves the side-effect-free products past the scheduling barriers and spills):
// past the end, the last tile is copied again into the free stage. LDS rows use
// the bf16 kernel's swizzle (16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7)).
#include "gemm_common.h"

#include <type_traits>

namespace h3dit {

namespace {

constexpr int KT = 128;                   // K per LDS stage (fp8 bytes per tile row)
constexpr int TILE_BYTES = 256 * KT;      // one operand tile (32 KB)
constexpr int SCALE_OFF = 4 * TILE_BYTES; // scale stages: W 0, W 1, X 0, X 1 (1 KB each)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// scaled 16x16x128 E4M3 product; OA / OB select the scale byte of sa / sb
template <int OA, int OB>
__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}

// A 16-byte global -> LDS copy by lanes 0 .. 7 only (dma16 with the other
// lanes disabled inside the same asm block, so no branch splits the caller's
// code): lane l < 8 reads base + voff and writes LDS bytes lds_addr + 16 l.
__device__ __forceinline__ void dma16_lanes8(const void *base, uint32_t voff, uint32_t lds_addr) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, 0xff\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "{m0}"(lds_addr)
      : "memory");
}

__device__ __forceinline__ i32x8 frag(const uint8_t *p, int o0, int o1) {
  const i32x4 lo = *reinterpret_cast<const i32x4 *>(p + o0);
  const i32x4 hi = *reinterpret_cast<const i32x4 *>(p + o1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_mx_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TILE_BYTES + 4 * 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;  // 2 x 4 waves of 128 features x 64 tokens
  const int tiles_n = (int)ceil_div(a.N, BN), tiles_t = (int)ceil_div(a.M, BT);
  const int ktot = a.K / KT;
  int tn, tt, piece = -1, kb0 = 0, ktiles = ktot;
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

  // global -> LDS: each wave fills 4 blocks of 1 KB (8 rows of 128 bytes) per
  // operand tile, as in the bf16 kernel; rows past the matrix edge repeat the
  // last row (their scales are 0 and their outputs are never stored).
  const char *wpanel = static_cast<const char *>(a.w) + (int64_t)n0 * a.K + kb0 * KT;
  const char *xpanel = static_cast<const char *>(a.x) + (int64_t)t0 * a.K + kb0 * KT;
  const char *wscale = reinterpret_cast<const char *>(a.w_scale) +
                       ((int64_t)tn * ktot + kb0) * 1024;
  const char *xscale = reinterpret_cast<const char *>(a.x_scale) +
                       ((int64_t)tt * ktot + kb0) * 1024;
  uint32_t woff[4], xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 8 + (lane >> 3);
    const int lc = swz(row, lane & 7);
    woff[j] = (uint32_t)(min(n0 + row, a.N - 1) - n0) * (uint32_t)a.K + lc * 16u;
    xoff[j] = (uint32_t)(min(t0 + row, a.M - 1) - t0) * (uint32_t)a.K + lc * 16u;
  }
  const uint32_t lds0 = lds_address(lds);
  auto wload = [&](int st, int kt, int j0, int j1) {
    const char *wp = wpanel + (int64_t)kt * KT;
    const uint32_t sw = lds0 + (uint32_t)(st * TILE_BYTES + wave * 4096);
#pragma unroll
    for (int j = j0; j < j1; ++j) dma16(wp, woff[j], sw + j * 1024);
  };
  auto xload = [&](int st, int kt, int j0, int j1) {
    const char *xp = xpanel + (int64_t)kt * KT;
    const uint32_t sx = lds0 + (uint32_t)((2 + st) * TILE_BYTES + wave * 4096);
#pragma unroll
    for (int j = j0; j < j1; ++j) dma16(xp, xoff[j], sx + j * 1024);
  };
  // scale tiles: wave w copies bytes 128 w .. 128 w + 127 of each (8 lanes)
  const uint32_t soff = (uint32_t)(wave * 128) + (uint32_t)(lane & 7) * 16u;
  auto sload = [&](int st, int kt) {
    dma16_lanes8(wscale + (int64_t)kt * 1024, soff, lds0 + SCALE_OFF + st * 1024 + wave * 128);
    dma16_lanes8(xscale + (int64_t)kt * 1024, soff,
                 lds0 + SCALE_OFF + 2048 + st * 1024 + wave * 128);
  };

  // fragment reads: row r16 of each 16-row block, K chunks kq and 4 + kq;
  // scales: this lane's row and 32-block kq, the 8 feature blocks (4 token
  // blocks) of the wave in consecutive bytes
  const int r16 = lane & 15, kq = lane >> 4;
  const int fa0 = (wn * 128 + r16) * KT + swz(r16, kq) * 16;
  const int fa1 = (wn * 128 + r16) * KT + swz(r16, 4 + kq) * 16;
  // the activation stages and the scales lie beyond the 64 KB reach of an
  // LDS read's immediate offset: their per-lane bases include the region start
  // and are kept opaque, so every read is base + (stage, block) immediate
  int fb0 = 2 * TILE_BYTES + (wt * 64 + r16) * KT + swz(r16, kq) * 16;
  int fb1 = 2 * TILE_BYTES + (wt * 64 + r16) * KT + swz(r16, 4 + kq) * 16;
  int sao = SCALE_OFF + (kq * 16 + r16) * 16 + wn * 8;
  int sbo = SCALE_OFF + 2048 + (kq * 16 + r16) * 16 + wt * 4;
  asm volatile("" : "+v"(fb0), "+v"(fb1), "+v"(sao), "+v"(sbo));

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // feature fragments in a ring of 4 (block i in slot i & 3), token fragments
  // of the 4 token blocks; scales of the tiles in stages 0 and 1
  i32x8 fa[4], fb[4];
  int sa[2][2], sb[2];
  auto sread = [&](int st) {
    const u32x2 w2 = *reinterpret_cast<const u32x2 *>(lds + sao + st * 1024);
    sa[st][0] = (int)w2[0];
    sa[st][1] = (int)w2[1];
    sb[st] = *reinterpret_cast<const int *>(lds + sbo + st * 1024);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;

  // product of feature block I and token block J of the tile in stage ST
  auto mm = [&](auto i_c, auto j_c, auto st_c) {
    constexpr int I = decltype(i_c)::value, J = decltype(j_c)::value;
    constexpr int ST = decltype(st_c)::value;
    acc[I][J] = mfma_mx<I & 3, J>(fa[I & 3], fb[J], acc[I][J], sa[ST][I >> 2], sb[ST]);
  };
  // feature block I against the 4 token blocks, then feature fragment `blk`
  // of the tile at p into its slot
  auto row = [&](auto i_c, auto st_c, const uint8_t *p, int blk) {
    constexpr int I = decltype(i_c)::value;
    mm(i_c, I0(), st_c);
    mm(i_c, I1(), st_c);
    mm(i_c, I2(), st_c);
    mm(i_c, I3(), st_c);
    __builtin_amdgcn_sched_barrier(0);
    fa[I & 3] = frag(p + blk * 16 * KT, fa0, fa1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // K tile kt in stage ST = kt & 1; on entry feature blocks 0 .. 3, the token
  // blocks and the scales of tile kt are in registers (or on their way). The
  // last K tile still reads (stale) fragments of the other stage, which is
  // harmless.
  auto ktile = [&](auto st_c, int kt) {
    constexpr int ST = decltype(st_c)::value, NS = ST ^ 1;
    const uint8_t *sw = lds + ST * TILE_BYTES;
    const uint8_t *swn = lds + NS * TILE_BYTES;
    const uint8_t *sxn = lds + NS * TILE_BYTES;  // + fb0 / fb1: activation stage NS
    row(I0(), st_c, sw, 4);
    row(I1(), st_c, sw, 5);
    row(I2(), st_c, sw, 6);
    row(I3(), st_c, sw, 7);
    mm(I4(), I0(), st_c);
    mm(I4(), I1(), st_c);
    mm(I4(), I2(), st_c);
    mm(I4(), I3(), st_c);
    // every wave has read all its fragments of tile kt (stage ST is free) and
    // every copy of tile kt + 1 has landed
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
    tile_barrier<0>();
    {  // past the end, the last tile is copied again into the free stage
      const int kc = min(kt + 2, ktiles - 1);
      wload(ST, kc, 0, 4);
      xload(ST, kc, 0, 4);
      sload(ST, kc);
    }
    __builtin_amdgcn_sched_barrier(0);
    sread(NS);
    fa[0] = frag(swn, fa0, fa1);
    __builtin_amdgcn_sched_barrier(0);
    row(I5(), st_c, swn, 1);
    row(I6(), st_c, swn, 2);
    // the last feature block; each token fragment is re-read once its product
    // has issued
    mm(I7(), I0(), st_c);
    __builtin_amdgcn_sched_barrier(0);
    fb[0] = frag(sxn, fb0, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mm(I7(), I1(), st_c);
    __builtin_amdgcn_sched_barrier(0);
    fb[1] = frag(sxn + 16 * KT, fb0, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mm(I7(), I2(), st_c);
    __builtin_amdgcn_sched_barrier(0);
    fb[2] = frag(sxn + 32 * KT, fb0, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mm(I7(), I3(), st_c);
    __builtin_amdgcn_sched_barrier(0);
    fb[3] = frag(sxn + 48 * KT, fb0, fb1);
    fa[3] = frag(swn + 3 * 16 * KT, fa0, fa1);
    __builtin_amdgcn_sched_barrier(0);
  };

  wload(0, 0, 0, 4);
  xload(0, 0, 0, 4);
  sload(0, 0);
  if (ktiles > 1) {
    wload(1, 1, 0, 4);
    xload(1, 1, 0, 4);
    sload(1, 1);
    // tile 0 has landed when at most tile 1's 10 copies are in flight
    tile_barrier<10>();
  } else {
    tile_barrier<0>();
  }
  sread(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = frag(lds + i * 16 * KT, fa0, fa1);
#pragma unroll
  for (int j = 0; j < 4; ++j) fb[j] = frag(lds + j * 16 * KT, fb0, fb1);
  int kt = 0;
  for (; kt + 1 < ktiles; kt += 2) {
    ktile(I0(), kt);
    ktile(I1(), kt + 1);
  }
  if (kt < ktiles) ktile(I0(), kt);
  // the last K tiles re-copy the final tile: let every copy land before the
  // workgroup's LDS is reused or released
  __builtin_amdgcn_s_waitcnt(0);

  if (piece >= 0) {  // a K slice: raw sums to the scratch, [register block][thread]
    f32x4 *dst = reinterpret_cast<f32x4 *>(a.partial) + (int64_t)piece * (32 * 512) + tid;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(i * 4 + j) * 512] = acc[i][j];
    return;
  }
  if constexpr (EPI == EPI_QKV_ROPE) {
    // every wave has read its last fragments
    __syncthreads();
    staged_bf16_epilogue<EPI>(a, reinterpret_cast<bf16 *>(lds), acc, n0, t0, wn, wt, r16, kq);
    return;
  }
  const int nb = n0 + wn * 128 + 4 * kq, tb = t0 + wt * 64 + r16;
  if constexpr (EPI == EPI_GELU_MX) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        gelu_mx_block(a, tb + 16 * j, nb + 32 * m, kq, acc[2 * m][j], acc[2 * m + 1][j]);
    return;
  }
  direct_epilogue<EPI, 4>(a, acc, nb, tb);
}

}  // namespace

size_t gemm_mx_split_scratch_bytes(int64_t M, int64_t N, int64_t K) {
  int rem = 0;
  const int split = plan_split(M, N, (int)(K / KT), kPlanCus, (size_t)-1, &rem);
  return split > 1 ? (size_t)rem * split * BN * BT * 4 : 0;
}

template <int EPI>
static hipError_t launch_mx_epi(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  const int tiles = (int)(ceil_div(a.N, BN) * ceil_div(a.M, BT));
  int rem = 0;
  a.split = a.partial ? plan_split(a.M, a.N, a.K / KT, kPlanCus, a.partial_bytes, &rem) : 1;
  a.full_tiles = tiles - (a.split > 1 ? rem : 0);
  const int grid = a.split > 1 ? a.full_tiles + rem * a.split : tiles;
  hipLaunchKernelGGL(gemm_mx_kernel<EPI>, dim3(grid), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split <= 1) return e;
  hipLaunchKernelGGL(gemm_fixup_kernel<EPI>, dim3(rem, 4), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(GemmEpilogue epi, const GemmArgs &a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV_ROPE: return launch_mx_epi<EPI_QKV_ROPE>(a, s);
    case EPI_RESID_BF16: return launch_mx_epi<EPI_RESID_BF16>(a, s);
    case EPI_RESID_F32: return launch_mx_epi<EPI_RESID_F32>(a, s);
    case EPI_GELU: return launch_mx_epi<EPI_GELU>(a, s);
    case EPI_F32: return launch_mx_epi<EPI_F32>(a, s);
    case EPI_GELU_MX: return launch_mx_epi<EPI_GELU_MX>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace h3dit
