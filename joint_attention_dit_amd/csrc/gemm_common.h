// Tile walk, epilogues, split-K fixup and split planning shared by the bf16
// GEMM (gemm.hip) and the MXFP8 GEMM (gemm_mx.hip). Both produce a 256 x 256
// output tile per workgroup of eight waves (2 x 4, 128 features x 64 tokens
// each) with the 16 x 16 matrix-core output layout: lane l of a wave holds
// output features 4 (l / 16) .. +3 of token l % 16 of each 16 x 16 block.
#pragma once

#include "common.h"
#include "kernels.h"
#include "mxfp8_device.h"

#include <algorithm>

namespace h3dit {

namespace {

constexpr int BN = 256;   // weight rows (output features) per tile
constexpr int BT = 256;   // activation rows (tokens) per tile
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

// 0.5 z (1 + tanh(y)) == z / (1 + e^(-2y)),  y = sqrt(2/pi) (z + 0.044715 z^3),
// with e^(-2y) = 2^(z (k1 + k3 z^2)) taken by the hardware exp2 and the division by
// the hardware reciprocal (each within 1 ulp): seven instructions instead of the
// 24 of expf and an IEEE division. The result is within about 2^-19 of the
// exact value, far inside the bf16 rounding that follows (an element's bf16
// value moves by one ulp in about 1e-4 of the elements). For z below about -11
// the reciprocal of 1 + e^(-2y) may flush to zero, giving -0 for a value whose
// magnitude is below 1e-36.
__device__ __forceinline__ float gelu_tanh(float z) {
  constexpr float k1 = (float)(-2.0 * 1.4426950408889634 * 0.7978845608028654);
  constexpr float k3 = (float)(-2.0 * 1.4426950408889634 * 0.7978845608028654 * 0.044715);
  const float a = z * fmaf(k3, z * z, k1);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}

// q or k: rotate the two adjacent pairs of the fp32 products, then round once;
// q also takes the softmax factor log2(e)/sqrt(128) before its rounding, so that
// attention scores leave the matrix cores in base-2 units.
// cos, sin of the two pairs of features n .. n + 3 (n % 4 == 0) of token t
__device__ __forceinline__ f32x4 rope_cs4(const GemmArgs &a, int t, int n) {
  const int p = (n & 127) >> 1;  // pair index within the head (0..63)
  return *reinterpret_cast<const f32x4 *>(a.table + ((int64_t)t * 64 + p) * 2);
}

__device__ __forceinline__ bf16x4 qk_rope4(const GemmArgs &a, int n, const f32x4 &cs, float v0,
                                           float v1, float v2, float v3) {
  const float u0 = v0, w0 = v1, u1 = v2, w1 = v3;
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

// token t of a V tile is stored at column vt_col(t): bits 4, 3, 2 of t move to
// bits 2, 4, 3, a permutation within each group of 32 keys (the key order of
// the attention kernel's P V fragments)
__device__ __forceinline__ int vt_col(int t) {
  return (t & ~28) | ((t & 12) << 1) | ((t & 16) >> 2);
}

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
          qk_rope4(a, n, rope_cs4(a, t, n), v0, v1, v2, v3);
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

// The epilogue of a whole tile from registers (every epilogue but QKV's and
// GELU_MX's): lane holds features nb + 16 i .. +3 of token tb + 16 j in
// acc[i][j]. Each operand load is issued unconditionally (addresses clamped
// into the matrix) and only the stores are predicated, so the residual rows of
// eight feature blocks are in flight together instead of one per round trip
// (a load guarded by the bounds branch of store4 waits for the previous
// block's store). Same arithmetic as store4. N % 4 == 0.
template <int EPI, int JB>
__device__ __forceinline__ void direct_epilogue(const GemmArgs &a, const f32x4 (&acc)[8][JB], int nb,
                                                int tb) {
  if constexpr (EPI == EPI_RESID_BF16 || EPI == EPI_RESID_F32) {
    float g[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int nc = min(nb + 16 * i, a.N - 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) g[i][e] = (float)a.gate[nc + e];
    }
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int t = tb + 16 * j;
      const int64_t row = (int64_t)min(t, a.M - 1) * a.N;
      f32x4 rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t off = row + min(nb + 16 * i, a.N - 4);
        if constexpr (EPI == EPI_RESID_BF16) {
          const bf16x4 rb = *reinterpret_cast<const bf16x4 *>(static_cast<const bf16 *>(a.resid) + off);
          rv[i] = f32x4{(float)rb[0], (float)rb[1], (float)rb[2], (float)rb[3]};
        } else {
          rv[i] = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.resid) + off);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = nb + 16 * i;
        if (t < a.M && n < a.N) {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = rv[i][e] + g[i][e] * acc[i][j][e];
          *reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + (int64_t)t * a.N + n) = ov;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        store4<EPI>(a, tb + 16 * j, nb + 16 * i, acc[i][j][0], acc[i][j][1], acc[i][j][2],
                    acc[i][j][3]);
  }
}

// GELU outputs of one block of 32 features of token t as bf16 (u) and as
// MXFP8 codes + scale. The calling lane holds features n .. n + 3 (v0) and
// n + 16 .. n + 19 (v1) with n = 32 m + 4 kq (kq = lane bits 4, 5); the four
// lanes kq = 0..3 together hold the block, so every lane of the wave must
// call this (the block maximum is exchanged across them). N % 32 == 0.
__device__ __forceinline__ void gelu_mx_block(const GemmArgs &a, int t, int n, int kq,
                                              const f32x4 &v0, const f32x4 &v1) {
  const bf16x4 g0 = gelu4(v0[0], v0[1], v0[2], v0[3]);
  const bf16x4 g1 = gelu4(v1[0], v1[1], v1[2], v1[3]);
  // magnitudes of the eight bf16 values from whole-vector bit patterns (a
  // bit cast of single vector elements kept only element 0 here)
  const u32x2 w0 = __builtin_bit_cast(u32x2, g0), w1 = __builtin_bit_cast(u32x2, g1);
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    amax = max(amax, max(w0[e] & 0x7FFFu, (w0[e] >> 16) & 0x7FFFu));
    amax = max(amax, max(w1[e] & 0x7FFFu, (w1[e] >> 16) & 0x7FFFu));
  }
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
  const int sbyte = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sbyte);
  if (t >= a.M || n >= a.N) return;
  const int64_t off = (int64_t)t * a.N + n;
  if (a.out) {  // the bf16 copy of u (left out when only the codes are consumed)
    bf16 *u = static_cast<bf16 *>(a.out);
    *reinterpret_cast<bf16x4 *>(u + off) = g0;
    *reinterpret_cast<bf16x4 *>(u + off + 16) = g1;
  }
  *reinterpret_cast<uint32_t *>(a.out_codes + off) =
      mx_code4((float)g0[0], (float)g0[1], (float)g0[2], (float)g0[3], inv);
  *reinterpret_cast<uint32_t *>(a.out_codes + off + 16) =
      mx_code4((float)g1[0], (float)g1[1], (float)g1[2], (float)g1[3], inv);
  if (kq == 0) a.out_scales[mx_scale_offset(t, n >> 5, a.N)] = (uint8_t)sbyte;
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
// JB: token blocks of 16 per wave (4: eight waves of 128 x 64, 8: four waves
// of 128 x 128); NT threads per workgroup.
template <int EPI, int JB = 4, int NT = 512>
__device__ __forceinline__ void staged_bf16_epilogue(const GemmArgs &a, bf16 *lds, const f32x4 (&acc)[8][JB],
                                                     int n0, int t0, int wn, int wt, int r16, int kq) {
  const int tid = threadIdx.x;
  bool vtile = false;
  if constexpr (EPI == EPI_QKV_ROPE) vtile = n0 >= 2 * a.A;
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int tl = wt * 16 * JB + 16 * j + r16, t = t0 + tl;
    if constexpr (EPI == EPI_QKV_ROPE) {
      if (vtile) {
        const bool live = t < a.M;
        const int col = vt_col(tl);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int fl = wn * 128 + 16 * i + 4 * kq;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lds[stage_off(fl + e, col)] = to_bf16(live ? acc[i][j][e] : 0.0f);
        }
        continue;
      }
      // the eight table entries of this token block are loaded together
      // (token clamped into the table), then rotated
      f32x4 cs[8];
      const int tc = min(t, a.M - 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) cs[i] = rope_cs4(a, tc, n0 + wn * 128 + 16 * i + 4 * kq);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int fl = wn * 128 + 16 * i + 4 * kq;
        const f32x4 v = acc[i][j];
        const bf16x4 r = t < a.M ? qk_rope4(a, n0 + fl, cs[i], v[0], v[1], v[2], v[3]) : bf16x4{};
        *reinterpret_cast<bf16x4 *>(lds + stage_off(tl, fl)) = r;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int fl = wn * 128 + 16 * i + 4 * kq;
        const f32x4 v = acc[i][j];
        *reinterpret_cast<bf16x4 *>(lds + stage_off(tl, fl)) = gelu4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int q = tid; q < 256 * 32; q += NT) {
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

// Sum of the K slices of split tile full_tiles + blockIdx.x (in slice order),
// then the epilogue, with the thread -> output mapping of the GEMM kernel of
// NW waves (partial sums stored [register block i * JB + j][thread]);
// workgroup blockIdx.y takes feature blocks 2 y and 2 y + 1 of every wave.
template <int EPI, int NW = 8>
__global__ __launch_bounds__(64 * NW) void gemm_fixup_kernel(GemmArgs a) {
  constexpr int JB = 32 / NW, NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wt = wave >> 1;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tiles_n = (int)ceil_div(a.N, BN), tiles_t = (int)ceil_div(a.M, BT);
  int tn, tt;
  walk_coords(a.full_tiles + blockIdx.x, tiles_n, tiles_t, tn, tt);
  const f32x4 *src =
      reinterpret_cast<const f32x4 *>(a.partial) + (int64_t)blockIdx.x * a.split * (32 * 512) + tid;
  const int nb = tn * BN + wn * 128 + 4 * kq, tb = tt * BT + wt * 16 * JB + r16;
  if constexpr (EPI == EPI_GELU_MX) {  // feature blocks 2 y, 2 y + 1 are one block of 32
    const int i = 2 * (int)blockIdx.y;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int64_t o0 = (i * JB + j) * NT, o1 = ((i + 1) * JB + j) * NT;
      f32x4 v0 = src[o0], v1 = src[o1];
      for (int sl = 1; sl < a.split; ++sl) {
        v0 += src[(int64_t)sl * (32 * 512) + o0];
        v1 += src[(int64_t)sl * (32 * 512) + o1];
      }
      gelu_mx_block(a, tb + 16 * j, nb + 16 * i, kq, v0, v1);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * (int)blockIdx.y + ii;
      const int64_t o = (i * JB + j) * NT;
      f32x4 v = src[o];
      for (int sl = 1; sl < a.split; ++sl) v += src[(int64_t)sl * (32 * 512) + o];
      store4<EPI>(a, tb + 16 * j, nb + 16 * i, v[0], v[1], v[2], v[3]);
    }
}

// The split plan is made for MI355X's 256 compute units on every device, so
// the order in which a tile's K slices are summed (and with it the fp32
// rounding of the result) never depends on the device the library runs on.
constexpr int kPlanCus = 256;

// One workgroup per CU at a time. The last, partial wave of `rem` tiles is cut
// along K into s slices (a second kernel adds them) when that shortens it: cut
// into s, its tiles take ceil(rem s / cus) waves of 1/s of a tile, plus the
// slices' own costs (writing and re-reading the fp32 partial sums and refilling
// the copy pipeline, about 8 % of a whole tile per slice), against one whole
// wave uncut. The smallest s within 0.05 waves of the lowest cost is taken, if
// it saves at least a tenth of a wave and fits the scratch. A tail of more than
// half a wave is only cut when at least 8 whole waves precede it: the split
// tiles' fixup (partial sums through memory, the QKV epilogue without LDS
// staging) costs more than the shorter tail saves when they are a larger share
// of the work (measured on the QKV GEMM: -3 % at 66 token tiles, +3 % at 17).
// Returns the slices per split tile (1: no split) and the number of split tiles.
static int plan_split(int64_t M, int64_t N, int ktiles, int cus, size_t scratch_bytes,
                      int *rem_out) {
  const int tiles = (int)(ceil_div(N, BN) * ceil_div(M, BT));
  const int rem = tiles % cus;
  *rem_out = 0;
  if (rem == 0 || ktiles < 2) return 1;
  if (2 * rem > cus && tiles / cus < 8) return 1;
  const size_t piece_bytes = (size_t)BN * BT * 4;
  const size_t fit = scratch_bytes / (piece_bytes * (size_t)rem);
  auto cost = [&](int sl) { return ((rem * sl + cus - 1) / cus) * (1.0 / sl + 0.08); };
  const int smax = std::min<int>(std::min(ktiles, 16), (int)std::min<size_t>(fit, 16));
  double lowest = 1.0;
  for (int sl = 2; sl <= smax; ++sl) lowest = std::min(lowest, cost(sl));
  int best = 1;
  for (int sl = 2; sl <= smax && best == 1; ++sl)
    if (cost(sl) <= lowest + 0.05) best = sl;
  if (best < 2 || cost(best) > 0.9) return 1;
  const int per = (ktiles + best - 1) / best;
  *rem_out = rem;
  return (ktiles + per - 1) / per;  // every slice non-empty
}

}  // namespace

}  // namespace h3dit
