// RMSNorm + AdaLN modulation (apxml.com spec page: RMS normalisation, scaled
// and shifted by the AdaLN modulation). One wavefront per token row:
//   pass 1: sum of squares in fp64 (squares of bf16 / fp32 values are exact);
//   pass 2: h = x * r * (1 + scale) + shift in fp64, one rounding to bf16.
// The output is bf16 (a matrix-core operand) or, for the final layer of the
// DiT stack, fp32. For rows of up to 8192 elements the row stays in registers between the
// passes, so x is read from memory once (with thousands of rows in flight the
// L2 does not keep a row until its second pass); longer rows are read twice.
// For the MXFP8 linears the register-row kernel can also quantise its bf16
// output to E4M3 codes and E8M0 scales (one per 32 consecutive elements; the
// four lanes that hold a block of 32 find its maximum with two exchanges).
#include "common.h"
#include "kernels.h"
#include "mxfp8_device.h"

#include <algorithm>
#include <type_traits>

namespace h3dit {

template <typename XT>
struct Chunk8;

// 8 consecutive elements kept in their storage type (bf16: 4 registers)
template <>
struct Chunk8<bf16> {
  typedef bf16x8 raw;
  // the block's input rows: read once, with the nontemporal hint
  static __device__ __forceinline__ raw fetch(const bf16 *p) {
    return load_once(reinterpret_cast<const bf16x8 *>(p));
  }
  static __device__ __forceinline__ float at(const raw &r, int j) { return (float)r[j]; }
  static __device__ __forceinline__ void load(const bf16 *p, float v[8]) {
    const raw t = fetch(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)t[j];
  }
};

template <>
struct Chunk8<float> {
  struct raw {
    f32x4 a, b;
  };
  // plain loads: fp32 rows are the residual stream that the previous kernel has
  // just written, partly still in the last-level cache (the nontemporal hint
  // measured 2-14 % slower on them)
  static __device__ __forceinline__ raw fetch(const float *p) {
    return raw{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
  }
  static __device__ __forceinline__ float at(const raw &r, int j) { return j < 4 ? r.a[j] : r.b[j - 4]; }
  static __device__ __forceinline__ void load(const float *p, float v[8]) {
    const raw t = fetch(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = at(t, j);
  }
};

// Store 8 consecutive results (fp64) as bf16 (one rounding) or fp32.
template <typename OT>
__device__ __forceinline__ void store8(OT *p, const double v[8]);
template <>
__device__ __forceinline__ void store8<bf16>(bf16 *p, const double v[8]) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = to_bf16(v[j]);
  *reinterpret_cast<bf16x8 *>(p) = o;
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const double v[8]) {
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = (float)v[j];
    b[j] = (float)v[4 + j];
  }
  *reinterpret_cast<f32x4 *>(p) = a;
  *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// Rows in registers: each wave normalises R rows; lane l holds their 16-byte
// chunks l, l + 64, ... (at most NC), and reads the fp64 shift and scale of its
// columns once for all R rows (for bf16 rows they are 8x the row's own bytes).
// R = 2 for bf16 rows; fp32 rows take twice the registers, and two of them
// would leave one wave per SIMD, so they go one per wave.
// With MX (bf16 output only), the rows are also written as MXFP8 codes [T, D]
// and scales (1 KB block layout of mxfp8_device.h).
template <typename XT, int NC, typename OT, bool MX = false, int R = (sizeof(XT) == 2 ? 2 : 1)>
__global__ __launch_bounds__(256) void rmsnorm_modulate_reg_kernel(
    const XT *__restrict__ x, const double *__restrict__ shift, const double *__restrict__ scale,
    OT *__restrict__ h, int T, int D, double eps, uint8_t *__restrict__ codes = nullptr,
    uint8_t *__restrict__ scales = nullptr) {
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (row0 >= T) return;
  const int chunks = D >> 3;

  typename Chunk8<XT>::raw v[R][NC];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const XT *xr = x + (int64_t)min(row0 + k, T - 1) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) v[k][i] = Chunk8<XT>::fetch(xr + c * 8);
    }
  }
  double rs[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i < chunks) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double e = (double)Chunk8<XT>::at(v[k][i], j);
          ss += e * e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    rs[k] = 1.0 / sqrt(ss / (double)D + eps);
  }

#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      double sc1[8], sh[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sc1[j] = 1.0 + scale[c * 8 + j];
        sh[j] = shift[c * 8 + j];
      }
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int row = row0 + k;
        if (row >= T) break;  // uniform across the wave
        double o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (double)Chunk8<XT>::at(v[k][i], j) * rs[k] * sc1[j] + sh[j];
        if (!MX || h) store8<OT>(h + (int64_t)row * D + c * 8, o);  // MX: h may be left out
        if constexpr (MX) {
          // chunks 4m .. 4m + 3 (lanes 4m' .. 4m' + 3; D % 128 == 0, so a group
          // of four lanes is active or idle together) form one block of 32
          float g[8];
          uint32_t amax = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16 b = to_bf16(o[j]);
            g[j] = (float)b;
            amax = max(amax, (uint32_t)__builtin_bit_cast(uint16_t, b) & 0x7FFFu);
          }
          amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
          amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
          const int sbyte = mx_scale_byte(amax);
          const float inv = mx_inv_scale(sbyte);
          const u32x2 q = {mx_code4(g[0], g[1], g[2], g[3], inv),
                           mx_code4(g[4], g[5], g[6], g[7], inv)};
          *reinterpret_cast<u32x2 *>(codes + (int64_t)row * D + c * 8) = q;
          if ((lane & 3) == 0) scales[mx_scale_offset(row, c >> 2, D)] = (uint8_t)sbyte;
        }
      }
    }
  }
}

// Rounds 8 fp64 values once to bf16 (nearest, ties to even) by way of fp32:
// f = fp32(o) rounds to nearest, and rounding f to bf16 then gives o's own bf16
// rounding unless f sits exactly on a midpoint between two bf16 values while o
// does not (o lies just beside that midpoint and f landed on it). Only then is
// f moved one fp32 step toward o, so that the bf16 rounding goes o's way. The
// check is two integer operations per value and the fix a wave-uniform branch
// that a wave's chunk of 8 x 64 values takes about once in a hundred times;
// the compiler's exact fp64-to-bf16 conversion costs about eight operations
// each. value(j) recomputes o[j] for the fix (from operands it reloads), so the
// doubles need not stay in registers until then.
template <typename F>
__device__ __forceinline__ void round8_via_f32(float f[8], F value) {
  uint64_t tie = 0;  // the lanes with a value on a midpoint (one compare and a scalar or each)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    tie |= __builtin_amdgcn_ballot_w64((__builtin_bit_cast(uint32_t, f[j]) & 0xFFFFu) == 0x8000u);
  if (__builtin_expect(tie != 0, 0)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = __builtin_bit_cast(uint32_t, f[j]);
      const double o = value(j);
      if ((u & 0xFFFFu) == 0x8000u && (double)f[j] != o)
        f[j] = __builtin_bit_cast(float, fabs((double)f[j]) < fabs(o) ? u + 1u : u - 1u);
    }
  }
}

// Store 8 values (already adjusted by round8_via_f32) as bf16, or fp32 ones.
__device__ __forceinline__ void store8f(bf16 *p, const float f[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const bf16x2 t = pack2(f[j], f[j + 1]);
    v[j] = t[0];
    v[j + 1] = t[1];
  }
  *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void store8f(float *p, const float f[8]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// Persistent form for rows of up to 8192 elements: one workgroup per CU stages
// (1 + scale) and shift (fp64) in LDS once, then each wave normalises rows
// w, w + W, ... (W waves in all; w numbers the waves wave-major across the
// workgroups, so the waves with one row more than the others are spread over
// all CUs), one row at a time, held in registers between the two passes.
// The per-row fp64 modulation vectors then come from LDS rather than from L2
// (for bf16 rows they are 16x the row's own bytes), and the many waves per CU
// (16 for bf16 rows, 12 for fp32 rows) keep enough row loads in flight.
// The fp64 results are rounded by round8_via_f32 (fp32 output: the plain
// rounding to fp32).
// LDS layout: element 8 c + 2 q + e of array a (0: 1 + scale, 1: shift) at
// double index ((a * 4 + q) * 64 NC + c) * 2 + e (NC: chunks per lane), so the
// 16-byte reads of consecutive lanes (consecutive c) are consecutive and every
// read of a lane is an immediate offset from one of two base addresses.
// Threads per workgroup: as many waves as the registers allow (fp32 rows, the
// MXFP8 epilogue and the longest rows take more registers per wave).
template <typename XT, int NC, bool MX>
struct LdsNorm {
  static constexpr int waves = (sizeof(XT) == 2 ? 16 : 12) - (MX || NC > 11 ? 4 : 0);
  static constexpr int threads = 64 * waves;
  static constexpr size_t lds_bytes = (size_t)2 * 8 * 64 * NC * sizeof(double);
};

// Keeps v opaque to the compiler between the two passes, so it re-converts
// the stored elements instead of holding 8 doubles per chunk across them.
__device__ __forceinline__ void opaque(bf16x8 &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(Chunk8<float>::raw &v) {
  asm volatile("" : "+v"(v.a), "+v"(v.b));
}

template <typename XT, int NC, typename OT, bool MX = false>
__global__ __launch_bounds__((LdsNorm<XT, NC, MX>::threads)) void rmsnorm_modulate_lds_kernel(
    const XT *__restrict__ x, const double *__restrict__ shift, const double *__restrict__ scale,
    OT *__restrict__ h, int T, int D, double eps, uint8_t *__restrict__ codes = nullptr,
    uint8_t *__restrict__ scales = nullptr) {
  constexpr int NT = LdsNorm<XT, NC, MX>::threads, NWG = NT / 64;
  extern __shared__ __attribute__((aligned(16))) double mod_lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunks = D >> 3;
  constexpr int PL = NC * 64;  // chunks per plane (a compile-time stride: immediate offsets)
  for (int i = tid; i < D; i += NT) {
    const int c = i >> 3, q = (i >> 1) & 3, e = i & 1;
    mod_lds[((0 * 4 + q) * PL + c) * 2 + e] = 1.0 + scale[i];
    mod_lds[((1 * 4 + q) * PL + c) * 2 + e] = shift[i];
  }
  __syncthreads();
  const int W = (int)gridDim.x * NWG;
  for (int row = wave * (int)gridDim.x + (int)blockIdx.x; row < T; row += W) {
    typename Chunk8<XT>::raw v[NC];
    const XT *xr = x + (int64_t)row * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) v[i] = Chunk8<XT>::fetch(xr + c * 8);
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (lane + 64 * i < chunks) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double e = (double)Chunk8<XT>::at(v[i], j);
          ss += e * e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const double rs = 1.0 / sqrt(ss / (double)D + eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) opaque(v[i]);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        // element j of chunk cc from the LDS vectors: (1 + scale) and shift
        auto mod = [&](int cc, int arr, int j) {
          return mod_lds[((arr * 4 + (j >> 1)) * PL + cc) * 2 + (j & 1)];
        };
        const typename Chunk8<XT>::raw vi = v[i];
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          f[j] = (float)((double)Chunk8<XT>::at(vi, j) * rs * mod(c, 0, j) + mod(c, 1, j));
        if constexpr (std::is_same<OT, bf16>::value) {
          round8_via_f32(f, [&](int j) {
            // opaque copies: the compiler reloads the operands instead of
            // keeping the fast path's doubles alive for this rare branch
            int cc = c;
            double r = rs;
            asm volatile("" : "+v"(cc), "+v"(r));
            return (double)Chunk8<XT>::at(vi, j) * r * mod(cc, 0, j) + mod(cc, 1, j);
          });
        }
        if (!MX || h) store8f(h + (int64_t)row * D + c * 8, f);  // MX: h may be left out
        if constexpr (MX) {
          float g[8];
          uint32_t amax = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16 bv = to_bf16(f[j]);
            g[j] = (float)bv;
            amax = max(amax, (uint32_t)__builtin_bit_cast(uint16_t, bv) & 0x7FFFu);
          }
          amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
          amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
          const int sbyte = mx_scale_byte(amax);
          const float inv = mx_inv_scale(sbyte);
          const u32x2 qv = {mx_code4(g[0], g[1], g[2], g[3], inv),
                            mx_code4(g[4], g[5], g[6], g[7], inv)};
          *reinterpret_cast<u32x2 *>(codes + (int64_t)row * D + c * 8) = qv;
          if ((lane & 3) == 0) scales[mx_scale_offset(row, c >> 2, D)] = (uint8_t)sbyte;
        }
      }
      // one chunk at a time: the other waves of the CU hide the LDS latency,
      // and the chunks' fp64 temporaries never pile up in registers
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Longer rows: two passes over memory.
template <typename XT, typename OT>
__global__ __launch_bounds__(256) void rmsnorm_modulate_kernel(const XT *__restrict__ x,
                                                               const double *__restrict__ shift,
                                                               const double *__restrict__ scale,
                                                               OT *__restrict__ h, int T, int D,
                                                               double eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const XT *xr = x + (int64_t)row * D;
  OT *hr = h + (int64_t)row * D;
  const int chunks = D >> 3;

  double ss = 0.0;
  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    Chunk8<XT>::load(xr + c * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += (double)v[j] * (double)v[j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double r = 1.0 / sqrt(ss / (double)D + eps);

  for (int c = lane; c < chunks; c += 64) {
    float v[8];
    Chunk8<XT>::load(xr + c * 8, v);
    double o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = c * 8 + j;
      o[j] = (double)v[j] * r * (1.0 + scale[col]) + shift[col];
    }
    store8<OT>(hr + c * 8, o);
  }
}

// One workgroup per CU (its LDS holds 16 D bytes); fewer when there are fewer
// rows than waves.
static int lds_grid(int T, int waves) { return (int)std::min<int64_t>(256, ceil_div(T, waves)); }

template <typename OT, bool MX>
static hipError_t launch_rn_lds(const void *x, bool x_is_f32, const double *shift,
                                const double *scale, OT *h, int T, int D, float eps, hipStream_t s,
                                uint8_t *codes, uint8_t *scales) {
  auto go = [&](auto nc_c) {
    constexpr int NC = decltype(nc_c)::value;
    if (x_is_f32) {
      auto k = rmsnorm_modulate_lds_kernel<float, NC, OT, MX>;
      constexpr size_t lds = LdsNorm<float, NC, MX>::lds_bytes;
      hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return e;
      constexpr int nt = LdsNorm<float, NC, MX>::threads;
      hipLaunchKernelGGL(k, dim3(lds_grid(T, nt / 64)), dim3(nt), lds, s, static_cast<const float *>(x),
                         shift, scale, h, T, D, (double)eps, codes, scales);
    } else {
      auto k = rmsnorm_modulate_lds_kernel<bf16, NC, OT, MX>;
      constexpr size_t lds = LdsNorm<bf16, NC, MX>::lds_bytes;
      hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return e;
      constexpr int nt = LdsNorm<bf16, NC, MX>::threads;
      hipLaunchKernelGGL(k, dim3(lds_grid(T, nt / 64)), dim3(nt), lds, s, static_cast<const bf16 *>(x),
                         shift, scale, h, T, D, (double)eps, codes, scales);
    }
    return hipGetLastError();
  };
  const int per_lane = (int)ceil_div(D, 64 * 8);  // 16-byte chunks per lane
  if (per_lane <= 1) return go(std::integral_constant<int, 1>());
  if (per_lane <= 4) return go(std::integral_constant<int, 4>());
  if (per_lane <= 8) return go(std::integral_constant<int, 8>());
  if (per_lane <= 11) return go(std::integral_constant<int, 11>());
  return go(std::integral_constant<int, 16>());
}

template <typename OT>
static hipError_t launch_rn(const void *x, bool x_is_f32, const double *shift, const double *scale,
                            OT *h, int T, int D, float eps, hipStream_t s) {
  if (D <= 8192)
    return launch_rn_lds<OT, false>(x, x_is_f32, shift, scale, h, T, D, eps, s, nullptr, nullptr);
  const int blocks = (int)ceil_div(T, 4);
  const int reg_blocks = (int)ceil_div(T, x_is_f32 ? 4 : 8);  // 4 waves of 1 (fp32) or 2 rows
  auto reg = [&](auto nc_c) {
    constexpr int NC = decltype(nc_c)::value;
    if (x_is_f32)
      hipLaunchKernelGGL((rmsnorm_modulate_reg_kernel<float, NC, OT>), dim3(reg_blocks), dim3(256),
                         0, s, static_cast<const float *>(x), shift, scale, h, T, D, (double)eps);
    else
      hipLaunchKernelGGL((rmsnorm_modulate_reg_kernel<bf16, NC, OT>), dim3(reg_blocks), dim3(256),
                         0, s, static_cast<const bf16 *>(x), shift, scale, h, T, D, (double)eps);
    return hipGetLastError();
  };
  const int per_lane = (int)ceil_div(D, 64 * 8);  // 16-byte chunks per lane
  if (per_lane <= 1) return reg(std::integral_constant<int, 1>());
  if (per_lane <= 4) return reg(std::integral_constant<int, 4>());
  if (per_lane <= 8) return reg(std::integral_constant<int, 8>());
  if (per_lane <= 11) return reg(std::integral_constant<int, 11>());
  if (per_lane <= 16) return reg(std::integral_constant<int, 16>());
  if (x_is_f32)
    hipLaunchKernelGGL((rmsnorm_modulate_kernel<float, OT>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const float *>(x), shift, scale, h, T, D, (double)eps);
  else
    hipLaunchKernelGGL((rmsnorm_modulate_kernel<bf16, OT>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const bf16 *>(x), shift, scale, h, T, D, (double)eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_modulate(const void *x, bool x_is_f32, const double *shift,
                                   const double *scale, void *h, int T, int D, float eps,
                                   hipStream_t s) {
  return launch_rn(x, x_is_f32, shift, scale, static_cast<bf16 *>(h), T, D, eps, s);
}

hipError_t launch_rmsnorm_modulate_mx(const void *x, bool x_is_f32, const double *shift,
                                      const double *scale, void *h, uint8_t *codes,
                                      uint8_t *scales, int T, int D, float eps, hipStream_t s,
                                      bool keep_h) {
  const int per_lane = (int)ceil_div(D, 64 * 8);
  if (D % 128 != 0) return hipErrorInvalidValue;
  if (per_lane > 16) {  // long rows: the two-pass normalisation, then the quantisation
    hipError_t e = launch_rmsnorm_modulate(x, x_is_f32, shift, scale, h, T, D, eps, s);
    if (e != hipSuccess) return e;
    return launch_mxfp8_quantize(h, T, D, codes, scales, s);
  }
  if (!keep_h) h = nullptr;  // only the codes and scales are written
  if (D <= 8192)
    return launch_rn_lds<bf16, true>(x, x_is_f32, shift, scale, static_cast<bf16 *>(h), T, D, eps,
                                     s, codes, scales);
  const int blocks = (int)ceil_div(T, x_is_f32 ? 4 : 8);  // 4 waves of 1 (fp32) or 2 rows
  auto reg = [&](auto nc_c) {
    constexpr int NC = decltype(nc_c)::value;
    if (x_is_f32)
      hipLaunchKernelGGL((rmsnorm_modulate_reg_kernel<float, NC, bf16, true>), dim3(blocks),
                         dim3(256), 0, s, static_cast<const float *>(x), shift, scale,
                         static_cast<bf16 *>(h), T, D, (double)eps, codes, scales);
    else
      hipLaunchKernelGGL((rmsnorm_modulate_reg_kernel<bf16, NC, bf16, true>), dim3(blocks),
                         dim3(256), 0, s, static_cast<const bf16 *>(x), shift, scale,
                         static_cast<bf16 *>(h), T, D, (double)eps, codes, scales);
    return hipGetLastError();
  };
  if (per_lane <= 1) return reg(std::integral_constant<int, 1>());
  if (per_lane <= 4) return reg(std::integral_constant<int, 4>());
  if (per_lane <= 8) return reg(std::integral_constant<int, 8>());
  if (per_lane <= 11) return reg(std::integral_constant<int, 11>());
  return reg(std::integral_constant<int, 16>());
}

hipError_t launch_rmsnorm_modulate_f32out(const void *x, bool x_is_f32, const double *shift,
                                          const double *scale, float *h, int T, int D, float eps,
                                          hipStream_t s) {
  return launch_rn(x, x_is_f32, shift, scale, h, T, D, eps, s);
}

}  // namespace h3dit
