// Internal launchers of the gfx950 kernels (C++ linkage, not exported).
// Each returns the hipError_t of its launch; shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3dit {

// mod[rows] (fp64) = w[rows, cols] (bf16) . cond[cols] (fp32); cols % 8 == 0
hipError_t launch_modulation(const void *w, const float *cond, double *mod, int rows, int cols,
                             hipStream_t s);

// mods[k * mod_stride + r] = (W . conds[k])[r] for k < n, each bitwise equal to
// launch_modulation with conds[k] (W read once per 8 vectors)
hipError_t launch_modulation_multi(const void *w, const float *conds, int n, double *mods,
                                   int64_t mod_stride, int rows, int cols, hipStream_t s);

// h[T, D] (bf16) = bf16(rmsnorm(x) * (1 + scale) + shift), fp64 math; D % 8 == 0
hipError_t launch_rmsnorm_modulate(const void *x, bool x_is_f32, const double *shift,
                                   const double *scale, void *h, int T, int D, float eps,
                                   hipStream_t s);

// same, and the bf16 output also as MXFP8 codes [T, D] + scales (D % 128 == 0);
// with keep_h false h may not be written (it is still needed as scratch for
// rows longer than 8192)
hipError_t launch_rmsnorm_modulate_mx(const void *x, bool x_is_f32, const double *shift,
                                      const double *scale, void *h, uint8_t *codes,
                                      uint8_t *scales, int T, int D, float eps, hipStream_t s,
                                      bool keep_h = true);

// same, fp32 output (the final layer of the DiT stack)
hipError_t launch_rmsnorm_modulate_f32out(const void *x, bool x_is_f32, const double *shift,
                                          const double *scale, float *h, int T, int D, float eps,
                                          hipStream_t s);

// table[T, 64] float2 (cos, sin)
hipError_t launch_rope_table(const int32_t *pos, float *table, int T, float base, hipStream_t s);

enum GemmEpilogue {
  EPI_QKV_ROPE = 0,
  EPI_RESID_BF16 = 1,
  EPI_RESID_F32 = 2,
  EPI_GELU = 3,
  EPI_F32 = 4,
  EPI_GELU_MX = 5  // EPI_GELU, and u also as MXFP8 codes + scales (MXFP8 GEMM only)
};

struct GemmArgs {
  const void *x;      // B operand rows: activations [M, K] bf16 (MXFP8: E4M3 codes)
  const void *w;      // A operand rows: weights [N, K] bf16 (MXFP8: E4M3 codes)
  const uint8_t *x_scale;  // MXFP8 only: E8M0 scales of x and w in the 1 KB
  const uint8_t *w_scale;  // block layout of launch_mxfp8_quantize
  int M, N, K;
  // epilogue operands
  void *out;          // QKV: qk [M, 2A]; RESID, F32: fp32 [M, N]; GELU: bf16 [M, N]
  void *out2;         // QKV: vt [H, 128, Mp]
  const void *resid;  // RESID: [M, N] bf16 or fp32
  const double *gate; // RESID: [N]
  const float *table; // QKV: rope table [M, 64] float2
  int A;              // QKV: attention width
  int Mp;             // QKV: padded token count of vt
  uint8_t *out_codes;   // GELU_MX: u as E4M3 codes [M, N]
  uint8_t *out_scales;  // GELU_MX: u's scales (1 KB block layout, K = N)
  // Optional scratch for splitting the last, partial wave of tiles along K
  // (nullptr: never split). Set by the caller; split and full_tiles are
  // filled in by launch_gemm.
  float *partial;
  size_t partial_bytes;
  int split;          // K slices per tile of the last wave (<= 1: no split)
  int full_tiles;     // tiles computed whole before the split ones
};

// Launches the GEMM and, when the last wave of tiles is split along K, the
// kernel that adds the slices and applies the epilogue.
hipError_t launch_gemm(GemmEpilogue epi, const GemmArgs &a, hipStream_t s);

// Scratch bytes that let launch_gemm split the last wave of an M x N x K GEMM
// on a 256-CU device (0: it would not split).
size_t gemm_split_scratch_bytes(int64_t M, int64_t N, int64_t K);

// The same GEMM with MXFP8 operands (E4M3 codes, one E8M0 scale per 32 along
// K); K % 128 == 0. Same epilogues, split and fixup as launch_gemm.
hipError_t launch_gemm_mx(GemmEpilogue epi, const GemmArgs &a, hipStream_t s);
size_t gemm_mx_split_scratch_bytes(int64_t M, int64_t N, int64_t K);

// codes [rows, K] + scales (1 KB per 256-row panel and 128-wide K tile) from
// bf16 x [rows, K]; K % 128 == 0
hipError_t launch_mxfp8_quantize(const void *x, int rows, int K, uint8_t *codes, uint8_t *scales,
                                 hipStream_t s);

// o[T, A] = attention over qk [T, 2A] and vt [H, 128, Tp]. With scratch
// (part, at least attention_split_scratch_bytes(T, H) bytes) the last, partial
// round of workgroups may be cut along the keys and merged by a second kernel.
hipError_t launch_attention(const void *qk, const void *vt, void *o, int T, int H, int Tp,
                            hipStream_t s, float *part = nullptr, size_t part_bytes = 0);
size_t attention_split_scratch_bytes(int T, int H);
// The same, o also as MXFP8 codes [T, H * 128] and scales (mxfp8_quantize layout);
// o may be null (then only the codes and scales are written).
hipError_t launch_attention_mx(const void *qk, const void *vt, void *o, uint8_t *o_codes,
                               uint8_t *o_scales, int T, int H, int Tp, hipStream_t s);

// ---- DiT stack (patch-embed, final layer, latent update) ----

// patches[gh * gw, C * p * p] fp32 from latent [C, gh * p, gw * p] fp32; token t = gy * gw + gx,
// feature c * p * p + dy * p + dx
hipError_t launch_patchify(const float *latent, float *patches, int C, int p, int gh, int gw,
                           hipStream_t s);

// latent-shaped v [C, gh * p, gw * p] from per-token rows vt [gh * gw, C * p * p] (inverse of
// patchify)
hipError_t launch_unpatchify(const float *vt, float *v, int C, int p, int gh, int gw,
                             hipStream_t s);

// y[M, N] (row stride ldy) = a[M, K] . b[N, K]^T, all fp32; K % 4 == 0
hipError_t launch_gemm_f32(const float *a, const float *b, float *y, int M, int N, int K, int ldy,
                           hipStream_t s);

// latent[i] += dt * v[i], i < n
hipError_t launch_latent_step(float *latent, const float *v, float dt, int64_t n, hipStream_t s);

}  // namespace h3dit
