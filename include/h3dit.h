/*
 * h3dit.h - C ABI of the MI355X (gfx950) library for one MiniMax-H3-Image DiT
 * block forward pass over the packed joint sequence of text and image tokens.
 *
 * What one block computes (apxml.com spec page, "Architecture Diagram", read
 * together with the Hugging Face model card, "Model Architecture"):
 *
 *   mod  = W_ada . cond                      -> shift1 scale1 gate1 shift2 scale2 gate2
 *   h1   = rmsnorm(x) * (1 + scale1) + shift1
 *   q,k,v = h1 . W_qkv^T ; q,k rotated by 2D axial RoPE
 *   o    = softmax(q k^T / sqrt(128)) v      (per head, all tokens, no mask)
 *   x1   = x + gate1 * (o . W_o^T)
 *   h2   = rmsnorm(x1) * (1 + scale2) + shift2
 *   out  = x1 + gate2 * (gelu_tanh(h2 . W_up^T) . W_down^T)
 *
 * Conventions fixed here where the pages are silent: no biases; RMSNorm has
 * no learned weight; RoPE rotates adjacent pairs (2i, 2i+1), dims 0..63 by
 * the row position and 64..127 by the column position, with frequency
 * rope_base^(-2i/64); text tokens use position (0, 0); GELU is the tanh form.
 *
 * Precision: weights and matrix-core operands are bf16 (round to nearest
 * even); products accumulate in fp32; the modulation vector and both
 * normalisations are computed in fp64; x1 and the output are fp32. The
 * stored query carries the softmax factor: q = bf16(rope(q) * log2(e)/sqrt(128)),
 * rounded once, so a score s = q.k is a base-2 exponent; the attention
 * weights are bf16(2^(s - m)) for an integer shift m per query, normalised by
 * their own sum. Since scaling by a power of two commutes with the rounding,
 * the result is that of m = the rounded-up maximum score for values of
 * magnitude 2^-94..2^32 (the kernel takes the first key tile's rounded-up
 * maximum plus 32, or the exact one when a weight would exceed about 2^72;
 * weights more than 2^94 below a row's largest may underflow to zero).
 *
 * Memory: every pointer argument is a DEVICE pointer unless marked (host);
 * matrices are row-major and dense; the caller owns all memory, including the
 * workspace; the library allocates nothing and keeps no device state.
 * Every device pointer must be 16-byte aligned.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns at once. Outputs are valid once the stream
 * has been synchronised. Device faults surface at the next synchronisation.
 *
 * Errors: every argument check runs on the host before any HIP call; a
 * failing check returns a negative h3dit_status and leaves all memory
 * untouched. h3dit_last_error() then describes the failure (thread-local).
 * A failed kernel launch returns H3DIT_EHIP. There is no CPU fallback.
 *
 * Threads: calls are reentrant for distinct workspaces / outputs.
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    H3DIT_OK = 0,
    H3DIT_EINVAL = -1,       /* null pointer, bad size, bad enum value          */
    H3DIT_EUNSUPPORTED = -2, /* valid but unsupported shape (e.g. head_dim != 128) */
    H3DIT_EWORKSPACE = -3,   /* workspace smaller than h3dit_workspace_size()   */
    H3DIT_EALIGN = -4,       /* a device pointer is not 16-byte aligned         */
    H3DIT_EHIP = -5          /* a HIP launch reported an error                  */
} h3dit_status;

typedef enum { H3DIT_BF16 = 0, H3DIT_F32 = 1 } h3dit_dtype;

/* Block shape (host struct). D = hidden, A = heads * head_dim, F = ffn, T = n_tokens.
 * Requirements: head_dim == 128; hidden, ffn multiples of 64; heads >= 1;
 * 1 <= n_tokens <= 1048576; hidden <= 65536; eps >= 0; rope_base > 0. */
typedef struct {
    int32_t hidden;     /* D: model width (5376 for the full-width block)            */
    int32_t heads;      /* H: attention heads (56)                                    */
    int32_t head_dim;   /* must be 128                                                */
    int32_t ffn;        /* F: MLP inner width (14336)                                 */
    int32_t n_tokens;   /* T: joint sequence length (text + image tokens)             */
    int32_t x_dtype;    /* h3dit_dtype of the block input x                           */
    float eps;          /* RMSNorm epsilon (1e-6)                                     */
    float rope_base;    /* RoPE base (10000)                                          */
} h3dit_config;

/* Block weights (host struct of device pointers), all bf16 row-major [out, in]. */
typedef struct {
    const void *w_ada;  /* [6D, D]  rows: shift1 | scale1 | gate1 | shift2 | scale2 | gate2 */
    const void *w_qkv;  /* [3A, D]  rows: q | k | v, each head-major (head h = rows h*128..) */
    const void *w_o;    /* [D, A]                                                         */
    const void *w_up;   /* [F, D]                                                         */
    const void *w_down; /* [D, F]                                                         */
} h3dit_weights;

/* Bytes of device workspace h3dit_block_forward needs for this shape.
 * Host-only; no HIP call. Returns H3DIT_OK and writes *bytes. */
int h3dit_workspace_size(const h3dit_config *cfg, size_t *bytes);

/* One DiT block forward (all nine steps of the block).
 *   x          [T, D], dtype cfg->x_dtype (bf16 or fp32)
 *   cond       [D] fp32 conditioning vector (the timestep embedding)
 *   w          weights (see h3dit_weights)
 *   positions  [T, 2] int32 RoPE positions (row, col); every int32 value is
 *              accepted (each becomes an fp64 angle; no range makes the
 *              kernels fail), so positions are not range-checked: a check
 *              would need a device-to-host copy and a synchronisation
 *   out        [T, D] fp32; must not overlap x or the workspace
 *   workspace  >= h3dit_workspace_size() bytes; contents are scratch
 */
int h3dit_block_forward(const h3dit_config *cfg, const void *x, const float *cond,
                        const h3dit_weights *w, const int32_t *positions, float *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the library's static device scratch used by h3dit_block_forward_noalloc. */
#define H3DIT_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* h3dit_block_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result, bitwise, with the
 * workspace taken from a static device array of H3DIT_NOALLOC_SCRATCH_BYTES
 * (256 MiB) that each GPU the library runs on holds until the process ends.
 * The call allocates nothing. Shapes whose h3dit_workspace_size() exceeds
 * that size return H3DIT_EWORKSPACE before any HIP call (at full width,
 * hidden 5376, from 1,521 tokens on, though some larger counts fit again as
 * the GEMMs' K-slice scratch varies with the token count:
 * h3dit_workspace_size() decides). The array belongs to the
 * current device (hipSetDevice), which must be the device of `stream`; calls
 * on one GPU share it, so two calls that overlap in time on the same GPU (on
 * different streams, or from different threads) race: order them on one
 * stream. Nothing in the array needs to start at zero. */
int h3dit_block_forward_noalloc(const h3dit_config *cfg, const void *x, const float *cond,
                                const h3dit_weights *w, const int32_t *positions, float *out,
                                void *stream);

/* Same as h3dit_block_forward, and records caller-created hipEvent_t handles
 * between the stages: events[i] is recorded on `stream` before stage i and
 * events[9] after the last, for stages (0) modulation, (1) RoPE table,
 * (2) RMSNorm1, (3) QKV+RoPE GEMM, (4) attention, (5) output projection,
 * (6) RMSNorm2, (7) MLP up + GELU, (8) MLP down. n_events must be 10. */
int h3dit_block_forward_timed(const h3dit_config *cfg, const void *x, const float *cond,
                              const h3dit_weights *w, const int32_t *positions, float *out,
                              void *workspace, size_t workspace_bytes, void *stream,
                              void *const *events, int n_events);

/* Where a block forward keeps its intermediate tensors in the workspace
 * (byte offsets from the workspace start; host-only). After h3dit_block_forward
 * (linears = 0) or h3dit_block_forward_mxfp8 (linears = 1) has completed, the
 * workspace holds: mod (fp64 [6D]), table (fp32 [T, 64, 2] RoPE cos/sin), h
 * (bf16 [T, D], the second normalisation's h2), qk (bf16 [T, 2A], q rotated
 * and scaled, then k rotated), vt (bf16 [H, 128, Tp], V transposed, token t in
 * the column described at h3dit_qkv_rope, zero past T), o (bf16 [T, A]), x1
 * (fp32 [T, D]) and u (bf16 [T, F]). For inspection and tests; the contents
 * are only defined between forwards on the same workspace. */
typedef struct {
    size_t mod, table, h, qk, vt, o, x1, u;
    /* MXFP8 forward only (0 otherwise): h2 and u as MXFP8 codes ([T, D] and
     * [T, F]) and their scales, in the layout of h3dit_mxfp8_quantize */
    size_t q_h2, q_h2_scale, q_u, q_u_scale;
} h3dit_workspace_map;

int h3dit_workspace_layout(const h3dit_config *cfg, int32_t linears, h3dit_workspace_map *map);

/* ---------------------------------------------------------------------------
 * Stage entry points: the same kernels that h3dit_block_forward runs, one
 * step at a time, for per-step parity checks and profiling. Shapes come from
 * cfg; layouts are the workspace layouts named below.
 * ------------------------------------------------------------------------- */

/* Step 1, AdaLN modulation (spec page diagram, "AdaLN Modulation"):
 * mod[6D] fp64 = W_ada[6D, D] (bf16) . cond[D] (fp32), fp64 accumulation. */
int h3dit_modulation(const h3dit_config *cfg, const void *w_ada, const float *cond,
                     double *mod, void *stream);

/* Step 1 for n conditioning vectors at once (AdaLN caching; vLLM blog, "Faster
 * DiT": the conditioning projections are precomputed once per request):
 *   conds [n, D] fp32, mods [n, 6D] fp64 (caller-owned, 16-byte aligned);
 *   mods[s] is bitwise what h3dit_modulation returns for conds[s], while each
 *   weight is read once per 8 vectors. 1 <= n <= 4096. */
int h3dit_modulation_table(const h3dit_config *cfg, const void *w_ada, const float *conds,
                           int n, double *mods, void *stream);

/* Steps 2 and 7, RMSNorm + modulation (spec page, "Specifications": RMS
 * Normalization; "Architecture Diagram": "AdaLN Modulation", scale and shift):
 * h[T, D] bf16 = bf16( x / sqrt(mean(x^2) + eps) * (1 + scale) + shift ),
 * computed in fp64; x is [T, D] of dtype x_dtype; shift, scale are fp64 [D]. */
int h3dit_rmsnorm_modulate(const h3dit_config *cfg, const void *x, int32_t x_dtype,
                           const double *shift, const double *scale, void *h, void *stream);

/* RoPE table for step 4 (model card, "Model Architecture": multimodal RoPE, read
 * as 2D axial; spec page, "Architecture Diagram": "Pos: RoPE"):
 * table[T, 64, 2] fp32: (cos, sin) of positions[t][j / 32] * rope_base^(-(j % 32)/32),
 * evaluated in fp64. */
int h3dit_rope_table(const h3dit_config *cfg, const int32_t *positions, float *table,
                     void *stream);

/* Steps 3 + 4, QKV projection with RoPE in the epilogue (spec page, "Architecture
 * Diagram": the attention block's Q, K, V projections and "Pos: RoPE"; model card,
 * "Model Architecture": 56 query and 56 key-value heads of 128, multimodal RoPE,
 * read as 2D axial):
 *   h [T, D] bf16, w_qkv [3A, D] bf16, table from h3dit_rope_table.
 *   qk [T, 2A] bf16: columns 0..A-1 = bf16(rope(q) * log2(e)/sqrt(128)),
 *      columns A..2A-1 = bf16(rope(k)); q and k are the fp32 products, rounded
 *      once after the rotation.
 *   vt [H, 128, Tp] bf16 with Tp = h3dit_padded_tokens(T): v transposed per head;
 *      the value of token t sits in column c(t) = (t & ~28) | ((t & 12) << 1)
 *      | ((t & 16) >> 2), i.e. bits 4, 3, 2 of t moved to bits 2, 4, 3 within
 *      each group of 32 tokens (the order in which the attention kernel's
 *      matrix-core fragments take keys); columns of tokens T..Tp-1 are written
 *      as zero. */
int h3dit_qkv_rope(const h3dit_config *cfg, const void *h, const void *w_qkv, const float *table,
                   void *qk, void *vt, void *stream);

/* Step 5, joint bidirectional attention over all T tokens, no mask (model card,
 * "Model Architecture": text and image tokens in one packed sequence of a
 * single-stream transformer; spec page, "Architecture Diagram": "Joint /
 * Cross-Attention"):
 *   qk, vt as written by h3dit_qkv_rope (q pre-scaled, so softmax(q.k) in base 2);
 *   o [T, A] bf16 (head h = columns h*128..). */
int h3dit_attention(const h3dit_config *cfg, const void *qk, const void *vt, void *o,
                    void *stream);

/* Step 6, output projection + gated residual (spec page, "Architecture Diagram":
 * the attention branch's output projection scaled by gate1 of the AdaLN
 * modulation and added to the residual stream, "+"):
 *   x1[T, D] fp32 = resid + gate * (o[T, A] . w_o[D, A]^T); resid is [T, D] of
 *   dtype resid_dtype; gate fp64 [D]. */
int h3dit_out_proj_residual(const h3dit_config *cfg, const void *o, const void *w_o,
                            const void *resid, int32_t resid_dtype, const double *gate,
                            float *x1, void *stream);

/* Step 8, MLP up-projection + tanh-GELU (spec page, "Architecture Diagram":
 * "Feed-Forward (MLP) GELU Intermediate: 14.3k"; model card, "Model
 * Architecture": FFN width 14336):
 *   u[T, F] bf16 = bf16(gelu_tanh(h2[T, D] . w_up[F, D]^T)). */
int h3dit_mlp_up_gelu(const h3dit_config *cfg, const void *h2, const void *w_up, void *u,
                      void *stream);

/* Step 9, MLP down-projection + gated residual (spec page, "Architecture
 * Diagram": the MLP branch scaled by gate2 and added to the residual stream, "+"):
 *   out[T, D] fp32 = x1 + gate * (u[T, F] . w_down[D, F]^T); x1 fp32, gate fp64 [D]. */
int h3dit_mlp_down_residual(const h3dit_config *cfg, const void *u, const void *w_down,
                            const float *x1, const double *gate, float *out, void *stream);

/* The matrix-core GEMM that the four projections share, with a plain fp32
 * epilogue (for tests and profiling):
 *   y[M, N] fp32 = x[M, K] (bf16) . w[N, K]^T (bf16), fp32 accumulation.
 * Requirements: M, N >= 1; K a positive multiple of 64. */
int h3dit_linear_f32(const void *x, const void *w, int32_t M, int32_t N, int32_t K, float *y,
                     void *stream);

/* ---------------------------------------------------------------------------
 * MXFP8 linears (vLLM blog "H3-Image Day-0 Support", section Inference
 * Optimizations: the DiT's linears run in MXFP8; element and block formats
 * from the OCP 8-bit floating point and Microscaling definitions).
 *
 * An MXFP8 matrix [rows, K] (K a multiple of 128) is a pair:
 *   codes  [rows, K] uint8, row-major: OCP FP8 E4M3 (bias 7, largest finite
 *          448, S.1111.111 is NaN and is never produced);
 *   scales h3dit_mxfp8_scale_bytes(rows, K) bytes of E8M0 exponents (byte
 *          X + 127 means 2^X), one per 32 consecutive K of a row, grouped in
 *          1 KB blocks: block (p, t) covers rows 256 p .. 256 p + 255 and K
 *          128 t .. 128 t + 127 and starts at byte (p * K / 128 + t) * 1024;
 *          inside it the scale of row 256 p + 16 b + r (b, r < 16) and of K
 *          block kb (< 4) is byte (kb * 16 + r) * 16 + b. Rows of the last
 *          block past `rows` hold byte 0.
 * The value of element (i, k) is e4m3(codes[i, k]) * 2^(scale - 127).
 *
 * Quantisation (h3dit_mxfp8_quantize): X = floor(log2(max |v| of the 32-block))
 * - 8, or -127 for an all-zero block; each element is v * 2^-X rounded to the
 * nearest E4M3 value, ties to even, saturating at +-448, sign kept on zero.
 * Inputs must be finite.
 * ------------------------------------------------------------------------- */

/* MXFP8 block weights (host struct of device pointers): each linear of
 * h3dit_weights as codes + scales, quantised from the bf16 weight with
 * h3dit_mxfp8_quantize ([out, in] rows, K = in). */
typedef struct {
    const uint8_t *w_qkv, *w_qkv_scale;   /* [3A, D] */
    const uint8_t *w_o, *w_o_scale;       /* [D, A]  */
    const uint8_t *w_up, *w_up_scale;     /* [F, D]  */
    const uint8_t *w_down, *w_down_scale; /* [D, F]  */
} h3dit_mxfp8_weights;

/* Bytes of the scale array of an MXFP8 matrix [rows, K] (host-only):
 * ceil(rows / 256) * 256 * K / 32; 0 if rows < 1 or K is not a positive
 * multiple of 128. */
size_t h3dit_mxfp8_scale_bytes(int64_t rows, int64_t K);

/* codes + scales (layout above) of the bf16 matrix x [rows, K].
 * rows in [1, 2^31), K a multiple of 128 in [128, 2^20]. */
int h3dit_mxfp8_quantize(const void *x, int64_t rows, int64_t K, uint8_t *codes,
                         uint8_t *scales, void *stream);

/* Step 5 for the MXFP8 output projection (vLLM blog "H3-Image Day-0
 * Support", section Inference Optimizations: the DiT linears in MXFP8):
 * h3dit_attention (same o, bitwise), and in the same pass o's MXFP8 codes
 * [T, A] and scales (layout above, h3dit_mxfp8_scale_bytes(T, A) bytes),
 * bitwise equal to h3dit_mxfp8_quantize of that o. */
int h3dit_attention_mxfp8(const h3dit_config *cfg, const void *qk, const void *vt, void *o,
                          uint8_t *o_codes, uint8_t *o_scales, void *stream);

/* y[M, N] fp32 = X . W^T for MXFP8 operands X [M, K] and W [N, K] (codes +
 * scales as above), fp32 accumulation in the matrix cores' scaled E4M3
 * product. N % 4 == 0, K a multiple of 128. */
int h3dit_linear_mxfp8(const uint8_t *x_codes, const uint8_t *x_scales, const uint8_t *w_codes,
                       const uint8_t *w_scales, int32_t M, int32_t N, int32_t K, float *y,
                       void *stream);

/* Workspace of h3dit_block_forward_mxfp8 for this shape (host-only). */
int h3dit_workspace_size_mxfp8(const h3dit_config *cfg, size_t *bytes);

/* h3dit_block_forward with the four linears in MXFP8: h1, o, h2 and u (the
 * bf16 tensors of the bf16 path) are quantised along K just before their
 * linear, and the weights come from q. w supplies only w_ada (its other
 * pointers are not read). hidden and ffn must be multiples of 128. Attention,
 * the normalisations, RoPE, GELU and the residuals are as in the bf16 path. */
int h3dit_block_forward_mxfp8(const h3dit_config *cfg, const void *x, const float *cond,
                              const h3dit_weights *w, const h3dit_mxfp8_weights *q,
                              const int32_t *positions, float *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Same, recording the 10 events of h3dit_block_forward_timed (each linear's
 * phase includes the quantisation of its input). */
int h3dit_block_forward_mxfp8_timed(const h3dit_config *cfg, const void *x, const float *cond,
                                    const h3dit_weights *w, const h3dit_mxfp8_weights *q,
                                    const int32_t *positions, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream, void *const *events,
                                    int n_events);

/* ---------------------------------------------------------------------------
 * The DiT stack around the blocks (model card, "Model Architecture": latents
 * cut into patches become the image tokens of the packed sequence; spec page,
 * "Specifications": 50 layers). One DiT evaluation, for a latent [C, H, W]
 * with patch size p (gh = H / p, gw = W / p image-token rows and columns):
 *   patch(t)[c*p*p + dy*p + dx] = latent[c, gy*p + dy, gx*p + dx],  t = gy*gw + gx
 *   x        = [ text ; patch . w_patch^T ]                  fp32 [T, D]
 *   x        = block_{n-1}( ... block_0(x) ... ), every block with the same cond
 *   (shift, scale) = w_ada_final . cond                      (fp64, like the blocks)
 *   vt(t)    = (rmsnorm(x_img(t)) * (1 + scale) + shift) . w_final^T   fp32, image tokens
 *   v[c, y, x] = vt(t of (y / p, x / p))[c*p*p + (y % p)*p + x % p]
 * The patch embedding and the final projection are fp32 (no matrix-core
 * rounding); the blocks run exactly as h3dit_block_forward with fp32 x.
 * ------------------------------------------------------------------------- */
typedef struct {
    int32_t n_blocks;     /* number of blocks (50 for the full model; 0 allowed)        */
    int32_t channels;     /* C: latent channels (24)                                    */
    int32_t patch;        /* p: patch size (2)                                          */
    int32_t grid_h;       /* gh: image-token rows                                       */
    int32_t grid_w;       /* gw: image-token columns                                    */
    int32_t text_tokens;  /* text tokens at the front of the sequence                   */
} h3dit_stack_config;

typedef struct {
    const float *w_patch;        /* fp32 [D, C*p*p]                                     */
    const void *w_ada_final;     /* bf16 [2D, D]  rows: shift | scale                   */
    const float *w_final;        /* fp32 [C*p*p, D]                                     */
    const h3dit_weights *blocks; /* host array of n_blocks block weight sets            */
} h3dit_stack_weights;

/* Bytes of device workspace h3dit_dit_forward needs (host-only, no HIP call).
 * cfg->n_tokens must equal text_tokens + grid_h * grid_w; C*p*p must be a
 * multiple of 4. */
int h3dit_stack_workspace_size(const h3dit_config *cfg, const h3dit_stack_config *st,
                               size_t *bytes);

/* One DiT evaluation (see above).
 *   latent     [C, gh*p, gw*p] fp32
 *   text       [text_tokens, D] fp32 (may be NULL when text_tokens == 0)
 *   cond       [D] fp32
 *   positions  [T, 2] int32 RoPE positions of the packed sequence
 *   v          [C, gh*p, gw*p] fp32; must not overlap the workspace
 * cfg->x_dtype is ignored (the residual stream between blocks is fp32). */
int h3dit_dit_forward(const h3dit_config *cfg, const h3dit_stack_config *st,
                      const h3dit_stack_weights *w, const float *latent, const float *text,
                      const float *cond, const int32_t *positions, float *v, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Every block's modulation and the final layer's for n_steps denoising steps,
 * one pass over each AdaLN weight (AdaLN caching, as for h3dit_modulation_table):
 *   conds [n_steps, D] fp32 (one conditioning vector per step);
 *   table [n_steps][n_blocks + 1][6D] fp64, caller-owned: entry [s][b] for
 *   b < n_blocks is block b's modulation for conds[s], entry [s][n_blocks] holds
 *   the final layer's (shift, scale) in its first 2D values (the rest is left
 *   untouched). w->w_patch, w->w_final and the blocks' other weights are not read.
 * 1 <= n_steps <= 4096. */
int h3dit_dit_modulation_table(const h3dit_config *cfg, const h3dit_stack_config *st,
                               const h3dit_stack_weights *w, const float *conds, int n_steps,
                               double *table, void *stream);

/* h3dit_dit_forward with the modulation taken from one step's row of the table
 * above (mods = table + s * (n_blocks + 1) * 6D) instead of computed from cond;
 * the blocks' w_ada and w->w_ada_final are not read. The result is bitwise that
 * of h3dit_dit_forward with conds[s]. */
int h3dit_dit_forward_mod(const h3dit_config *cfg, const h3dit_stack_config *st,
                          const h3dit_stack_weights *w, const float *latent, const float *text,
                          const double *mods, const int32_t *positions, float *v, void *workspace,
                          size_t workspace_bytes, void *stream);

/* The DiT evaluation with every block's four linears in MXFP8 (vLLM blog "H3-Image
 * Day-0 Support", section Inference Optimizations: MXFP8 GEMMs for the DiT's
 * linears). q holds st->n_blocks entries, block l's weights quantised with
 * h3dit_mxfp8_quantize; w->blocks[l] then supplies only w_ada (and is not read
 * at all by the _mod form). hidden and ffn must be multiples of 128. The patch
 * embedding and final projection stay fp32. Workspace from
 * h3dit_stack_workspace_size_mxfp8 (host-only). q may be NULL when n_blocks is 0. */
int h3dit_stack_workspace_size_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                                     size_t *bytes);
int h3dit_dit_forward_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                            const h3dit_stack_weights *w, const h3dit_mxfp8_weights *q,
                            const float *latent, const float *text, const float *cond,
                            const int32_t *positions, float *v, void *workspace,
                            size_t workspace_bytes, void *stream);
int h3dit_dit_forward_mod_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                                const h3dit_stack_weights *w, const h3dit_mxfp8_weights *q,
                                const float *latent, const float *text, const double *mods,
                                const int32_t *positions, float *v, void *workspace,
                                size_t workspace_bytes, void *stream);

/* latent[i] += dt * v[i] for i < n (fp32): the explicit Euler update between
 * denoising steps. */
int h3dit_latent_step(float *latent, const float *v, float dt, int64_t n, void *stream);

/* Padded token count used by the vt layout (T rounded up to a multiple of 64). */
int64_t h3dit_padded_tokens(int64_t n_tokens);

/* Human-readable name of a status code (static string). */
const char *h3dit_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *h3dit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* H3DIT_H */
