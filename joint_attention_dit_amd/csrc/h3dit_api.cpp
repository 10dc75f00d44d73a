// C ABI of the DiT block library: argument validation, workspace plan and the
// order in which the block's kernels are enqueued (apxml.com spec page,
// "Architecture Diagram": modulation, RMSNorm, attention, residual,
// modulation, RMSNorm, GELU MLP, residual).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/h3dit.h"
#include "kernels.h"

using namespace h3dit;

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return H3DIT_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(H3DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Test hook: H3DIT_FAULT_INJECT=launch makes every launch report failure
// before anything is enqueued, so the error path can be exercised on a host.
bool fault_injected() {
  const char *v = getenv("H3DIT_FAULT_INJECT");
  return v && strcmp(v, "launch") == 0;
}

int check_config(const h3dit_config *cfg) {
  if (!cfg) return fail(H3DIT_EINVAL, "cfg is NULL");
  if (cfg->head_dim != 128)
    return fail(H3DIT_EUNSUPPORTED, "head_dim must be 128 (got %d)", cfg->head_dim);
  if (cfg->heads < 1) return fail(H3DIT_EINVAL, "heads must be >= 1 (got %d)", cfg->heads);
  if (cfg->hidden < 64 || cfg->hidden % 64 != 0 || cfg->hidden > 65536)
    return fail(H3DIT_EUNSUPPORTED, "hidden must be a multiple of 64 in [64, 65536] (got %d)",
                cfg->hidden);
  if (cfg->ffn < 64 || cfg->ffn % 64 != 0 || cfg->ffn > 262144)
    return fail(H3DIT_EUNSUPPORTED, "ffn must be a multiple of 64 in [64, 262144] (got %d)",
                cfg->ffn);
  if ((int64_t)cfg->heads * 128 > 65536)
    return fail(H3DIT_EUNSUPPORTED, "heads * 128 must be <= 65536 (got %d heads)", cfg->heads);
  if (cfg->n_tokens < 1 || cfg->n_tokens > (1 << 20))
    return fail(H3DIT_EINVAL, "n_tokens must be in [1, 1048576] (got %d)", cfg->n_tokens);
  if (cfg->x_dtype != H3DIT_BF16 && cfg->x_dtype != H3DIT_F32)
    return fail(H3DIT_EINVAL, "x_dtype must be H3DIT_BF16 or H3DIT_F32 (got %d)", cfg->x_dtype);
  if (!(cfg->eps >= 0.0f) || !(cfg->eps < 1.0f))
    return fail(H3DIT_EINVAL, "eps must be in [0, 1)");
  if (!(cfg->rope_base > 1.0f) || !(cfg->rope_base < 1e30f))
    return fail(H3DIT_EINVAL, "rope_base must be > 1");
  return H3DIT_OK;
}

#define CHECK_PTR(p)                                                        \
  do {                                                                      \
    if (!(p)) return fail(H3DIT_EINVAL, "%s is NULL", #p);                  \
    if (!aligned16(p)) return fail(H3DIT_EALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

#define CHECK_CFG(cfg)                  \
  do {                                  \
    const int st_ = check_config(cfg);  \
    if (st_ != H3DIT_OK) return st_;    \
  } while (0)

#define LAUNCH(expr, what)                                          \
  do {                                                              \
    if (fault_injected()) return fail(H3DIT_EHIP, "%s: injected launch fault", what); \
    const hipError_t e_ = (expr);                                   \
    if (e_ != hipSuccess) return hip_fail(e_, what);                \
  } while (0)

struct Plan {
  int64_t T, D, A, H, F, Tp;
  size_t mod, table, h, qk, vt, o, x1, u, split, split_bytes, att, att_bytes, total;
  // MXFP8: codes and scales of the linears' inputs: region a holds h1, then o,
  // then h2; region b holds u (written while h2's codes are being read)
  size_t qa, qas, qb, qbs;
};

size_t mx_scale_bytes(int64_t rows, int64_t K) {
  return (size_t)((rows + 255) / 256) * 256 * (size_t)(K / 32);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Plan make_plan(const h3dit_config *c, bool mx = false) {
  Plan p;
  p.T = c->n_tokens;
  p.D = c->hidden;
  p.H = c->heads;
  p.A = p.H * 128;
  p.F = c->ffn;
  p.Tp = h3dit_padded_tokens(p.T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  p.mod = take(sizeof(double) * 6 * p.D);
  p.table = take(sizeof(float) * 128 * p.T);
  p.h = take(2 * p.T * p.D);
  p.qk = take(2 * p.T * 2 * p.A);
  p.vt = take(2 * p.A * p.Tp);
  p.o = take(2 * p.T * p.A);
  p.x1 = take(4 * p.T * p.D);
  p.u = take(2 * p.T * p.F);
  // K slices of the four GEMMs' last waves (one GEMM at a time)
  auto split_bytes = mx ? gemm_mx_split_scratch_bytes : gemm_split_scratch_bytes;
  p.split_bytes = std::max(std::max(split_bytes(p.T, 3 * p.A, p.D), split_bytes(p.T, p.D, p.A)),
                           std::max(split_bytes(p.T, p.F, p.D), split_bytes(p.T, p.D, p.F)));
  p.split = take(p.split_bytes);
  // key-range pieces of the attention's last round of workgroups (bf16 path)
  p.att_bytes = mx ? 0 : attention_split_scratch_bytes((int)p.T, (int)p.H);
  p.att = take(p.att_bytes);
  p.qa = p.qas = p.qb = p.qbs = 0;
  if (mx) {
    const int64_t ka = std::max(p.D, p.A);
    p.qa = take((size_t)(p.T * ka));
    p.qas = take(mx_scale_bytes(p.T, ka));
    p.qb = take((size_t)(p.T * p.F));
    p.qbs = take(mx_scale_bytes(p.T, p.F));
  }
  p.total = off;
  return p;
}

template <typename T>
T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

GemmArgs gemm_args(const void *x, const void *w, int64_t M, int64_t N, int64_t K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.x = x;
  g.w = w;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  return g;
}

// mod_in: the block's modulation (fp64 [6D]) computed beforehand, or NULL to
// compute it from cond and w->w_ada.
// q: MXFP8 weights (the four linears in MXFP8; w's linear weights unused), or
// NULL for the bf16 linears.
int forward_impl(const h3dit_config *cfg, const void *x, const float *cond, const h3dit_weights *w,
                 const int32_t *positions, float *out, void *ws, size_t ws_bytes, void *stream,
                 void *const *events, int n_events, const double *mod_in = nullptr,
                 const h3dit_mxfp8_weights *q = nullptr, bool lean = false,
                 bool table_ready = false) {
  // lean (MXFP8 only): the producers write only the codes the next linear
  // consumes, not the bf16 copies of h1, o, h2 and u kept for inspection.
  // table_ready: the workspace's RoPE table region already holds the table of
  // these positions (the DiT stack computes it once for all its blocks).
  CHECK_CFG(cfg);
  if (!w) return fail(H3DIT_EINVAL, "w is NULL");
  CHECK_PTR(x);
  CHECK_PTR(positions);
  CHECK_PTR(out);
  CHECK_PTR(ws);
  if (!mod_in) {
    CHECK_PTR(cond);
    CHECK_PTR(w->w_ada);
  }
  if (q) {
    if (cfg->hidden % 128 != 0 || cfg->ffn % 128 != 0)
      return fail(H3DIT_EUNSUPPORTED, "MXFP8 linears need hidden and ffn multiples of 128 "
                  "(got %d, %d)", cfg->hidden, cfg->ffn);
    CHECK_PTR(q->w_qkv);
    CHECK_PTR(q->w_qkv_scale);
    CHECK_PTR(q->w_o);
    CHECK_PTR(q->w_o_scale);
    CHECK_PTR(q->w_up);
    CHECK_PTR(q->w_up_scale);
    CHECK_PTR(q->w_down);
    CHECK_PTR(q->w_down_scale);
  } else {
    CHECK_PTR(w->w_qkv);
    CHECK_PTR(w->w_o);
    CHECK_PTR(w->w_up);
    CHECK_PTR(w->w_down);
  }
  if (events) {
    if (n_events != 10) return fail(H3DIT_EINVAL, "n_events must be 10 (got %d)", n_events);
    for (int i = 0; i < 10; ++i)
      if (!events[i]) return fail(H3DIT_EINVAL, "events[%d] is NULL", i);
  }
  const Plan p = make_plan(cfg, q != nullptr);
  if (ws_bytes < p.total)
    return fail(H3DIT_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p.total);
  {
    const size_t xb = (cfg->x_dtype == H3DIT_F32 ? 4 : 2) * (size_t)(p.T * p.D);
    const size_t ob = 4 * (size_t)(p.T * p.D);
    const char *xs = static_cast<const char *>(x), *os = reinterpret_cast<const char *>(out);
    const char *wss = static_cast<const char *>(ws);
    if (os < xs + xb && xs < os + ob) return fail(H3DIT_EINVAL, "out overlaps x");
    if (os < wss + p.total && wss < os + ob) return fail(H3DIT_EINVAL, "out overlaps workspace");
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const double *mod = mod_in ? mod_in : at<double>(ws, p.mod);
  float *table = at<float>(ws, p.table);
  void *h = at<void>(ws, p.h);
  void *qk = at<void>(ws, p.qk);
  void *vt = at<void>(ws, p.vt);
  void *o = at<void>(ws, p.o);
  float *x1 = at<float>(ws, p.x1);
  void *u = at<void>(ws, p.u);
  const int T = (int)p.T, D = (int)p.D, A = (int)p.A, F = (int)p.F, H = (int)p.H;
  float *split = at<float>(ws, p.split);

  auto mark = [&](int i) -> hipError_t {
    if (!events) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  };
  // one linear: bf16 operands, or (MXFP8) the input's codes xq / xqs (written
  // by its producer, or quantised here when quantise is set) and the MXFP8
  // weight wq / wqs
  uint8_t *qa = at<uint8_t>(ws, p.qa), *qas = at<uint8_t>(ws, p.qas);
  uint8_t *qb = at<uint8_t>(ws, p.qb), *qbs = at<uint8_t>(ws, p.qbs);
  auto linear = [&](GemmEpilogue epi, GemmArgs g, const uint8_t *wq, const uint8_t *wqs,
                    uint8_t *xq, uint8_t *xqs, bool quantise) -> hipError_t {
    g.partial = split;
    g.partial_bytes = p.split_bytes;
    if (!q) return launch_gemm(epi, g, s);
    if (quantise) {
      const hipError_t e = launch_mxfp8_quantize(g.x, g.M, g.K, xq, xqs, s);
      if (e != hipSuccess) return e;
    }
    g.x = xq;
    g.x_scale = xqs;
    g.w = wq;
    g.w_scale = wqs;
    return launch_gemm_mx(epi, g, s);
  };

  LAUNCH(mark(0), "event record");
  if (!mod_in)
    LAUNCH(launch_modulation(w->w_ada, cond, at<double>(ws, p.mod), 6 * D, D, s), "modulation");
  LAUNCH(mark(1), "event record");
  if (!table_ready)
    LAUNCH(launch_rope_table(positions, table, T, cfg->rope_base, s), "rope table");
  LAUNCH(mark(2), "event record");
  if (q)  // h1 in bf16 and as MXFP8 codes for the QKV linear
    LAUNCH(launch_rmsnorm_modulate_mx(x, cfg->x_dtype == H3DIT_F32, mod + 0 * D, mod + 1 * D, h, qa,
                                      qas, T, D, cfg->eps, s, !lean),
           "rmsnorm 1");
  else
    LAUNCH(launch_rmsnorm_modulate(x, cfg->x_dtype == H3DIT_F32, mod + 0 * D, mod + 1 * D, h, T,
                                   D, cfg->eps, s),
           "rmsnorm 1");
  LAUNCH(mark(3), "event record");
  {
    GemmArgs g = gemm_args(h, w->w_qkv, T, 3 * (int64_t)A, D);
    g.out = qk;
    g.out2 = vt;
    g.table = table;
    g.A = A;
    g.Mp = (int)p.Tp;
    LAUNCH(linear(EPI_QKV_ROPE, g, q ? q->w_qkv : nullptr, q ? q->w_qkv_scale : nullptr, qa, qas,
                  false),
           "qkv gemm");
  }
  LAUNCH(mark(4), "event record");
  if (q)  // o in bf16 and as MXFP8 codes for the output projection
    LAUNCH(launch_attention_mx(qk, vt, lean ? nullptr : o, qa, qas, T, H, (int)p.Tp, s),
           "attention");
  else
    LAUNCH(launch_attention(qk, vt, o, T, H, (int)p.Tp, s, at<float>(ws, p.att), p.att_bytes),
           "attention");
  LAUNCH(mark(5), "event record");
  {
    GemmArgs g = gemm_args(o, w->w_o, T, D, A);
    g.out = x1;
    g.resid = x;
    g.gate = mod + 2 * D;
    LAUNCH(linear(cfg->x_dtype == H3DIT_F32 ? EPI_RESID_F32 : EPI_RESID_BF16, g,
                  q ? q->w_o : nullptr, q ? q->w_o_scale : nullptr, qa, qas, false),
           "output projection");
  }
  LAUNCH(mark(6), "event record");
  if (q)
    LAUNCH(launch_rmsnorm_modulate_mx(x1, true, mod + 3 * D, mod + 4 * D, h, qa, qas, T, D,
                                      cfg->eps, s, !lean),
           "rmsnorm 2");
  else
    LAUNCH(launch_rmsnorm_modulate(x1, true, mod + 3 * D, mod + 4 * D, h, T, D, cfg->eps, s),
           "rmsnorm 2");
  LAUNCH(mark(7), "event record");
  {
    GemmArgs g = gemm_args(h, w->w_up, T, F, D);
    g.out = q && lean ? nullptr : u;
    g.out_codes = qb;  // MXFP8: u also as codes for the down linear
    g.out_scales = qbs;
    LAUNCH(linear(q ? EPI_GELU_MX : EPI_GELU, g, q ? q->w_up : nullptr,
                  q ? q->w_up_scale : nullptr, qa, qas, false),
           "mlp up");
  }
  LAUNCH(mark(8), "event record");
  {
    GemmArgs g = gemm_args(u, w->w_down, T, D, F);
    g.out = out;
    g.resid = x1;
    g.gate = mod + 5 * D;
    LAUNCH(linear(EPI_RESID_F32, g, q ? q->w_down : nullptr, q ? q->w_down_scale : nullptr, qb,
                  qbs, false),
           "mlp down");
  }
  LAUNCH(mark(9), "event record");
  return ok();
}

struct StackPlan {
  int64_t T, D, Ti, F;  // tokens, hidden, image tokens, features per patch
  size_t block, xa, xb, patches, modf, hf, vt, total;
  size_t block_bytes;
};

int check_stack(const h3dit_config *cfg, const h3dit_stack_config *st) {
  CHECK_CFG(cfg);
  if (!st) return fail(H3DIT_EINVAL, "st is NULL");
  if (st->n_blocks < 0 || st->channels < 1 || st->patch < 1 || st->grid_h < 1 || st->grid_w < 1 ||
      st->text_tokens < 0)
    return fail(H3DIT_EINVAL, "stack config: need n_blocks >= 0, channels, patch, grid >= 1, "
                "text_tokens >= 0");
  const int64_t F = (int64_t)st->channels * st->patch * st->patch;
  if (F % 4 != 0 || F > 65536)
    return fail(H3DIT_EUNSUPPORTED, "channels * patch^2 must be a multiple of 4 up to 65536 "
                "(got %lld)", (long long)F);
  if ((int64_t)st->text_tokens + (int64_t)st->grid_h * st->grid_w != cfg->n_tokens)
    return fail(H3DIT_EINVAL, "n_tokens (%d) must equal text_tokens + grid_h * grid_w", cfg->n_tokens);
  return H3DIT_OK;
}

h3dit_config stack_block_config(const h3dit_config *cfg) {
  h3dit_config c = *cfg;
  c.x_dtype = H3DIT_F32;
  return c;
}

StackPlan make_stack_plan(const h3dit_config *cfg, const h3dit_stack_config *st, bool mx = false) {
  StackPlan p;
  p.T = cfg->n_tokens;
  p.D = cfg->hidden;
  p.Ti = (int64_t)st->grid_h * st->grid_w;
  p.F = (int64_t)st->channels * st->patch * st->patch;
  const h3dit_config bc = stack_block_config(cfg);
  p.block_bytes = make_plan(&bc, mx).total;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  p.block = take(p.block_bytes);
  p.xa = take(4 * p.T * p.D);
  p.xb = take(4 * p.T * p.D);
  p.patches = take(4 * p.Ti * p.F);
  p.modf = take(sizeof(double) * 2 * p.D);
  p.hf = take(4 * p.Ti * p.D);
  p.vt = take(4 * p.Ti * p.F);
  p.total = off;
  return p;
}

// mods: every block's modulation and the final layer's, fp64 [(n_blocks + 1) * 6D]
// (entry n_blocks holds the final layer's shift and scale in its first 2D values),
// or NULL to compute them from cond. q: n_blocks MXFP8 weight sets (the blocks'
// linears in MXFP8), or NULL for bf16 linears.
int dit_impl(const h3dit_config *cfg, const h3dit_stack_config *st, const h3dit_stack_weights *w,
             const float *latent, const float *text, const float *cond, const int32_t *positions,
             float *v, void *ws, size_t ws_bytes, void *stream, const double *mods = nullptr,
             const h3dit_mxfp8_weights *q = nullptr) {
  {
    const int st_ = check_stack(cfg, st);
    if (st_ != H3DIT_OK) return st_;
  }
  if (!w) return fail(H3DIT_EINVAL, "w is NULL");
  CHECK_PTR(w->w_patch);
  if (!mods) CHECK_PTR(w->w_ada_final);
  CHECK_PTR(w->w_final);
  if (st->n_blocks > 0 && !w->blocks) return fail(H3DIT_EINVAL, "w->blocks is NULL");
  CHECK_PTR(latent);
  if (st->text_tokens > 0) CHECK_PTR(text);
  if (!mods) CHECK_PTR(cond);
  CHECK_PTR(positions);
  CHECK_PTR(v);
  CHECK_PTR(ws);
  if (q && st->n_blocks > 0 && (cfg->hidden % 128 != 0 || cfg->ffn % 128 != 0))
    return fail(H3DIT_EUNSUPPORTED, "MXFP8 linears need hidden and ffn multiples of 128 "
                "(got %d, %d)", cfg->hidden, cfg->ffn);
  const StackPlan p = make_stack_plan(cfg, st, q != nullptr);
  if (ws_bytes < p.total)
    return fail(H3DIT_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p.total);
  {
    const size_t vb = 4 * (size_t)(p.Ti * p.F);
    const char *vs = reinterpret_cast<const char *>(v), *wss = static_cast<const char *>(ws);
    if (vs < wss + p.total && wss < vs + vb) return fail(H3DIT_EINVAL, "v overlaps workspace");
  }
  for (int l = 0; l < st->n_blocks; ++l) {  // every block's weights, before anything is enqueued
    const h3dit_weights &b = w->blocks[l];
    const void *lin[8] = {b.w_qkv, b.w_o, b.w_up, b.w_down, nullptr, nullptr, nullptr, nullptr};
    int nlin = 4;
    if (q) {
      const h3dit_mxfp8_weights &m = q[l];
      const void *mq[8] = {m.w_qkv, m.w_qkv_scale, m.w_o, m.w_o_scale,
                           m.w_up,  m.w_up_scale,  m.w_down, m.w_down_scale};
      for (int i = 0; i < 8; ++i) lin[i] = mq[i];
      nlin = 8;
    }
    bool null = !mods && !b.w_ada, misaligned = !mods && !aligned16(b.w_ada);
    for (int i = 0; i < nlin; ++i) {
      null = null || !lin[i];
      misaligned = misaligned || !aligned16(lin[i]);
    }
    if (null) return fail(H3DIT_EINVAL, "block %d has a NULL weight pointer", l);
    if (misaligned)
      return fail(H3DIT_EALIGN, "block %d has a weight pointer that is not 16-byte aligned", l);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = (int)p.D, Ti = (int)p.Ti, F = (int)p.F, text_tokens = st->text_tokens;
  float *xa = at<float>(ws, p.xa), *xb = at<float>(ws, p.xb);
  float *patches = at<float>(ws, p.patches), *hf = at<float>(ws, p.hf), *vt = at<float>(ws, p.vt);
  double *modf = at<double>(ws, p.modf);

  // x = [text ; patch embedding]
  if (text_tokens > 0)
    LAUNCH(hipMemcpyAsync(xa, text, 4 * (size_t)text_tokens * D, hipMemcpyDeviceToDevice, s),
           "text copy");
  LAUNCH(launch_patchify(latent, patches, st->channels, st->patch, st->grid_h, st->grid_w, s),
         "patchify");
  LAUNCH(launch_gemm_f32(patches, w->w_patch, xa + (size_t)text_tokens * D, Ti, D, F, D, s),
         "patch embedding");
  // the blocks, ping-ponging the fp32 residual stream; every block uses the same
  // positions, so the RoPE table is made once, in the block workspace's table region
  const h3dit_config bc = stack_block_config(cfg);
  if (st->n_blocks > 0)
    LAUNCH(launch_rope_table(positions,
                             at<float>(at<void>(ws, p.block), make_plan(&bc, q != nullptr).table),
                             bc.n_tokens, bc.rope_base, s),
           "rope table");
  float *cur = xa, *nxt = xb;
  for (int l = 0; l < st->n_blocks; ++l) {
    const int rc = forward_impl(&bc, cur, cond, &w->blocks[l], positions, nxt, at<void>(ws, p.block),
                                p.block_bytes, stream, nullptr, 0,
                                mods ? mods + (size_t)l * 6 * D : nullptr, q ? &q[l] : nullptr,
                                /*lean=*/q != nullptr, /*table_ready=*/true);
    if (rc != H3DIT_OK) return rc;
    float *t = cur;
    cur = nxt;
    nxt = t;
  }
  // final layer on the image tokens
  const double *mf = modf;
  if (mods)
    mf = mods + (size_t)st->n_blocks * 6 * D;
  else
    LAUNCH(launch_modulation(w->w_ada_final, cond, modf, 2 * D, D, s), "final modulation");
  LAUNCH(launch_rmsnorm_modulate_f32out(cur + (size_t)text_tokens * D, true, mf, mf + D, hf, Ti,
                                        D, cfg->eps, s),
         "final rmsnorm");
  LAUNCH(launch_gemm_f32(hf, w->w_final, vt, Ti, F, D, F, s), "final projection");
  LAUNCH(launch_unpatchify(vt, v, st->channels, st->patch, st->grid_h, st->grid_w, s), "unpatchify");
  return ok();
}

// ---- the block forward without a workspace argument ----------------------
// Its scratch is this file-scope device array; each GPU holds its own copy at
// its own address. In host code `scratch` names a host-side stand-in, so the
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever handed to kernels.
__device__ __align__(256) unsigned char scratch[H3DIT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int scratch_address(void **ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(H3DIT_EUNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    const hipError_t e2 = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e2 != hipSuccess) return hip_fail(e2, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(H3DIT_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return H3DIT_OK;
}

}  // namespace

extern "C" {

int h3dit_block_forward_noalloc(const h3dit_config *cfg, const void *x, const float *cond,
                                const h3dit_weights *w, const int32_t *positions, float *out,
                                void *stream) {
  // every argument check before the first HIP call (forward_impl repeats them)
  CHECK_CFG(cfg);
  if (!w) return fail(H3DIT_EINVAL, "w is NULL");
  CHECK_PTR(x);
  CHECK_PTR(cond);
  CHECK_PTR(positions);
  CHECK_PTR(out);
  CHECK_PTR(w->w_ada);
  CHECK_PTR(w->w_qkv);
  CHECK_PTR(w->w_o);
  CHECK_PTR(w->w_up);
  CHECK_PTR(w->w_down);
  const size_t need = make_plan(cfg).total;
  if (need > (size_t)H3DIT_NOALLOC_SCRATCH_BYTES)
    return fail(H3DIT_EWORKSPACE, "this block needs %zu bytes of scratch; the static scratch "
                "holds %zu (use h3dit_block_forward with a workspace)", need,
                (size_t)H3DIT_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != H3DIT_OK) return st;
  return forward_impl(cfg, x, cond, w, positions, out, ws, need, stream, nullptr, 0);
}

int h3dit_stack_workspace_size(const h3dit_config *cfg, const h3dit_stack_config *st,
                               size_t *bytes) {
  const int rc = check_stack(cfg, st);
  if (rc != H3DIT_OK) return rc;
  if (!bytes) return fail(H3DIT_EINVAL, "bytes is NULL");
  *bytes = make_stack_plan(cfg, st).total;
  return ok();
}

int h3dit_dit_forward(const h3dit_config *cfg, const h3dit_stack_config *st,
                      const h3dit_stack_weights *w, const float *latent, const float *text,
                      const float *cond, const int32_t *positions, float *v, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return dit_impl(cfg, st, w, latent, text, cond, positions, v, workspace, workspace_bytes, stream);
}

int h3dit_dit_modulation_table(const h3dit_config *cfg, const h3dit_stack_config *st,
                               const h3dit_stack_weights *w, const float *conds, int n_steps,
                               double *table, void *stream) {
  const int rc = check_stack(cfg, st);
  if (rc != H3DIT_OK) return rc;
  if (!w) return fail(H3DIT_EINVAL, "w is NULL");
  CHECK_PTR(w->w_ada_final);
  if (st->n_blocks > 0 && !w->blocks) return fail(H3DIT_EINVAL, "w->blocks is NULL");
  CHECK_PTR(conds);
  CHECK_PTR(table);
  if (n_steps < 1 || n_steps > 4096)
    return fail(H3DIT_EINVAL, "n_steps must be in [1, 4096] (got %d)", n_steps);
  for (int l = 0; l < st->n_blocks; ++l) {
    const void *wa = w->blocks[l].w_ada;
    if (!wa) return fail(H3DIT_EINVAL, "block %d has a NULL w_ada", l);
    if (!aligned16(wa)) return fail(H3DIT_EALIGN, "block %d w_ada is not 16-byte aligned", l);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = cfg->hidden;
  const int64_t stride = (int64_t)(st->n_blocks + 1) * 6 * D;
  for (int l = 0; l < st->n_blocks; ++l)
    LAUNCH(launch_modulation_multi(w->blocks[l].w_ada, conds, n_steps, table + (int64_t)l * 6 * D,
                                   stride, 6 * D, D, s),
           "block modulation table");
  LAUNCH(launch_modulation_multi(w->w_ada_final, conds, n_steps,
                                 table + (int64_t)st->n_blocks * 6 * D, stride, 2 * D, D, s),
         "final modulation table");
  return ok();
}

int h3dit_dit_forward_mod(const h3dit_config *cfg, const h3dit_stack_config *st,
                          const h3dit_stack_weights *w, const float *latent, const float *text,
                          const double *mods, const int32_t *positions, float *v, void *workspace,
                          size_t workspace_bytes, void *stream) {
  CHECK_PTR(mods);
  return dit_impl(cfg, st, w, latent, text, nullptr, positions, v, workspace, workspace_bytes,
                  stream, mods);
}

int h3dit_stack_workspace_size_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                                     size_t *bytes) {
  const int rc = check_stack(cfg, st);
  if (rc != H3DIT_OK) return rc;
  if (!bytes) return fail(H3DIT_EINVAL, "bytes is NULL");
  *bytes = make_stack_plan(cfg, st, true).total;
  return ok();
}

int h3dit_dit_forward_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                            const h3dit_stack_weights *w, const h3dit_mxfp8_weights *q,
                            const float *latent, const float *text, const float *cond,
                            const int32_t *positions, float *v, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!q && st && st->n_blocks > 0) return fail(H3DIT_EINVAL, "q is NULL");
  // (with no blocks there is nothing to quantise: q may be NULL)
  return dit_impl(cfg, st, w, latent, text, cond, positions, v, workspace, workspace_bytes, stream,
                  nullptr, q);
}

int h3dit_dit_forward_mod_mxfp8(const h3dit_config *cfg, const h3dit_stack_config *st,
                                const h3dit_stack_weights *w, const h3dit_mxfp8_weights *q,
                                const float *latent, const float *text, const double *mods,
                                const int32_t *positions, float *v, void *workspace,
                                size_t workspace_bytes, void *stream) {
  CHECK_PTR(mods);
  if (!q && st && st->n_blocks > 0) return fail(H3DIT_EINVAL, "q is NULL");
  return dit_impl(cfg, st, w, latent, text, nullptr, positions, v, workspace, workspace_bytes,
                  stream, mods, q);
}

int h3dit_latent_step(float *latent, const float *v, float dt, int64_t n, void *stream) {
  CHECK_PTR(latent);
  CHECK_PTR(v);
  if (n < 1) return fail(H3DIT_EINVAL, "n must be >= 1 (got %lld)", (long long)n);
  if (!(dt == dt)) return fail(H3DIT_EINVAL, "dt is NaN");
  LAUNCH(launch_latent_step(latent, v, dt, n, static_cast<hipStream_t>(stream)), "latent step");
  return ok();
}


int64_t h3dit_padded_tokens(int64_t n_tokens) { return (n_tokens + 63) / 64 * 64; }

int h3dit_workspace_layout(const h3dit_config *cfg, int32_t linears, h3dit_workspace_map *map) {
  CHECK_CFG(cfg);
  if (!map) return fail(H3DIT_EINVAL, "map is NULL");
  if (linears != 0 && linears != 1)
    return fail(H3DIT_EINVAL, "linears must be 0 (bf16) or 1 (MXFP8) (got %d)", linears);
  const Plan p = make_plan(cfg, linears == 1);
  map->mod = p.mod;
  map->table = p.table;
  map->h = p.h;
  map->qk = p.qk;
  map->vt = p.vt;
  map->o = p.o;
  map->x1 = p.x1;
  map->u = p.u;
  map->q_h2 = p.qa;
  map->q_h2_scale = p.qas;
  map->q_u = p.qb;
  map->q_u_scale = p.qbs;
  return ok();
}

int h3dit_workspace_size(const h3dit_config *cfg, size_t *bytes) {
  CHECK_CFG(cfg);
  if (!bytes) return fail(H3DIT_EINVAL, "bytes is NULL");
  *bytes = make_plan(cfg).total;
  return ok();
}

int h3dit_block_forward(const h3dit_config *cfg, const void *x, const float *cond,
                        const h3dit_weights *w, const int32_t *positions, float *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(cfg, x, cond, w, positions, out, workspace, workspace_bytes, stream, nullptr,
                      0);
}

int h3dit_block_forward_timed(const h3dit_config *cfg, const void *x, const float *cond,
                              const h3dit_weights *w, const int32_t *positions, float *out,
                              void *workspace, size_t workspace_bytes, void *stream,
                              void *const *events, int n_events) {
  if (!events) return fail(H3DIT_EINVAL, "events is NULL");
  return forward_impl(cfg, x, cond, w, positions, out, workspace, workspace_bytes, stream, events,
                      n_events);
}

int h3dit_modulation(const h3dit_config *cfg, const void *w_ada, const float *cond, double *mod,
                     void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(w_ada);
  CHECK_PTR(cond);
  CHECK_PTR(mod);
  LAUNCH(launch_modulation(w_ada, cond, mod, 6 * cfg->hidden, cfg->hidden,
                           static_cast<hipStream_t>(stream)),
         "modulation");
  return ok();
}

int h3dit_modulation_table(const h3dit_config *cfg, const void *w_ada, const float *conds,
                           int n, double *mods, void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(w_ada);
  CHECK_PTR(conds);
  CHECK_PTR(mods);
  if (n < 1 || n > 4096) return fail(H3DIT_EINVAL, "n must be in [1, 4096] (got %d)", n);
  const int D = cfg->hidden;
  LAUNCH(launch_modulation_multi(w_ada, conds, n, mods, 6 * (int64_t)D, 6 * D, D,
                                 static_cast<hipStream_t>(stream)),
         "modulation table");
  return ok();
}

int h3dit_rmsnorm_modulate(const h3dit_config *cfg, const void *x, int32_t x_dtype,
                           const double *shift, const double *scale, void *h, void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(x);
  CHECK_PTR(shift);
  CHECK_PTR(scale);
  CHECK_PTR(h);
  if (x_dtype != H3DIT_BF16 && x_dtype != H3DIT_F32)
    return fail(H3DIT_EINVAL, "x_dtype must be H3DIT_BF16 or H3DIT_F32 (got %d)", x_dtype);
  LAUNCH(launch_rmsnorm_modulate(x, x_dtype == H3DIT_F32, shift, scale, h, cfg->n_tokens,
                                 cfg->hidden, cfg->eps, static_cast<hipStream_t>(stream)),
         "rmsnorm");
  return ok();
}

int h3dit_rope_table(const h3dit_config *cfg, const int32_t *positions, float *table,
                     void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(positions);
  CHECK_PTR(table);
  LAUNCH(launch_rope_table(positions, table, cfg->n_tokens, cfg->rope_base,
                           static_cast<hipStream_t>(stream)),
         "rope table");
  return ok();
}

int h3dit_qkv_rope(const h3dit_config *cfg, const void *h, const void *w_qkv, const float *table,
                   void *qk, void *vt, void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(h);
  CHECK_PTR(w_qkv);
  CHECK_PTR(table);
  CHECK_PTR(qk);
  CHECK_PTR(vt);
  const int64_t A = (int64_t)cfg->heads * 128;
  GemmArgs g = gemm_args(h, w_qkv, cfg->n_tokens, 3 * A, cfg->hidden);
  g.out = qk;
  g.out2 = vt;
  g.table = table;
  g.A = (int)A;
  g.Mp = (int)h3dit_padded_tokens(cfg->n_tokens);
  LAUNCH(launch_gemm(EPI_QKV_ROPE, g, static_cast<hipStream_t>(stream)), "qkv gemm");
  return ok();
}

int h3dit_attention(const h3dit_config *cfg, const void *qk, const void *vt, void *o,
                    void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(qk);
  CHECK_PTR(vt);
  CHECK_PTR(o);
  LAUNCH(launch_attention(qk, vt, o, cfg->n_tokens, cfg->heads,
                          (int)h3dit_padded_tokens(cfg->n_tokens), static_cast<hipStream_t>(stream)),
         "attention");
  return ok();
}

int h3dit_attention_mxfp8(const h3dit_config *cfg, const void *qk, const void *vt, void *o,
                          uint8_t *o_codes, uint8_t *o_scales, void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(qk);
  CHECK_PTR(vt);
  CHECK_PTR(o);
  CHECK_PTR(o_codes);
  CHECK_PTR(o_scales);
  LAUNCH(launch_attention_mx(qk, vt, o, o_codes, o_scales, cfg->n_tokens, cfg->heads,
                             (int)h3dit_padded_tokens(cfg->n_tokens),
                             static_cast<hipStream_t>(stream)),
         "attention");
  return ok();
}

int h3dit_out_proj_residual(const h3dit_config *cfg, const void *o, const void *w_o,
                            const void *resid, int32_t resid_dtype, const double *gate, float *x1,
                            void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(o);
  CHECK_PTR(w_o);
  CHECK_PTR(resid);
  CHECK_PTR(gate);
  CHECK_PTR(x1);
  if (resid_dtype != H3DIT_BF16 && resid_dtype != H3DIT_F32)
    return fail(H3DIT_EINVAL, "resid_dtype must be H3DIT_BF16 or H3DIT_F32 (got %d)", resid_dtype);
  GemmArgs g = gemm_args(o, w_o, cfg->n_tokens, cfg->hidden, (int64_t)cfg->heads * 128);
  g.out = x1;
  g.resid = resid;
  g.gate = gate;
  LAUNCH(launch_gemm(resid_dtype == H3DIT_F32 ? EPI_RESID_F32 : EPI_RESID_BF16, g,
                     static_cast<hipStream_t>(stream)),
         "output projection");
  return ok();
}

int h3dit_mlp_up_gelu(const h3dit_config *cfg, const void *h2, const void *w_up, void *u,
                      void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(h2);
  CHECK_PTR(w_up);
  CHECK_PTR(u);
  GemmArgs g = gemm_args(h2, w_up, cfg->n_tokens, cfg->ffn, cfg->hidden);
  g.out = u;
  LAUNCH(launch_gemm(EPI_GELU, g, static_cast<hipStream_t>(stream)), "mlp up");
  return ok();
}

int h3dit_mlp_down_residual(const h3dit_config *cfg, const void *u, const void *w_down,
                            const float *x1, const double *gate, float *out, void *stream) {
  CHECK_CFG(cfg);
  CHECK_PTR(u);
  CHECK_PTR(w_down);
  CHECK_PTR(x1);
  CHECK_PTR(gate);
  CHECK_PTR(out);
  GemmArgs g = gemm_args(u, w_down, cfg->n_tokens, cfg->hidden, cfg->ffn);
  g.out = out;
  g.resid = x1;
  g.gate = gate;
  LAUNCH(launch_gemm(EPI_RESID_F32, g, static_cast<hipStream_t>(stream)), "mlp down");
  return ok();
}

int h3dit_linear_f32(const void *x, const void *w, int32_t M, int32_t N, int32_t K, float *y,
                     void *stream) {
  CHECK_PTR(x);
  CHECK_PTR(w);
  CHECK_PTR(y);
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || N % 4 != 0)
    return fail(H3DIT_EUNSUPPORTED, "linear: need M, N >= 1, N %% 4 == 0, K a multiple of 64 "
                "(got M=%d N=%d K=%d)", M, N, K);
  GemmArgs g = gemm_args(x, w, M, N, K);
  g.out = y;
  LAUNCH(launch_gemm(EPI_F32, g, static_cast<hipStream_t>(stream)), "linear");
  return ok();
}

size_t h3dit_mxfp8_scale_bytes(int64_t rows, int64_t K) {
  if (rows < 1 || K < 128 || K % 128 != 0) return 0;
  return mx_scale_bytes(rows, K);
}

int h3dit_mxfp8_quantize(const void *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales,
                         void *stream) {
  CHECK_PTR(x);
  CHECK_PTR(codes);
  CHECK_PTR(scales);
  if (rows < 1 || rows >= ((int64_t)1 << 31) || K < 128 || K % 128 != 0 || K > (1 << 20))
    return fail(H3DIT_EUNSUPPORTED, "mxfp8 quantize: need rows in [1, 2^31) and K a multiple of "
                "128 in [128, 2^20] (got rows=%lld K=%lld)", (long long)rows, (long long)K);
  LAUNCH(launch_mxfp8_quantize(x, (int)rows, (int)K, codes, scales,
                               static_cast<hipStream_t>(stream)),
         "mxfp8 quantize");
  return ok();
}

int h3dit_linear_mxfp8(const uint8_t *x_codes, const uint8_t *x_scales, const uint8_t *w_codes,
                       const uint8_t *w_scales, int32_t M, int32_t N, int32_t K, float *y,
                       void *stream) {
  CHECK_PTR(x_codes);
  CHECK_PTR(x_scales);
  CHECK_PTR(w_codes);
  CHECK_PTR(w_scales);
  CHECK_PTR(y);
  if (M < 1 || N < 1 || N % 4 != 0 || K < 128 || K % 128 != 0 || K > (1 << 20))
    return fail(H3DIT_EUNSUPPORTED, "mxfp8 linear: need M, N >= 1, N %% 4 == 0, K a multiple of "
                "128 (got M=%d N=%d K=%d)", M, N, K);
  GemmArgs g = gemm_args(x_codes, w_codes, M, N, K);
  g.x_scale = x_scales;
  g.w_scale = w_scales;
  g.out = y;
  LAUNCH(launch_gemm_mx(EPI_F32, g, static_cast<hipStream_t>(stream)), "mxfp8 linear");
  return ok();
}

int h3dit_workspace_size_mxfp8(const h3dit_config *cfg, size_t *bytes) {
  CHECK_CFG(cfg);
  if (!bytes) return fail(H3DIT_EINVAL, "bytes is NULL");
  *bytes = make_plan(cfg, true).total;
  return ok();
}

int h3dit_block_forward_mxfp8(const h3dit_config *cfg, const void *x, const float *cond,
                              const h3dit_weights *w, const h3dit_mxfp8_weights *q,
                              const int32_t *positions, float *out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  if (!q) return fail(H3DIT_EINVAL, "q is NULL");
  return forward_impl(cfg, x, cond, w, positions, out, workspace, workspace_bytes, stream, nullptr,
                      0, nullptr, q);
}

int h3dit_block_forward_mxfp8_timed(const h3dit_config *cfg, const void *x, const float *cond,
                                    const h3dit_weights *w, const h3dit_mxfp8_weights *q,
                                    const int32_t *positions, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream, void *const *events,
                                    int n_events) {
  if (!q) return fail(H3DIT_EINVAL, "q is NULL");
  if (!events) return fail(H3DIT_EINVAL, "events is NULL");
  return forward_impl(cfg, x, cond, w, positions, out, workspace, workspace_bytes, stream, events,
                      n_events, nullptr, q);
}

const char *h3dit_status_string(int status) {
  switch (status) {
    case H3DIT_OK: return "H3DIT_OK";
    case H3DIT_EINVAL: return "H3DIT_EINVAL: invalid argument";
    case H3DIT_EUNSUPPORTED: return "H3DIT_EUNSUPPORTED: unsupported shape";
    case H3DIT_EWORKSPACE: return "H3DIT_EWORKSPACE: workspace too small";
    case H3DIT_EALIGN: return "H3DIT_EALIGN: pointer not 16-byte aligned";
    case H3DIT_EHIP: return "H3DIT_EHIP: HIP launch failed";
    default: return "unknown h3dit status";
  }
}

const char *h3dit_last_error(void) { return g_last_error; }

}  // extern "C"
