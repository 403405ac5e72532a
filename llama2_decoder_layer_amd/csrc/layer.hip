// C ABI of the decoder layer: argument validation, workspace carving and the
// launch sequence of prefill and decode.  No allocation, no synchronisation.
//
// Two launch plans, chosen from the token count and format only (so the
// workspace size is known in advance):
//  * "token-skinny" (decode, and prefill of <= 32 tokens or float32):
//      QKV projection with fused RMSNorm + RoPE + cache append  (gemv)
//      split-over-context attention + log-sum-exp merge          (attn_decode)
//      O projection + residual                                   (gemv)
//      gate/up projection with fused RMSNorm + SwiGLU            (gemv)
//      down projection + residual                                (gemv)
//    Float32 layers with more than 32 tokens run this plan 32 tokens at a time.
//  * "token-wide" (prefill of > 32 tokens in bf16/f16):
//      RMSNorm, QKV GEMM + RoPE + cache append, causal MFMA attention,
//      O GEMM + residual, RMSNorm, gate/up GEMM + SwiGLU, down GEMM + residual.
#include <climits>
#include <cmath>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "llama_layer.h"

namespace ll {

static size_t esize(int dt) { return dt == LL_F32 ? 4 : 2; }
static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Timing hooks.
// ---------------------------------------------------------------------------
static const char* kernel_names[KID_COUNT] = {
    "rmsnorm",        "gemv_qkv",    "gemv_o",    "gemv_gate_up",   "gemv_down",  "gemm_qkv",
    "gemm_o",         "gemm_gate_up", "gemm_down", "attn_decode",   "attn_prefill",
    "sample"};

struct Timer {
  int kid = -1;
  int max = 0;
  int count = 0;
  std::vector<hipEvent_t> ev;  // 2 per launch
};
static Timer g_timer;

static ArmedEvents g_armed = {nullptr, nullptr};
static bool g_armed_taken = false;

void timer_before(int kid, hipStream_t) {
  g_armed = {nullptr, nullptr};
  g_armed_taken = false;
  if (g_timer.kid != kid || g_timer.count >= g_timer.max) return;
  g_armed = {g_timer.ev[2 * g_timer.count], g_timer.ev[2 * g_timer.count + 1]};
}
ArmedEvents take_armed_events() {
  const ArmedEvents e = g_armed;
  if (e.start) g_armed_taken = true;
  g_armed = {nullptr, nullptr};
  return e;
}
void timer_after(int kid, hipStream_t) {
  if (g_timer.kid == kid && g_armed_taken) ++g_timer.count;
  g_armed = {nullptr, nullptr};
  g_armed_taken = false;
}

// ---------------------------------------------------------------------------
// Validation.
// ---------------------------------------------------------------------------
static int check_config(const ll_config* c) {
  if (!c) return LL_ENULL;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->max_pos <= 0)
    return LL_EINVAL;
  if (c->n_heads % c->n_kv_heads) return LL_EINVAL;
  if (c->hidden % 8 || c->intermediate % 8 || c->head_dim % 2) return LL_EINVAL;
  if (!(c->eps > 0.f) || !(c->eps < 1.f) || !(c->rope_theta > 1.f)) return LL_EINVAL;
  if (c->act_dtype < LL_F32 || c->act_dtype > LL_F16 || c->kv_dtype < LL_F32 || c->kv_dtype > LL_F16)
    return LL_EINVAL;
  if ((c->act_dtype == LL_F32) != (c->kv_dtype == LL_F32)) return LL_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return LL_EUNSUPPORTED;
  return LL_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return LL_ENULL;
  for (const void* p : ps)
    if (!aligned16(p)) return LL_EALIGN;
  return LL_OK;
}

static int check_weights(const ll_weights* w) {
  if (!w) return LL_ENULL;
  return check_ptrs({w->attn_norm, w->w_q, w->w_k, w->w_v, w->w_o, w->ffn_norm, w->w_gate, w->w_up,
                     w->w_down, w->rope_cos, w->rope_sin});
}

// int32 id/length arrays and float32 logits are accessed element by element.
static int check_ptrs4(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return LL_ENULL;
  for (const void* p : ps)
    if ((uintptr_t)p & 3u) return LL_EALIGN;
  return LL_OK;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// ---------------------------------------------------------------------------
// Workspace layout.
// ---------------------------------------------------------------------------
static bool wide_plan(const ll_config* c, int64_t tokens_total, bool decode) {
  return !decode && c->act_dtype != LL_F32 && tokens_total > 32;
}

struct Layout {
  size_t q32, pm, pl, pacc, part, ssq, u, q16, o, h1, a, total;
  int nsplit_max;
};

// nsplit_max < 0: room for the attention splits of any context up to s_max.
static Layout layout(const ll_config* c, int64_t bt, int s_max, bool wide, int nsplit_max = -1) {
  Layout L{};
  const size_t act = esize(c->act_dtype);
  const size_t qd = (size_t)c->n_heads * c->head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  if (wide) {
    L.u = take(bt * c->hidden * act);
    L.q16 = take(bt * qd * esize(c->kv_dtype));
    // K-split partials of the prefill GEMMs.
    const int H = c->hidden, I = c->intermediate, M = (int)bt;
    const int qkv = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
    size_t pb = gemm_partial_bytes(EPI_QKV, qkv, M, H);
    pb = std::max(pb, gemm_partial_bytes(EPI_RESID, H, M, (int)qd));
    pb = std::max(pb, gemm_partial_bytes(EPI_SWIGLU, I, M, H));
    pb = std::max(pb, gemm_partial_bytes(EPI_RESID, H, M, I));
    L.part = take(pb);
  } else {
    // Token-skinny plans process at most 32 tokens at a time.
    const int64_t g = std::min<int64_t>(bt, 32);
    const int cmin = attn_min_chunk(c->head_dim);
    L.nsplit_max = nsplit_max >= 0 ? nsplit_max : (s_max + cmin - 1) / cmin;
    L.u = take(g * c->hidden * act);   // norm pre-pass when the LDS stage is too small
    L.q32 = take(g * qd * 4);
    L.pm = take(g * c->n_heads * L.nsplit_max * 4);
    L.pl = take(g * c->n_heads * L.nsplit_max * 4);
    L.pacc = take(g * c->n_heads * L.nsplit_max * c->head_dim * 4);
    // K-split partials of the streaming projections.
    const int H = c->hidden, I = c->intermediate;
    const int qkv = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
    const int qd_ = c->n_heads * c->head_dim;
    size_t pf = 0;
    for (int m = 1; m <= g; ++m) {
      pf = std::max(pf, gemv_dma_partial_floats(EPI_QKV, qkv, H, m));
      pf = std::max(pf, gemv_dma_partial_floats(EPI_RESID, H, qd_, m));
      pf = std::max(pf, gemv_dma_partial_floats(EPI_SWIGLU, I, H, m));
      pf = std::max(pf, gemv_dma_partial_floats(EPI_RESID, H, I, m));
    }
    L.part = take(pf * 4);
    // Partial sums of squares of a deferred FFN norm: 16 slots per token.
    L.ssq = take(g * 16 * 4);
  }
  L.o = take(bt * qd * act);
  L.h1 = take(bt * c->hidden * act);
  L.a = take(bt * c->intermediate * act);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Launch plans.
// ---------------------------------------------------------------------------
#define LL_TRY(expr)                           \
  do {                                         \
    if ((expr) != hipSuccess) return LL_EHIP;  \
  } while (0)

static ProjArgs base_args(const ll_config* c) {
  ProjArgs p;
  memset(&p, 0, sizeof(p));
  p.eps = c->eps;
  p.nh = c->n_heads;
  p.nkv = c->n_kv_heads;
  p.hd = c->head_dim;
  p.kv_dt = c->kv_dtype;
  return p;
}

// Token-skinny plan for tokens [tok0, tok0 + m) of B*T.
// With w8 set (and w unused) the projections take quantised weights and
// per-row scales: int8 codes (wbits 8) or packed int4 codes (wbits 4, the
// fields then point to the packed rows; m at most 4).
// With pages.table set, kc and vc are the pools of a paged cache.
static int run_skinny(const ll_config* c, const ll_weights* w, const ll_weights_w8* w8,
                      const void* x, void* y, void* kc, void* vc, const int32_t* ctx_len,
                      int start_pos, int T, int max_ctx, int s_max, int64_t tok0, int m,
                      uint8_t* ws, const Layout& L, hipStream_t s, const KvPages& pages = {},
                      int wbits = 8) {
  const int dt = c->act_dtype;
  const size_t act = esize(dt);
  const int H = c->hidden, I = c->intermediate;
  const int qd = c->n_heads * c->head_dim, kd = c->n_kv_heads * c->head_dim;
  const uint8_t* xm = (const uint8_t*)x + tok0 * H * act;
  uint8_t* ym = (uint8_t*)y + tok0 * H * act;
  uint8_t* o = ws + L.o + tok0 * qd * act;
  uint8_t* h1 = ws + L.h1 + tok0 * H * act;
  uint8_t* a = ws + L.a + tok0 * I * act;

  // RMSNorm is fused into the projection when the m activation rows fit its
  // LDS stage; otherwise a norm pass writes u first.
  const bool fuse_norm = w8 ? gemv_w8_fits(dt, m, H) : gemv_fits_lds(dt, m, H);
  void* u = ws + L.u;
  const void* attn_norm = w8 ? w8->attn_norm : w->attn_norm;
  const void* ffn_norm = w8 ? w8->ffn_norm : w->ffn_norm;
  auto proj = [&](int epi, const ProjArgs& pa) {
    if (!w8) return launch_gemv(dt, epi, pa, s);
    ProjArgs q = pa;
    q.wbits = wbits;
    return launch_gemv_w8(dt, epi, q, s);
  };

  float* part = (float*)(ws + L.part);
  // Without a fused norm, the FFN norm can ride on the O projection's K-split
  // reduction (h1 * gamma and partial sums of squares) and the gate/up
  // epilogue (the 1/rms factor), which saves the norm pass: 'deferred' is
  // the number of partial sums per token, or 0.
  const int deferred =
      fuse_norm || wbits == 4 ? 0 : gemv_dma_norm_parts(dt, w8 != nullptr, m, H, qd, I);
  float* ssq = (float*)(ws + L.ssq);

  // 1. QKV + RMSNorm + RoPE + cache append.
  ProjArgs p = base_args(c);
  p.part = part;
  if (w8) {
    p.w[0] = w8->w_q; p.w[1] = w8->w_k; p.w[2] = w8->w_v;
    p.wscale[0] = w8->s_q; p.wscale[1] = w8->s_k; p.wscale[2] = w8->s_v;
  } else {
    p.w[0] = w->w_q; p.w[1] = w->w_k; p.w[2] = w->w_v;
  }
  p.seg1 = qd; p.seg2 = qd + kd;
  p.N = qd + 2 * kd; p.K = H; p.M = m; p.tok0 = (int)tok0;
  if (fuse_norm) {
    p.x = xm; p.gamma = attn_norm;
  } else {
    timer_before(KID_RMSNORM, s);
    LL_TRY(launch_rmsnorm(dt, xm, attn_norm, u, m, H, c->eps, s));
    timer_after(KID_RMSNORM, s);
    p.x = u;
  }
  p.q32 = (float*)(ws + L.q32);
  p.kc = kc; p.vc = vc; p.ctx_len = ctx_len; p.start_pos = start_pos; p.T = T;
  p.max_ctx = max_ctx; p.s_max = s_max; p.pages = pages;
  p.rcos = w8 ? w8->rope_cos : w->rope_cos;
  p.rsin = w8 ? w8->rope_sin : w->rope_sin;
  timer_before(KID_GEMV_QKV, s);
  LL_TRY(proj(EPI_QKV, p));
  timer_after(KID_GEMV_QKV, s);

  // 2. Attention over the cache.
  AttnDecodeArgs at;
  memset(&at, 0, sizeof(at));
  at.q = p.q32; at.kc = kc; at.vc = vc; at.ctx_len = ctx_len; at.start_pos = start_pos;
  at.T = T; at.max_ctx = max_ctx; at.nq = m; at.nh = c->n_heads; at.nkv = c->n_kv_heads;
  at.hd = c->head_dim; at.s_max = s_max; at.kv_dt = c->kv_dtype; at.act_dt = dt;
  const int max_keys = ctx_len ? max_ctx + 1 : start_pos + T;
  at.chunk = attn_pick_chunk(c->head_dim, max_keys, m, c->n_kv_heads, c->n_heads / c->n_kv_heads,
                             c->kv_dtype);
  if (at.chunk < 0) return LL_EUNSUPPORTED;
  at.nsplit = (max_keys + at.chunk - 1) / at.chunk;
  if (at.nsplit > L.nsplit_max) return LL_EWORKSPACE;
  at.part_m = (float*)(ws + L.pm); at.part_l = (float*)(ws + L.pl);
  at.part_acc = (float*)(ws + L.pacc); at.o = o;
  // Query n of this launch is global token tok0 + n.  Decode: sequence tok0 + n
  // at ctx_len[tok0 + n].  Prefill: the launch lies inside one sequence
  // b0 = tok0 / T, its queries at positions start_pos + tok0 % T + n.
  const size_t seq_bytes = (size_t)c->n_kv_heads * s_max * c->head_dim * esize(c->kv_dtype);
  int64_t b0;
  if (ctx_len) {
    b0 = tok0;
    at.ctx_len = ctx_len + tok0;
    at.T = 1;
  } else {
    if ((tok0 % T) + m > T) return LL_EINVAL;
    b0 = tok0 / T;
    at.start_pos = start_pos + (int)(tok0 % T);
    at.T = m;
  }
  if (pages.table) {
    at.kc = kc;
    at.vc = vc;
    at.pages = pages;
    at.pages.table = pages.table + b0 * pages.stride;
  } else {
    at.kc = (const uint8_t*)kc + b0 * seq_bytes;
    at.vc = (const uint8_t*)vc + b0 * seq_bytes;
  }
  timer_before(KID_ATTN_DECODE, s);
  LL_TRY(launch_attn_decode(at, s));
  timer_after(KID_ATTN_DECODE, s);

  // 3. O projection + residual.
  ProjArgs po = base_args(c);
  po.part = part;
  po.w[0] = w8 ? (const void*)w8->w_o : w->w_o; po.seg1 = po.seg2 = H;
  if (w8) po.wscale[0] = w8->s_o;
  po.N = H; po.K = qd; po.M = m; po.x = o; po.resid = xm; po.y = h1;
  if (deferred) {
    po.nout = u; po.ngamma = ffn_norm; po.ssq = ssq; po.ssq_parts = deferred;
  }
  timer_before(KID_GEMV_O, s);
  LL_TRY(proj(EPI_RESID, po));
  timer_after(KID_GEMV_O, s);

  // 4. gate/up + RMSNorm + SwiGLU.
  ProjArgs pg = base_args(c);
  pg.ssq = deferred ? ssq : nullptr;
  pg.ssq_parts = deferred;
  pg.part = part;
  if (w8) {
    pg.w[0] = w8->w_gate; pg.w[1] = w8->w_up;
    pg.wscale[0] = w8->s_gate; pg.wscale[1] = w8->s_up;
  } else {
    pg.w[0] = w->w_gate; pg.w[1] = w->w_up;
  }
  pg.N = I; pg.K = H; pg.M = m; pg.y = a;
  if (fuse_norm) {
    pg.x = h1; pg.gamma = ffn_norm;
  } else if (deferred) {
    pg.x = u;  // h1 * gamma from the O projection's reduction
  } else {
    timer_before(KID_RMSNORM, s);
    LL_TRY(launch_rmsnorm(dt, h1, ffn_norm, u, m, H, c->eps, s));
    timer_after(KID_RMSNORM, s);
    pg.x = u;
  }
  timer_before(KID_GEMV_GATEUP, s);
  LL_TRY(proj(EPI_SWIGLU, pg));
  timer_after(KID_GEMV_GATEUP, s);

  // 5. down + residual.
  ProjArgs pd = base_args(c);
  pd.part = part;
  pd.w[0] = w8 ? (const void*)w8->w_down : w->w_down; pd.seg1 = pd.seg2 = H;
  if (w8) pd.wscale[0] = w8->s_down;
  pd.N = H; pd.K = I; pd.M = m; pd.x = a; pd.resid = h1; pd.y = ym;
  timer_before(KID_GEMV_DOWN, s);
  LL_TRY(proj(EPI_RESID, pd));
  timer_after(KID_GEMV_DOWN, s);
  return LL_OK;
}

static int run_wide(const ll_config* c, const ll_weights* w, const void* x, void* y, void* kc,
                    void* vc, int B, int T, int start_pos, int s_max, uint8_t* ws,
                    const Layout& L, hipStream_t s,
                    const KvPages& pages = {}) {
  const int dt = c->act_dtype;
  const int H = c->hidden, I = c->intermediate;
  const int qd = c->n_heads * c->head_dim, kd = c->n_kv_heads * c->head_dim;
  const int M = B * T;
  void* u = ws + L.u;

  timer_before(KID_RMSNORM, s);
  LL_TRY(launch_rmsnorm(dt, x, w->attn_norm, u, M, H, c->eps, s));
  timer_after(KID_RMSNORM, s);

  float* part = (float*)(ws + L.part);
  ProjArgs p = base_args(c);
  p.part = part;
  p.w[0] = w->w_q; p.w[1] = w->w_k; p.w[2] = w->w_v;
  p.seg1 = qd; p.seg2 = qd + kd;
  p.N = qd + 2 * kd; p.K = H; p.M = M; p.x = u;
  p.q16 = ws + L.q16; p.kc = kc; p.vc = vc; p.start_pos = start_pos; p.T = T;
  p.pages = pages;
  p.s_max = s_max; p.rcos = w->rope_cos; p.rsin = w->rope_sin;
  timer_before(KID_GEMM_QKV, s);
  LL_TRY(launch_gemm(dt, EPI_QKV, p, s));
  timer_after(KID_GEMM_QKV, s);

  AttnPrefillArgs ap;
  ap.q = ws + L.q16; ap.kc = kc; ap.vc = vc; ap.o = ws + L.o;
  ap.B = B; ap.T = T; ap.start_pos = start_pos; ap.nh = c->n_heads; ap.nkv = c->n_kv_heads;
  ap.hd = c->head_dim; ap.s_max = s_max; ap.dt = c->kv_dtype; ap.out_dt = dt;
  ap.pages = pages;
  timer_before(KID_ATTN_PREFILL, s);
  LL_TRY(launch_attn_prefill(ap, s));
  timer_after(KID_ATTN_PREFILL, s);

  ProjArgs po = base_args(c);
  po.part = part;
  po.w[0] = w->w_o; po.seg1 = po.seg2 = H;
  po.N = H; po.K = qd; po.M = M; po.x = ws + L.o; po.resid = x; po.y = ws + L.h1;
  timer_before(KID_GEMM_O, s);
  LL_TRY(launch_gemm(dt, EPI_RESID, po, s));
  timer_after(KID_GEMM_O, s);

  timer_before(KID_RMSNORM, s);
  LL_TRY(launch_rmsnorm(dt, ws + L.h1, w->ffn_norm, u, M, H, c->eps, s));
  timer_after(KID_RMSNORM, s);

  ProjArgs pg = base_args(c);
  pg.part = part;
  pg.w[0] = w->w_gate; pg.w[1] = w->w_up;
  pg.N = I; pg.K = H; pg.M = M; pg.x = u; pg.y = ws + L.a;
  timer_before(KID_GEMM_GATEUP, s);
  LL_TRY(launch_gemm(dt, EPI_SWIGLU, pg, s));
  timer_after(KID_GEMM_GATEUP, s);

  ProjArgs pd = base_args(c);
  pd.part = part;
  pd.w[0] = w->w_down; pd.seg1 = pd.seg2 = H;
  pd.N = H; pd.K = I; pd.M = M; pd.x = ws + L.a; pd.resid = ws + L.h1; pd.y = y;
  timer_before(KID_GEMM_DOWN, s);
  LL_TRY(launch_gemm(dt, EPI_RESID, pd, s));
  timer_after(KID_GEMM_DOWN, s);
  return LL_OK;
}

}  // namespace ll

using namespace ll;

extern "C" {

size_t llama_layer_workspace_size(const ll_config* cfg, int32_t batch, int32_t tokens, int32_t s_max) {
  if (check_config(cfg) != LL_OK || batch <= 0 || tokens <= 0 || s_max <= 0) return 0;
  const int64_t bt = (int64_t)batch * tokens;
  size_t need = layout(cfg, bt, s_max, wide_plan(cfg, bt, false)).total;
  // tokens == 1 also sizes a decode of `batch` sequences (the token-skinny plan).
  if (tokens == 1) need = std::max(need, layout(cfg, bt, s_max, false).total);
  return need;
}

// Prefill over contiguous caches, or (pages.table set) the pools of a paged
// cache whose tables address s_max positions per sequence.
static int prefill_impl(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                        void* k_cache, void* v_cache, int32_t batch, int32_t tokens,
                        int32_t start_pos, int32_t s_max, void* ws, size_t ws_bytes, void* stream,
                        const KvPages& pages) {
  if (batch <= 0 || tokens <= 0 || start_pos < 0 || s_max <= 0) return LL_EINVAL;
  if ((int64_t)start_pos + tokens > s_max || (int64_t)start_pos + tokens > cfg->max_pos)
    return LL_ECACHE_FULL;
  const int64_t bt = (int64_t)batch * tokens;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, bt * cfg->hidden * act, y, bt * cfg->hidden * act)) return LL_EINVAL;
  const bool wide = wide_plan(cfg, bt, false);
  const Layout L = layout(cfg, bt, s_max, wide);
  if (!ws) return LL_EWORKSPACE;
  if (!aligned16(ws)) return LL_EALIGN;
  if (ws_bytes < L.total) return LL_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (wide)
    return run_wide(cfg, w, x, y, k_cache, v_cache, batch, tokens, start_pos, s_max,
                    (uint8_t*)ws, L, s, pages);
  // Token-skinny prefill: groups of <= 32 tokens that never straddle sequences.
  for (int b = 0; b < batch; ++b) {
    for (int t0 = 0; t0 < tokens; t0 += 32) {
      const int m = std::min(32, tokens - t0);
      const int rc = run_skinny(cfg, w, nullptr, x, y, k_cache, v_cache, nullptr, start_pos,
                                tokens, 0, s_max, (int64_t)b * tokens + t0, m, (uint8_t*)ws, L, s,
                                pages);
      if (rc) return rc;
    }
  }
  return LL_OK;
}

int llama_layer_prefill(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                        void* k_cache, void* v_cache, int32_t batch, int32_t tokens,
                        int32_t start_pos, int32_t s_max, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if ((rc = check_ptrs({x, y, k_cache, v_cache}))) return rc;
  return prefill_impl(cfg, w, x, y, k_cache, v_cache, batch, tokens, start_pos, s_max, ws,
                      ws_bytes, stream, KvPages{});
}

int llama_layer_decode(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                       void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                       int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if ((rc = check_ptrs({x, y, k_cache, v_cache}))) return rc;
  if ((rc = check_ptrs4({ctx_len}))) return rc;
  if (batch <= 0 || max_ctx < 0 || s_max <= 0) return LL_EINVAL;
  if ((int64_t)max_ctx + 1 > s_max || (int64_t)max_ctx + 1 > cfg->max_pos) return LL_ECACHE_FULL;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, (size_t)batch * cfg->hidden * act, y, (size_t)batch * cfg->hidden * act))
    return LL_EINVAL;
  const Layout L = layout(cfg, batch, s_max, false);
  if (!ws) return LL_EWORKSPACE;
  if (!aligned16(ws)) return LL_EALIGN;
  if (ws_bytes < L.total) return LL_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  for (int b0 = 0; b0 < batch; b0 += 32) {
    const int m = std::min(32, batch - b0);
    rc = run_skinny(cfg, w, nullptr, x, y, k_cache, v_cache, ctx_len, 0, 1, max_ctx, s_max, b0,
                    m, (uint8_t*)ws, L, s);
    if (rc) return rc;
  }
  return LL_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free decode.  The workspace is a file-scope device array, one
// copy per device (the loader places it with the code object; it lives until
// the process ends).  Host code never passes `scratch` itself to a kernel:
// that name is a host-side stand-in.  Its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static std::vector<uint8_t*> g_scratch_dev;  // device index -> address of `scratch`

static int scratch_address(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LL_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_dev.size()) g_scratch_dev.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LL_EHIP;
    g_scratch_dev[dev] = (uint8_t*)p;
  }
  *out = g_scratch_dev[dev];
  return LL_OK;
}

// Attention splits a decode of `batch` sequences needs at contexts up to
// max_ctx: the largest over the launch groups it runs (32 sequences, then the
// rest), with the chunk each group's launch picks.
static int decode_nsplit_need(const ll_config* c, int batch, int max_ctx) {
  const int max_keys = max_ctx + 1, g = c->n_heads / c->n_kv_heads;
  int need = 0;
  for (int m : {std::min(batch, 32), batch % 32}) {
    if (m <= 0) continue;
    const int chunk = attn_pick_chunk(c->head_dim, max_keys, m, c->n_kv_heads, g, c->kv_dtype);
    if (chunk <= 0) return -1;
    need = std::max(need, (max_keys + chunk - 1) / chunk);
  }
  return need;
}

static int check_pages(int32_t n_blocks, int32_t max_blocks, int32_t block_size, int* log2_bs) {
  if (n_blocks <= 0 || max_blocks <= 0) return LL_EINVAL;
  int l = 0;
  while ((1 << l) < block_size && l < 30) ++l;
  if (block_size < 16 || block_size > 1024 || (1 << l) != block_size) return LL_EINVAL;
  *log2_bs = l;
  return LL_OK;
}

int llama_layer_decode_noalloc(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                               void* k_cache, void* v_cache, const int32_t* ctx_len,
                               int32_t batch, int32_t max_ctx, int32_t s_max, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if ((rc = check_ptrs({x, y, k_cache, v_cache}))) return rc;
  if ((rc = check_ptrs4({ctx_len}))) return rc;
  if (batch <= 0 || max_ctx < 0 || s_max <= 0) return LL_EINVAL;
  if ((int64_t)max_ctx + 1 > s_max || (int64_t)max_ctx + 1 > cfg->max_pos) return LL_ECACHE_FULL;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, (size_t)batch * cfg->hidden * act, y, (size_t)batch * cfg->hidden * act))
    return LL_EINVAL;
  const int nsplit = decode_nsplit_need(cfg, batch, max_ctx);
  if (nsplit < 0) return LL_EUNSUPPORTED;
  // Sized for this call's contexts, not for s_max.
  const Layout L = layout(cfg, batch, s_max, false, nsplit);
  if (L.total > NOALLOC_SCRATCH_BYTES) return LL_ESCRATCH;
  uint8_t* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  for (int b0 = 0; b0 < batch; b0 += 32) {
    const int m = std::min(32, batch - b0);
    rc = run_skinny(cfg, w, nullptr, x, y, k_cache, v_cache, ctx_len, 0, 1, max_ctx, s_max, b0,
                    m, ws, L, s);
    if (rc) return rc;
  }
  return LL_OK;
}

int llama_layer_decode_paged(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                             void* k_pool, void* v_pool, int32_t n_blocks, int32_t block_size,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* ctx_len, int32_t batch, int32_t max_ctx, void* ws,
                             size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if ((rc = check_ptrs({x, y, k_pool, v_pool}))) return rc;
  if ((rc = check_ptrs4({ctx_len, block_table}))) return rc;
  int log2_bs = 0;
  if ((rc = check_pages(n_blocks, max_blocks, block_size, &log2_bs))) return rc;
  if (batch <= 0 || max_ctx < 0) return LL_EINVAL;
  const int64_t cap = (int64_t)max_blocks * block_size;
  if (cap > INT32_MAX) return LL_EINVAL;
  const int s_max = (int)cap;  // positions a sequence's table can address
  if ((int64_t)max_ctx + 1 > s_max || (int64_t)max_ctx + 1 > cfg->max_pos) return LL_ECACHE_FULL;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, (size_t)batch * cfg->hidden * act, y, (size_t)batch * cfg->hidden * act))
    return LL_EINVAL;
  const Layout L = layout(cfg, batch, s_max, false);
  if (!ws) return LL_EWORKSPACE;
  if (!aligned16(ws)) return LL_EALIGN;
  if (ws_bytes < L.total) return LL_EWORKSPACE;
  const KvPages pages{block_table, max_blocks, log2_bs, n_blocks};
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  for (int b0 = 0; b0 < batch; b0 += 32) {
    const int m = std::min(32, batch - b0);
    rc = run_skinny(cfg, w, nullptr, x, y, k_pool, v_pool, ctx_len, 0, 1, max_ctx, s_max, b0, m,
                    (uint8_t*)ws, L, s, pages);
    if (rc) return rc;
  }
  return LL_OK;
}

int llama_layer_prefill_paged(const ll_config* cfg, const ll_weights* w, const void* x, void* y,
                              void* k_pool, void* v_pool, int32_t n_blocks, int32_t block_size,
                              const int32_t* block_table, int32_t max_blocks, int32_t batch,
                              int32_t tokens, int32_t start_pos, void* ws, size_t ws_bytes,
                              void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if ((rc = check_ptrs({x, y, k_pool, v_pool}))) return rc;
  if ((rc = check_ptrs4({block_table}))) return rc;
  int log2_bs = 0;
  if ((rc = check_pages(n_blocks, max_blocks, block_size, &log2_bs))) return rc;
  const int64_t cap = (int64_t)max_blocks * block_size;
  if (cap > INT32_MAX) return LL_EINVAL;
  return prefill_impl(cfg, w, x, y, k_pool, v_pool, batch, tokens, start_pos, (int32_t)cap, ws,
                      ws_bytes, stream, KvPages{block_table, max_blocks, log2_bs, n_blocks});
}

int llama_kv_pages_write(const void* k_src, const void* v_src, int32_t s_max, int32_t start,
                         int32_t count, void* k_pool, void* v_pool, int32_t n_blocks,
                         int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                         int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t kv_dtype,
                         void* stream) {
  int rc = check_ptrs({k_src, v_src, k_pool, v_pool});
  if (rc) return rc;
  if ((rc = check_ptrs4({block_table}))) return rc;
  int log2_bs = 0;
  if ((rc = check_pages(n_blocks, max_blocks, block_size, &log2_bs))) return rc;
  if (batch <= 0 || n_kv_heads <= 0 || head_dim <= 0 || kv_dtype < LL_F32 || kv_dtype > LL_F16 ||
      (head_dim * (int)esize(kv_dtype)) % 16 || s_max <= 0 || start < 0 || count < 0)
    return LL_EINVAL;
  if ((int64_t)start + count > s_max || (int64_t)start + count > (int64_t)max_blocks * block_size)
    return LL_ECACHE_FULL;
  if (count == 0) return LL_OK;
  const KvPages pages{block_table, max_blocks, log2_bs, n_blocks};
  (void)hipGetLastError();
  if (launch_kv_pages_write(k_src, v_src, s_max, start, count, k_pool, v_pool, pages, batch,
                            n_kv_heads, head_dim, kv_dtype, (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

int llama_quantize_w8(const void* w, int8_t* q, float* scale, int32_t rows, int32_t cols,
                      int32_t dtype, void* stream) {
  int rc = check_ptrs({w, q});
  if (rc) return rc;
  if ((rc = check_ptrs4({scale}))) return rc;
  if (rows <= 0 || cols <= 0 || cols % 16 || dtype < LL_F32 || dtype > LL_F16) return LL_EINVAL;
  (void)hipGetLastError();
  if (launch_quantize_w8(dtype, w, q, scale, rows, cols, (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

// Tokens per launch group of the int8 decode: 32 through the LDS-streaming
// kernel (16-bit activations, reductions a multiple of 64); else at most 4
// (the row kernel), fewer when the activations of the longest K would not
// fit its LDS stage.
static int w8_group(const ll_config* c) {
  const int qd = c->n_heads * c->head_dim;
  if (c->act_dtype != LL_F32 && c->hidden % 64 == 0 && c->intermediate % 64 == 0 && qd % 64 == 0)
    return 32;
  const int kmax = std::max(std::max(c->hidden, c->intermediate), qd);
  int g = 4;
  while (g > 0 && !gemv_w8_fits(c->act_dtype, g, kmax)) --g;
  return g;
}

int llama_layer_decode_w8(const ll_config* cfg, const ll_weights_w8* w, const void* x, void* y,
                          void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                          int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes,
                          void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w) return LL_ENULL;
  if ((rc = check_ptrs({w->attn_norm, w->ffn_norm, w->w_q, w->w_k, w->w_v, w->w_o, w->w_gate,
                        w->w_up, w->w_down, w->rope_cos, w->rope_sin})))
    return rc;
  if ((rc = check_ptrs4({w->s_q, w->s_k, w->s_v, w->s_o, w->s_gate, w->s_up, w->s_down})))
    return rc;
  if ((rc = check_ptrs({x, y, k_cache, v_cache}))) return rc;
  if ((rc = check_ptrs4({ctx_len}))) return rc;
  if (batch <= 0 || max_ctx < 0 || s_max <= 0) return LL_EINVAL;
  if (cfg->hidden % 16 || cfg->intermediate % 16 || (cfg->n_heads * cfg->head_dim) % 16)
    return LL_EINVAL;
  if ((int64_t)max_ctx + 1 > s_max || (int64_t)max_ctx + 1 > cfg->max_pos) return LL_ECACHE_FULL;
  const int g = w8_group(cfg);
  if (g < 1) return LL_EUNSUPPORTED;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, (size_t)batch * cfg->hidden * act, y, (size_t)batch * cfg->hidden * act))
    return LL_EINVAL;
  const Layout L = layout(cfg, batch, s_max, false);
  if (!ws) return LL_EWORKSPACE;
  if (!aligned16(ws)) return LL_EALIGN;
  if (ws_bytes < L.total) return LL_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  for (int b0 = 0; b0 < batch; b0 += g) {
    const int m = std::min(g, batch - b0);
    rc = run_skinny(cfg, nullptr, w, x, y, k_cache, v_cache, ctx_len, 0, 1, max_ctx, s_max, b0, m,
                    (uint8_t*)ws, L, s);
    if (rc) return rc;
  }
  return LL_OK;
}

int llama_quantize_w4(const void* w, uint8_t* q, float* scale, int32_t rows, int32_t cols,
                      int32_t dtype, void* stream) {
  int rc = check_ptrs({w, q});
  if (rc) return rc;
  if ((rc = check_ptrs4({scale}))) return rc;
  if (rows <= 0 || cols <= 0 || cols % 32 || dtype < LL_F32 || dtype > LL_F16) return LL_EINVAL;
  (void)hipGetLastError();
  if (launch_quantize_w4(dtype, w, q, scale, rows, cols, (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

int llama_layer_decode_w4(const ll_config* cfg, const ll_weights_w4* w, const void* x, void* y,
                          void* k_cache, void* v_cache, const int32_t* ctx_len, int32_t batch,
                          int32_t max_ctx, int32_t s_max, void* ws, size_t ws_bytes,
                          void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w) return LL_ENULL;
  if ((rc = check_ptrs({w->attn_norm, w->ffn_norm, w->w_q, w->w_k, w->w_v, w->w_o, w->w_gate,
                        w->w_up, w->w_down, w->rope_cos, w->rope_sin})))
    return rc;
  if ((rc = check_ptrs4({w->s_q, w->s_k, w->s_v, w->s_o, w->s_gate, w->s_up, w->s_down})))
    return rc;
  if ((rc = check_ptrs({x, y, k_cache, v_cache}))) return rc;
  if ((rc = check_ptrs4({ctx_len}))) return rc;
  if (batch <= 0 || max_ctx < 0 || s_max <= 0) return LL_EINVAL;
  if (cfg->hidden % 32 || cfg->intermediate % 32 || (cfg->n_heads * cfg->head_dim) % 32)
    return LL_EINVAL;
  if ((int64_t)max_ctx + 1 > s_max || (int64_t)max_ctx + 1 > cfg->max_pos) return LL_ECACHE_FULL;
  // Groups of at most 4 sequences through the row kernel.
  const int kmax = std::max(std::max(cfg->hidden, cfg->intermediate),
                            cfg->n_heads * cfg->head_dim);
  int g = 4;
  while (g > 0 && !gemv_w8_fits(cfg->act_dtype, g, kmax)) --g;
  if (g < 1) return LL_EUNSUPPORTED;
  const size_t act = esize(cfg->act_dtype);
  if (overlap(x, (size_t)batch * cfg->hidden * act, y, (size_t)batch * cfg->hidden * act))
    return LL_EINVAL;
  const Layout L = layout(cfg, batch, s_max, false);
  if (!ws) return LL_EWORKSPACE;
  if (!aligned16(ws)) return LL_EALIGN;
  if (ws_bytes < L.total) return LL_EWORKSPACE;
  // Same field layout as the int8 weights; the kernels read packed int4 rows.
  ll_weights_w8 w8;
  w8.attn_norm = w->attn_norm; w8.ffn_norm = w->ffn_norm;
  w8.w_q = (const int8_t*)w->w_q; w8.w_k = (const int8_t*)w->w_k;
  w8.w_v = (const int8_t*)w->w_v; w8.w_o = (const int8_t*)w->w_o;
  w8.w_gate = (const int8_t*)w->w_gate; w8.w_up = (const int8_t*)w->w_up;
  w8.w_down = (const int8_t*)w->w_down;
  w8.s_q = w->s_q; w8.s_k = w->s_k; w8.s_v = w->s_v; w8.s_o = w->s_o;
  w8.s_gate = w->s_gate; w8.s_up = w->s_up; w8.s_down = w->s_down;
  w8.rope_cos = w->rope_cos; w8.rope_sin = w->rope_sin;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  for (int b0 = 0; b0 < batch; b0 += g) {
    const int m = std::min(g, batch - b0);
    rc = run_skinny(cfg, nullptr, &w8, x, y, k_cache, v_cache, ctx_len, 0, 1, max_ctx, s_max, b0,
                    m, (uint8_t*)ws, L, s, KvPages{}, 4);
    if (rc) return rc;
  }
  return LL_OK;
}

int llama_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                     float rope_theta, void* stream) {
  if (!cos_out || !sin_out) return LL_ENULL;
  if (max_pos <= 0 || head_dim <= 0 || head_dim % 2 || !(rope_theta > 1.f)) return LL_EINVAL;
  (void)hipGetLastError();
  if (launch_rope_table(cos_out, sin_out, max_pos, head_dim, (double)rope_theta,
                        (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

int llama_rope_table_ntk(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                         float rope_theta, float ntk_scale, void* stream) {
  if (!cos_out || !sin_out) return LL_ENULL;
  if (max_pos <= 0 || head_dim < 4 || head_dim % 2 || !(rope_theta > 1.f) ||
      !(ntk_scale >= 1.f) || !std::isfinite(ntk_scale))
    return LL_EINVAL;
  // The base grows by scale^(d/(d-2)), so theta_i = base^(-2i/d) shrinks by
  // scale^(-2i/(d-2)): 1 for i = 0, 1/scale for i = d/2 - 1.
  const double d = (double)head_dim;
  const double base = (double)rope_theta * std::pow((double)ntk_scale, d / (d - 2.0));
  (void)hipGetLastError();
  if (launch_rope_table(cos_out, sin_out, max_pos, head_dim, base, (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

int llama_embed(const void* table, const int32_t* ids, void* h, int32_t n, int32_t hidden,
                int32_t vocab, int32_t dtype, void* stream) {
  int rc = check_ptrs({table, h});
  if (rc) return rc;
  if ((rc = check_ptrs4({ids}))) return rc;
  if (n <= 0 || hidden <= 0 || hidden % 8 || vocab <= 0 || dtype < LL_F32 || dtype > LL_F16)
    return LL_EINVAL;
  (void)hipGetLastError();
  if (launch_embed(table, ids, h, n, hidden, vocab, dtype, (hipStream_t)stream) != hipSuccess)
    return LL_EHIP;
  return LL_OK;
}

int llama_head_argmax(const void* final_norm, const void* w_lm, const void* h, int32_t* ids_out,
                      float* logits, int32_t n, int32_t hidden, int32_t vocab, float eps,
                      int32_t dtype, void* stream) {
  int rc = check_ptrs({final_norm, w_lm, h});
  if (rc) return rc;
  if ((rc = check_ptrs4({ids_out, logits}))) return rc;
  if (n <= 0 || hidden <= 0 || hidden % 8 || vocab <= 0 || dtype < LL_F32 || dtype > LL_F16 ||
      !(eps > 0.f))
    return LL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const size_t esz = esize(dtype);
  // Rows go through the fused-norm projection in groups whose activations fit its LDS stage.
  int group = 16;
  while (group > 1 && !gemv_fits_lds(dtype, group, hidden)) group >>= 1;
  if (!gemv_fits_lds(dtype, group, hidden)) return LL_EUNSUPPORTED;
  for (int r0 = 0; r0 < n; r0 += group) {
    ProjArgs p;
    memset(&p, 0, sizeof(p));
    p.w[0] = w_lm; p.seg1 = p.seg2 = vocab;
    p.N = vocab; p.K = hidden; p.M = std::min(group, n - r0);
    p.x = (const uint8_t*)h + (size_t)r0 * hidden * esz;
    p.gamma = final_norm; p.eps = eps;
    p.y = logits + (size_t)r0 * vocab;
    if (launch_gemv(dtype, EPI_LOGITS, p, s) != hipSuccess) return LL_EHIP;
  }
  if (launch_argmax(logits, ids_out, n, vocab, s) != hipSuccess) return LL_EHIP;
  return LL_OK;
}

int llama_sample(const float* logits, const int32_t* history, int32_t n_hist, const float* u,
                 int32_t* ids_out, int32_t n, int32_t vocab, float temperature, int32_t top_k,
                 float top_p, float penalty, void* stream) {
  int rc = check_ptrs4({logits, u, ids_out});
  if (rc) return rc;
  if (n_hist < 0 || n < 0) return LL_EINVAL;
  if (n_hist > 0 && (rc = check_ptrs4({history}))) return rc;
  if (vocab < 1 || vocab > SAMPLE_MAX_VOCAB || top_k < 1 || top_k > 1024 || !(top_p > 0.f && top_p <= 1.f) ||
      !(temperature >= 0.f) || !std::isfinite(temperature) || !(penalty > 0.f) ||
      !std::isfinite(penalty))
    return LL_EINVAL;
  if (n == 0) return LL_OK;
  SampleArgs a;
  a.logits = logits;
  a.history = n_hist > 0 ? history : nullptr;
  a.n_hist = n_hist;
  a.u = u;
  a.ids_out = ids_out;
  a.n = n;
  a.vocab = vocab;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.penalty = penalty;
  (void)hipGetLastError();
  timer_before(KID_SAMPLE, (hipStream_t)stream);
  const hipError_t e = launch_sample(a, (hipStream_t)stream);
  timer_after(KID_SAMPLE, (hipStream_t)stream);
  return e == hipSuccess ? LL_OK : LL_EHIP;
}

const char* llama_layer_strerror(int code) {
  switch (code) {
    case LL_OK: return "ok";
    case LL_EINVAL: return "invalid configuration or size";
    case LL_ENULL: return "a required pointer is NULL";
    case LL_EALIGN: return "a pointer is not 16-byte aligned";
    case LL_ECACHE_FULL: return "positions would run past the KV-cache capacity or RoPE table";
    case LL_EWORKSPACE: return "workspace missing or too small";
    case LL_EHIP: return "HIP launch error";
    case LL_EUNSUPPORTED: return "configuration not supported (head_dim must be 64 or 128)";
    case LL_ESCRATCH:
      return "the call needs more workspace than the 64 MiB built-in scratch of "
             "llama_layer_decode_noalloc (use llama_layer_decode with a workspace)";
  }
  return "unknown error";
}

int llama_layer_timer_start(int32_t kernel_id, int32_t max_launches) {
  if (kernel_id < 0 || kernel_id >= KID_COUNT || max_launches <= 0) return LL_EINVAL;
  for (hipEvent_t e : g_timer.ev) (void)hipEventDestroy(e);
  g_timer.ev.assign(2 * (size_t)max_launches, nullptr);
  // No system-scope fence at the events: a release to system scope writes back
  // and invalidates caches, which would be counted as kernel time.
  for (auto& e : g_timer.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return LL_EHIP;
  g_timer.kid = kernel_id;
  g_timer.max = max_launches;
  g_timer.count = 0;
  return LL_OK;
}

int llama_layer_timer_stop(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return LL_ENULL;
  double tot = 0.0;
  int rc = LL_OK;
  for (int i = 0; i < g_timer.count; ++i) {
    if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess) { rc = LL_EHIP; break; }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess) {
      rc = LL_EHIP;
      break;
    }
    tot += ms;
  }
  *total_ms = tot;
  *launches = g_timer.count;
  for (hipEvent_t e : g_timer.ev) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.kid = -1;
  g_timer.max = g_timer.count = 0;
  return rc;
}

const char* llama_layer_kernel_name(int32_t kernel_id) {
  if (kernel_id < 0 || kernel_id >= KID_COUNT) return nullptr;
  return kernel_names[kernel_id];
}

}  // extern "C"
