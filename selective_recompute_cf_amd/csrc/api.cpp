// libcf host side: argument validation, workspace layout, launch plan and the C ABI of
// include/cf.h. Every step of the path is a kernel launch on the caller's stream; the host
// never waits for the device inside a call (a streamed prefill waits only for the previous
// streamed call of its context).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "cf.h"
#include "kernels.h"
#include "status.h"

struct cf_ctx {
  cf_model_cfg cfg;
  int device;
  int max_pos;
  int n_cu;
  float* cos_t;  // [max_pos][head_dim/2]
  float* sin_t;
  // host-to-device copies of a chunk store in host memory (cf_blend_prefill_streamed): a copy
  // stream (default priority), the call-start event and, per staging slot, a layer-ready event
  hipStream_t copy_st;
  hipEvent_t start_ev, copied[2];
  // end of the last two streamed calls (by call parity) and the number of streamed calls made
  hipEvent_t done[2];
  mutable long long streamed_calls;
};

namespace {

thread_local std::string g_err;

cf_status fail(cf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

namespace cf {
void clear_error() { g_err.clear(); }
cf_status set_error(cf_status s, const char* msg) {
  g_err = msg;
  return s;
}
}  // namespace cf

namespace {

#define CF_CHECK(cond, status, ...) \
  do {                              \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define CF_HIP(expr)                                                                         \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) return fail(CF_EHIP, "%s: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

// ------------------------------------------------------------------ optional kernel timing
// While enabled, each launch is bracketed by two HIP events recorded on the launch's own
// stream; cf_profile_report() waits for them and sums the elapsed times per kernel name.
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
std::string g_report;

hipEvent_t prof_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing only, never a memory order for a reader: without the system-scope release a default
  // event adds after a kernel (an L2 write-back), which would be timed as part of the launch
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(const char* name, hipStream_t st, F launch) {
  if (!g_prof) return launch();
  hipEvent_t a = prof_event(), b = prof_event();
  if (a) (void)hipEventRecord(a, st);
  const hipError_t e = launch();
  if (b) (void)hipEventRecord(b, st);
  if (a && b) g_recs.push_back({name, a, b});
  return e;
}
#define CF_RUN(name, expr) CF_HIP(timed(name, st, [&]() { return (expr); }))

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Makes the context's device current for the duration of a call and restores the caller's.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

cf::Dt dt_of(const cf_ctx* c) { return c->cfg.dtype == CF_BF16 ? cf::BF16 : cf::F32; }
size_t esize(const cf_ctx* c) { return c->cfg.dtype == CF_BF16 ? 2 : 4; }
size_t al(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------------ workspace of one layer pass
struct LayerPlan {
  cf::GemmPlan qkv, o, gu, down, ksel;
  int attn_P;
};

LayerPlan layer_plan(const cf_ctx* c, int L, int R, int ksel_rows) {
  const cf_model_cfg& m = c->cfg;
  const cf::Dt dt = dt_of(c);
  const int d = m.d_model, qd = m.n_q_heads * m.head_dim, kvd = m.n_kv_heads * m.head_dim, F = m.d_ffn;
  LayerPlan p{};
  p.qkv = cf::gemm_plan(dt, R, qd + 2 * kvd, d, false, true, c->n_cu);
  p.o = cf::gemm_plan(dt, R, d, qd, false, true, c->n_cu);
  p.gu = cf::gemm_plan(dt, R, F, d, true, false, c->n_cu);
  p.down = cf::gemm_plan(dt, R, d, F, false, true, c->n_cu);
  p.ksel = cf::gemm_plan(dt, ksel_rows, kvd, d, false, true, c->n_cu);
  cf::attn_plan(dt, R, m.n_q_heads, m.n_kv_heads, c->n_cu, &p.attn_P);
  return p;
}

struct LayerWs {
  size_t x, qkv, q, ao, hs, act, gu, part, opart, mlpart, sched, total;
  LayerPlan plan;
};

// Scratch of one layer pass over R rows of an L-row request; ksel_rows > 0 also sizes the
// selection-layer key projection of that many context rows (it reuses x and qkv).
LayerWs layer_ws(const cf_ctx* c, int L, int R, int ksel_rows = 0) {
  const cf_model_cfg& m = c->cfg;
  const size_t es = esize(c);
  const size_t d = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim, kvd = (size_t)m.n_kv_heads * m.head_dim;
  const size_t F = m.d_ffn;
  LayerWs w{};
  w.plan = layer_plan(c, L, R, ksel_rows);
  const LayerPlan& p = w.plan;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  w.x = take((size_t)std::max(R, ksel_rows) * d * es);
  w.qkv = take(std::max((size_t)p.qkv.splits * R * (qd + 2 * kvd), (size_t)p.ksel.splits * ksel_rows * kvd) * 4);
  w.q = take((size_t)R * qd * es);
  w.ao = take((size_t)R * qd * es);
  w.hs = take((size_t)R * d * 4);
  w.act = take((size_t)R * F * es);
  w.gu = take(m.dtype == CF_BF16 ? 0 : (size_t)R * 2 * F * 4);
  const int ps = std::max(p.o.splits, p.down.splits);
  w.part = take(ps > 1 ? (size_t)ps * R * d * 4 : 0);
  // attention partial sums of the balanced pieces: [hkv][P][128][hd] and [hkv][P][128][2]
  const size_t pieces = (size_t)m.n_kv_heads * p.attn_P * 128;
  w.opart = take(pieces * m.head_dim * 4);
  w.mlpart = take(pieces * 2 * 4);
  w.sched = take(p.attn_P > 0 ? sizeof(cf::AttnSched) : 0);
  w.total = off;
  return w;
}

struct PrefillWs {
  size_t hidden, sel, sel2, ident, dev, dev2, devh, topk, topk_bytes, stage, layer, total;
};

// ks: the per-layer counts of gradual filtering (nks of them, ks[0] = k), or null.
// stage_rows > 0: two staging slots of one store layer (K then V, stage_rows rows each).
PrefillWs prefill_ws(const cf_ctx* c, int N, int U, int k, int mode, const int32_t* ks = nullptr, int nks = 0,
                     int stage_rows = 0) {
  const int L = N + U;
  PrefillWs p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  p.stage = take((size_t)2 * 2 * stage_rows * c->cfg.n_kv_heads * c->cfg.head_dim * esize(c));
  p.hidden = take((size_t)L * c->cfg.d_model * 4);
  p.sel = take((size_t)L * 4);
  p.ident = take((size_t)L * 4);
  p.dev = take((size_t)std::max(N, 1) * 4);
  // the layer scratch serves full-row layers (R = L) and selected-row layers (R = k + U)
  const LayerWs a = layer_ws(c, L, L, mode == CF_SEL_ALL ? 0 : N), b = layer_ws(c, L, std::min(L, k + U));
  size_t layer = std::max(a.total, b.total), topk = cf_topk_workspace_size(N, mode);
  if (ks) {  // a second set buffer, the per-head and per-row deviations of a set, each set size's scratch
    p.sel2 = take((size_t)L * 4);
    p.dev2 = take((size_t)std::max(k, 1) * 4);
    p.devh = take((size_t)std::max(k, 1) * c->cfg.n_kv_heads * 4);
    for (int i = 0; i < nks; ++i) {
      layer = std::max(layer, layer_ws(c, L, std::min(L, ks[i] + U)).total);
      topk = std::max(topk, cf_topk_workspace_size(ks[i], mode));
    }
  }
  p.topk = take(topk);
  p.topk_bytes = topk;
  p.layer = take(layer);
  p.total = off;
  return p;
}

cf_status check_layer(const cf_ctx* c, const cf_layer_weights* w, int idx) {
  CF_CHECK(w, CF_EINVAL, "layer %d: null weight struct", idx);
  const void* ptrs[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  const char* names[] = {"attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 9; ++i) {
    CF_CHECK(ptrs[i], CF_EINVAL, "layer %d: %s is NULL", idx, names[i]);
    CF_CHECK(aligned16(ptrs[i]), CF_EINVAL, "layer %d: %s is not 16-byte aligned", idx, names[i]);
  }
  if (c->cfg.qk_norm) {
    CF_CHECK(w->q_norm && w->k_norm, CF_EINVAL, "layer %d: qk_norm model needs q_norm and k_norm", idx);
  }
  return CF_OK;
}

// ------------------------------------------------------------------ one layer on rows `sel`
// x_ready: the attention-norm input X of these rows is already in the workspace (written by the
// previous layer on the same rows). next_norm: the next layer's attention-norm gain; when the down
// projection is split along K, its reduction then also writes the next layer's X (bit-identical
// to a separate normalisation) and *x_next is set.
// Attention mass of the layer's rows on the context keys [0, n_ctx), added to score (QCFuse
// Eq. 10): ml [n][hq][2] and part [hkv][n_ctx] are scratch; first = this layer starts the sum.
struct MassHook {
  float* ml; float* part; float* score; int n_ctx; bool first;
};

// dev_heads: also measure, for the first n_dev rows, each kv head's squared distance between the
// fresh key and the cached key it replaces ([n_dev][n_kv_heads]).
cf_status run_layer(const cf_ctx* c, const cf_layer_weights* w, float* hidden, void* kc, void* vc,
                    const int* sel, int n, int L, char* ws, const LayerWs& lw, hipStream_t st,
                    bool x_ready = false, const float* next_norm = nullptr, bool* x_next = nullptr,
                    bool* sched_ready = nullptr, float* dev_heads = nullptr, int n_dev = 0,
                    const MassHook* mass = nullptr, int rope_off = 0) {
  if (x_next) *x_next = false;
  if (n == 0) return CF_OK;
  const cf_model_cfg& m = c->cfg;
  const cf::Dt dt = dt_of(c);
  const int d = m.d_model, hd = m.head_dim, qd = m.n_q_heads * hd, kvd = m.n_kv_heads * hd, F = m.d_ffn;
  void* X = ws + lw.x;
  float* QKV = reinterpret_cast<float*>(ws + lw.qkv);
  void* Q = ws + lw.q;
  void* AO = ws + lw.ao;
  float* HS = reinterpret_cast<float*>(ws + lw.hs);
  void* ACT = ws + lw.act;

  const LayerPlan& P = lw.plan;
  if (!x_ready)
    CF_RUN("rmsnorm_rows", cf::launch_rmsnorm_rows(dt, hidden, sel, n, L, d, w->attn_norm, m.rms_eps, X, d, st));
  cf::GemmArgs g{};
  g.dt = dt; g.cfg = P.qkv.cfg; g.splits = P.qkv.splits;
  g.A = X; g.lda = d;
  g.B[0] = w->wq; g.B[1] = w->wk; g.B[2] = w->wv; g.nb0 = qd; g.nb1 = qd + kvd;
  g.M = n; g.N = qd + 2 * kvd; g.K = d; g.epi = g.splits > 1 ? cf::EPI_PARTIAL : cf::EPI_F32;
  g.C = QKV; g.ldc = qd + 2 * kvd;
  CF_RUN("gemm/qkv", cf::launch_gemm(g, st));

  cf::QkvPost qp{};
  qp.qkv = QKV; qp.ld = qd + 2 * kvd; qp.rows = sel; qp.n = n; qp.L = L;
  qp.splits = g.splits; qp.split_stride = (int64_t)n * (qd + 2 * kvd);
  qp.hq = m.n_q_heads; qp.hkv = m.n_kv_heads; qp.hd = hd; qp.qk_norm = m.qk_norm;
  qp.qn = w->q_norm; qp.kn = w->k_norm; qp.eps = m.rms_eps; qp.cos_t = c->cos_t; qp.sin_t = c->sin_t;
  qp.q_out = Q; qp.k_cache = kc; qp.v_cache = vc;
  qp.dev_heads = dev_heads; qp.n_dev = dev_heads ? n_dev : 0; qp.rope_off = rope_off;
  CF_RUN("qkv_post", cf::launch_qkv_post(dt, qp, st));

  cf::AttnArgs at{};
  at.dt = dt; at.q = Q; at.ldq = qd; at.pos = sel; at.n = n; at.k = kc; at.v = vc; at.L = L;
  at.hq = m.n_q_heads; at.hkv = m.n_kv_heads; at.hd = hd; at.out = AO; at.ldo = qd;
  at.o_part = reinterpret_cast<float*>(ws + lw.opart);
  at.ml_part = reinterpret_cast<float*>(ws + lw.mlpart);
  if (P.attn_P > 0) {
    // the pieces depend only on the rows' positions: built once for layers that share `sel`
    cf::AttnSched* sch = reinterpret_cast<cf::AttnSched*>(ws + lw.sched);
    at.P = P.attn_P;
    if (!sched_ready || !*sched_ready) CF_RUN("attn_sched", cf::launch_attention_sched(at, sch, st));
    if (sched_ready) *sched_ready = true;
    at.sched = sch;
  }
  at.ml_out = mass ? mass->ml : nullptr;
  CF_RUN("attention", cf::launch_attention(at, st));
  if (at.sched) CF_RUN("attn_merge", cf::launch_attention_merge(at, st));
  if (mass) {
    cf::QMassArgs qm{};
    qm.q = Q; qm.ldq = qd; qm.n = n; qm.k = kc; qm.n_ctx = mass->n_ctx;
    qm.hq = m.n_q_heads; qm.hkv = m.n_kv_heads; qm.hd = hd;
    qm.ml = mass->ml; qm.part = mass->part; qm.score = mass->score;
    CF_RUN("query_mass", cf::launch_query_mass(dt, qm, mass->first ? 1 : 0, st));
  }

  float* part = reinterpret_cast<float*>(ws + lw.part);
  auto proj = [&](const cf::GemmPlan& pl, const void* A, int lda, const void* B, int K) {
    cf::GemmArgs r{};
    r.dt = dt; r.cfg = pl.cfg; r.splits = pl.splits;
    r.A = A; r.lda = lda; r.B[0] = r.B[1] = r.B[2] = B; r.nb0 = r.nb1 = d;
    r.M = n; r.N = d; r.K = K; r.L = L;
    return r;
  };
  // O projection + residual (+ the MLP RMSNorm when split-K needs a reduction pass anyway)
  cf::GemmArgs o = proj(P.o, AO, qd, w->wo, qd);
  if (o.splits > 1) {
    o.epi = cf::EPI_PARTIAL; o.C = part; o.ldc = d;
    CF_RUN("gemm/o", cf::launch_gemm(o, st));
    CF_RUN("reduce_resid_norm", cf::launch_reduce_resid_norm(dt, part, o.splits, n, d, hidden, sel, HS, nullptr, L,
                                                              w->mlp_norm, m.rms_eps, X, st));
  } else {
    o.epi = cf::EPI_RESID; o.resid = hidden; o.resid_rows = sel; o.out = HS; o.out_rows = nullptr;
    CF_RUN("gemm/o", cf::launch_gemm(o, st));
    CF_RUN("rmsnorm_rows", cf::launch_rmsnorm_rows(dt, HS, nullptr, n, n, d, w->mlp_norm, m.rms_eps, X, d, st));
  }

  cf::GemmArgs gu{};
  gu.dt = dt; gu.cfg = P.gu.cfg; gu.splits = 1;
  gu.A = X; gu.lda = d; gu.B[0] = w->w_gate; gu.B[1] = w->w_up; gu.B[2] = w->w_up;
  gu.M = n; gu.K = d;
  if (dt == cf::BF16) {
    gu.N = F; gu.nb0 = F; gu.nb1 = F; gu.epi = cf::EPI_SWIGLU; gu.act = ACT; gu.ld_act = F;
    CF_RUN("gemm/gate_up", cf::launch_gemm(gu, st));
  } else {
    float* GU = reinterpret_cast<float*>(ws + lw.gu);
    gu.N = 2 * F; gu.nb0 = F; gu.nb1 = 2 * F; gu.epi = cf::EPI_F32; gu.C = GU; gu.ldc = 2 * F;
    CF_RUN("gemm/gate_up", cf::launch_gemm(gu, st));
    CF_RUN("swiglu", cf::launch_swiglu(dt, GU, n, F, ACT, st));
  }
  // down projection + residual, written back to the selected rows
  cf::GemmArgs dn = proj(P.down, ACT, F, w->w_down, F);
  if (dn.splits > 1) {
    dn.epi = cf::EPI_PARTIAL; dn.C = part; dn.ldc = d;
    CF_RUN("gemm/down", cf::launch_gemm(dn, st));
    if (next_norm) {
      CF_RUN("reduce_resid_norm", cf::launch_reduce_resid_norm(dt, part, dn.splits, n, d, HS, nullptr, hidden, sel, L,
                                                                next_norm, m.rms_eps, X, st));
      if (x_next) *x_next = true;
    } else {
      CF_RUN("splitk_reduce", cf::launch_splitk_reduce(part, dn.splits, n, d, HS, nullptr, hidden, sel, L, st));
    }
  } else {
    dn.epi = cf::EPI_RESID; dn.resid = HS; dn.resid_rows = nullptr; dn.out = hidden; dn.out_rows = sel;
    CF_RUN("gemm/down", cf::launch_gemm(dn, st));
  }
  return CF_OK;
}

// Current keys of the N context rows at the selection layer and their deviation from the
// stitched keys (Request Order Matters §2.2 Eq. 1): X = RMSNorm(h[0..N)) in the model dtype,
// K = X Wk^T (fp32, `plan` picks the block shape and split-K factor), then qk-norm and RoPE at
// position i, and dev[i] = sum over the kvd entries of (K_i - k_ref[i])^2 in fp32. k_ref is the
// layer's stitched cache [>= N][kvd]; X holds N x d_model elements, KN splits x N x kvd floats.
cf_status enqueue_sel_deviation(const cf_ctx* c, const cf_layer_weights* w, const float* hidden, int N, int L,
                                const void* k_ref, float* dev, void* X, float* KN, const cf::GemmPlan& plan,
                                hipStream_t st) {
  const cf_model_cfg& mc = c->cfg;
  const cf::Dt dt = dt_of(c);
  const int kvd = mc.n_kv_heads * mc.head_dim;
  CF_RUN("rmsnorm_rows", cf::launch_rmsnorm_rows(dt, hidden, nullptr, N, L, mc.d_model, w->attn_norm, mc.rms_eps, X,
                                                 mc.d_model, st));
  cf::GemmArgs g{};
  g.dt = dt; g.cfg = plan.cfg; g.splits = plan.splits;
  g.A = X; g.lda = mc.d_model; g.B[0] = g.B[1] = g.B[2] = w->wk; g.nb0 = g.nb1 = kvd;
  g.M = N; g.N = kvd; g.K = mc.d_model; g.epi = g.splits > 1 ? cf::EPI_PARTIAL : cf::EPI_F32;
  g.C = KN; g.ldc = kvd;
  CF_RUN("gemm/k_sel", cf::launch_gemm(g, st));
  cf::QkvPost qp{};
  qp.qkv = KN; qp.ld = kvd; qp.rows = nullptr; qp.n = N; qp.L = L;
  qp.splits = g.splits; qp.split_stride = (int64_t)N * kvd;
  qp.hq = mc.n_q_heads; qp.hkv = mc.n_kv_heads; qp.hd = mc.head_dim; qp.qk_norm = mc.qk_norm;
  qp.qn = w->q_norm; qp.kn = w->k_norm; qp.eps = mc.rms_eps; qp.cos_t = c->cos_t; qp.sin_t = c->sin_t;
  qp.dev = dev; qp.k_ref = k_ref;
  CF_RUN("qkv_post/dev", cf::launch_qkv_post(dt, qp, st));
  return CF_OK;
}

cf_status check_ctx(const cf_ctx* c) {
  CF_CHECK(c, CF_EINVAL, "null context");
  return CF_OK;
}

cf_status check_chunks(const cf_ctx* c, const int32_t* tab, int m, int store_rows, int blend_rows,
                       int N_cover) {
  CF_CHECK(m >= 0 && m <= CF_MAX_CHUNKS, CF_EINVAL, "chunk count %d outside [0, %d]", m, CF_MAX_CHUNKS);
  CF_CHECK(m == 0 || tab, CF_EINVAL, "null chunk table");
  std::vector<std::pair<int, int>> dst;
  for (int i = 0; i < m; ++i) {
    const int row = tab[4 * i], src = tab[4 * i + 1], dp = tab[4 * i + 2], len = tab[4 * i + 3];
    CF_CHECK(len > 0, CF_EINVAL, "chunk %d: length %d", i, len);
    CF_CHECK(row >= 0 && (int64_t)row + len <= store_rows, CF_EINVAL, "chunk %d: store rows [%d, %d) outside [0, %d)",
             i, row, row + len, store_rows);
    CF_CHECK(dp >= 0 && (int64_t)dp + len <= blend_rows, CF_EINVAL, "chunk %d: rows [%d, %d) outside [0, %d)", i, dp,
             dp + len, blend_rows);
    CF_CHECK(src >= 0, CF_EINVAL, "chunk %d: negative source position", i);
    CF_CHECK(std::abs((int64_t)dp - src) < c->max_pos, CF_EINVAL, "chunk %d: offset %d not below max_pos %d", i,
             dp - src, c->max_pos);
    dst.push_back({dp, len});
  }
  std::sort(dst.begin(), dst.end());
  for (size_t i = 1; i < dst.size(); ++i)
    CF_CHECK(dst[i - 1].first + dst[i - 1].second <= dst[i].first, CF_EINVAL, "chunk destinations overlap");
  if (N_cover >= 0) {
    int at = 0;
    for (auto& p : dst) {
      CF_CHECK(p.first == at, CF_EINVAL, "chunks do not tile the context rows [0, %d)", N_cover);
      at += p.second;
    }
    CF_CHECK(at == N_cover, CF_EINVAL, "chunks cover %d rows, context has %d", at, N_cover);
  }
  return CF_OK;
}

cf_status enqueue_reposition(const cf_ctx* c, const void* ks, const void* vs, int64_t sls, void* kb, void* vb,
                             int64_t bls, const int32_t* tab, int m, int lb, int le, hipStream_t st) {
  const int kvd = c->cfg.n_kv_heads * c->cfg.head_dim;
  for (int c0 = 0; c0 < m; c0 += cf::CHUNKS_PER_LAUNCH) {
    cf::ChunkBatch cb{};
    cb.n = std::min(cf::CHUNKS_PER_LAUNCH, m - c0);
    cb.blk0[0] = 0;
    for (int i = 0; i < cb.n; ++i) {
      const int32_t* t = tab + 4 * (c0 + i);
      cb.row[i] = t[0];
      cb.dst[i] = t[2];
      cb.len[i] = t[3];
      cb.delta[i] = t[2] - t[1];
      cb.blk0[i + 1] = cb.blk0[i] + (t[3] + cf::REPOS_ROWS_PER_BLOCK - 1) / cf::REPOS_ROWS_PER_BLOCK;
    }
    CF_RUN("reposition", cf::launch_reposition(dt_of(c), ks, vs, sls, kb, vb, bls, cb, kvd, c->cfg.head_dim,
                                               c->cos_t, c->sin_t, lb, le - lb, st));
  }
  return CF_OK;
}

constexpr int SEL_GIVEN = CF_SEL_GIVEN;

bool span_mode(int mode) {
  return mode == CF_SEL_DOC_SPANS || mode == CF_SEL_RANKED_SPANS || mode == CF_SEL_SPAN_HEADS;
}

// Span bounds (and, for the ranked mode, the order after them: a permutation of the spans).
cf_status check_spans(const int32_t* b, int ns, int n, int mode = CF_SEL_DOC_SPANS) {
  CF_CHECK(ns >= 1 && ns <= CF_MAX_SPANS, CF_EINVAL, "span count %d outside [1, %d]", ns, CF_MAX_SPANS);
  CF_CHECK(b, CF_EINVAL, "null span bounds");
  CF_CHECK(b[0] == 0 && b[ns] == n, CF_EINVAL, "span bounds must run from 0 to %d", n);
  for (int i = 0; i < ns; ++i) CF_CHECK(b[i] < b[i + 1], CF_EINVAL, "span bounds not strictly increasing at %d", i);
  if (mode == CF_SEL_RANKED_SPANS) {
    std::vector<char> seen(ns, 0);
    for (int r = 0; r < ns; ++r) {
      const int j = b[ns + 1 + r];
      CF_CHECK(j >= 0 && j < ns && !seen[j], CF_EINVAL, "span order is not a permutation of the %d spans", ns);
      seen[j] = 1;
    }
  }
  return CF_OK;
}

// Frees what a context holds (members not yet created are null); the context's device is current.
void destroy_ctx(cf_ctx* c) {
  if (c->copy_st) (void)hipStreamSynchronize(c->copy_st);
  for (hipEvent_t ev : {c->start_ev, c->copied[0], c->copied[1], c->done[0], c->done[1]})
    if (ev) (void)hipEventDestroy(ev);
  if (c->copy_st) (void)hipStreamDestroy(c->copy_st);
  if (c->cos_t) (void)hipFree(c->cos_t);
  if (c->sin_t) (void)hipFree(c->sin_t);
  delete c;
}

cf_status enqueue_select(const float* dev, int n, int k, int mode, const int32_t* bounds, int ns, int* out,
                         double* ws, size_t ws_bytes, hipStream_t st) {
  if (k == 0) return CF_OK;
  if (mode == CF_SEL_TOKEN_TOPK) {
    CF_RUN("topk_token", cf::launch_topk_token(dev, n, k, out, ws, ws_bytes, st));
  } else {
    cf::SpanArgs sp{};
    sp.n_spans = ns;
    sp.mode = mode == CF_SEL_RANKED_SPANS ? cf::SPAN_RANKED : mode == CF_SEL_SPAN_HEADS ? cf::SPAN_HEADS : cf::SPAN_DOC;
    for (int i = 0; i <= ns; ++i) sp.b[i] = bounds[i];
    if (mode == CF_SEL_RANKED_SPANS)
      for (int r = 0; r < ns; ++r) sp.order[r] = bounds[ns + 1 + r];
    CF_RUN("topk_spans", cf::launch_topk_spans(dev, n, k, sp, out, ws, st));
  }
  return CF_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* cf_last_error(void) { return g_err.c_str(); }

const char* cf_version(void) { return "libcf 0.1 (gfx950)"; }

cf_status cf_mfma_loop(int32_t device, int32_t blocks_per_cu, int32_t iters, float* out, double* flops,
                       hipStream_t st) {
  g_err.clear();
  CF_CHECK(blocks_per_cu >= 1 && blocks_per_cu <= 64 && iters >= 1, CF_EINVAL, "need 1 <= blocks_per_cu <= 64, iters >= 1");
  CF_CHECK(out && flops, CF_EINVAL, "null pointer");
  DeviceGuard guard(device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  int n_cu = 0;
  CF_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && n_cu > 0,
           CF_EHIP, "cannot query the CU count");
  *flops = cf::launch_mfma_loop(blocks_per_cu * n_cu, iters, out, st);
  CF_CHECK(hipGetLastError() == hipSuccess, CF_EHIP, "launch failed");
  return CF_OK;
}

cf_status cf_copy_loop(int32_t device, const void* src, void* dst, int64_t bytes, hipStream_t st) {
  g_err.clear();
  CF_CHECK(src && dst && aligned16(src) && aligned16(dst), CF_EINVAL, "pointers must be non-null and 16-byte aligned");
  CF_CHECK(bytes >= 0 && bytes % 16 == 0, CF_EINVAL, "bytes must be a non-negative multiple of 16");
  const char *s = (const char*)src, *d = (const char*)dst;
  CF_CHECK(s + bytes <= d || d + bytes <= s, CF_EINVAL, "source and destination overlap");
  if (bytes == 0) return CF_OK;
  DeviceGuard guard(device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  cf::launch_copy_loop(src, dst, bytes / 16, st);
  CF_CHECK(hipGetLastError() == hipSuccess, CF_EHIP, "launch failed");
  return CF_OK;
}

cf_status cf_profile_enable(int32_t on) {
  g_err.clear();
  g_prof = on != 0;
  return CF_OK;
}

const char* cf_profile_report(void) {
  std::vector<std::pair<std::string, std::pair<long, double>>> acc;
  for (const ProfRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) ms = -1.f;
    auto it = std::find_if(acc.begin(), acc.end(), [&](const auto& p) { return p.first == r.name; });
    if (it == acc.end()) {
      acc.push_back({r.name, {0, 0.0}});
      it = acc.end() - 1;
    }
    it->second.first += 1;
    it->second.second += ms;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_report = "{";
  char buf[160];
  for (size_t i = 0; i < acc.size(); ++i) {
    snprintf(buf, sizeof buf, "%s\"%s\": [%ld, %.6f]", i ? ", " : "", acc[i].first.c_str(), acc[i].second.first,
             acc[i].second.second);
    g_report += buf;
  }
  g_report += "}";
  return g_report.c_str();
}

cf_status cf_ctx_create(const cf_model_cfg* cfg, int32_t max_pos, int32_t device, cf_ctx** out) {
  g_err.clear();
  CF_CHECK(cfg && out, CF_EINVAL, "null argument");
  const cf_model_cfg& m = *cfg;
  CF_CHECK(m.dtype == CF_F32 || m.dtype == CF_BF16, CF_EDTYPE, "unknown dtype %d", m.dtype);
  CF_CHECK(m.n_layers > 0 && m.d_model > 0 && m.n_q_heads > 0 && m.n_kv_heads > 0 && m.d_ffn > 0 && m.vocab > 0,
           CF_ESHAPE, "non-positive model dimension");
  CF_CHECK(m.head_dim == 64 || m.head_dim == 128, CF_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", m.head_dim);
  CF_CHECK(m.n_q_heads % m.n_kv_heads == 0, CF_ESHAPE, "n_q_heads %% n_kv_heads != 0");
  CF_CHECK(m.n_q_heads / m.n_kv_heads <= 16 && 64 % (m.n_q_heads / m.n_kv_heads) == 0, CF_EUNSUPPORTED,
           "query heads per kv head must divide 64 and be <= 16");
  CF_CHECK(m.d_model % 8 == 0 && m.d_ffn % 8 == 0, CF_EUNSUPPORTED, "d_model and d_ffn must be multiples of 8");
  CF_CHECK(m.rope_theta > 0.f && m.rms_eps >= 0.f, CF_EINVAL, "bad rope_theta or rms_eps");
  CF_CHECK(max_pos > 0, CF_EINVAL, "max_pos must be positive");
  int ndev = 0;
  CF_HIP(hipGetDeviceCount(&ndev));
  CF_CHECK(device >= 0 && device < ndev, CF_EINVAL, "device %d outside [0, %d)", device, ndev);
  DeviceGuard guard(device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice(%d) failed", device);
  cf_ctx* c = new cf_ctx{};
  c->cfg = m;
  c->device = device;
  c->max_pos = max_pos;
  if (hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || c->n_cu <= 0)
    c->n_cu = 256;
  const int half = m.head_dim / 2;
  std::vector<float> cs((size_t)max_pos * half), sn((size_t)max_pos * half);
  for (int p = 0; p < max_pos; ++p)
    for (int j = 0; j < half; ++j) {
      const double omega = std::pow((double)m.rope_theta, -2.0 * j / (double)m.head_dim);
      const double ang = (double)p * omega;
      cs[(size_t)p * half + j] = (float)std::cos(ang);
      sn[(size_t)p * half + j] = (float)std::sin(ang);
    }
  const size_t bytes = cs.size() * sizeof(float);
  hipError_t e = hipMalloc(&c->cos_t, bytes);
  if (e == hipSuccess) e = hipMalloc(&c->sin_t, bytes);
  if (e == hipSuccess) e = hipMemcpy(c->cos_t, cs.data(), bytes, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->sin_t, sn.data(), bytes, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->copy_st, hipStreamNonBlocking);
  hipEvent_t* evs[] = {&c->start_ev, &c->copied[0], &c->copied[1], &c->done[0], &c->done[1]};
  for (hipEvent_t* ev : evs)
    if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    destroy_ctx(c);
    return fail(CF_EHIP, "context set-up: %s", hipGetErrorString(e));
  }
  *out = c;
  return CF_OK;
}

void cf_ctx_destroy(cf_ctx* c) {
  if (!c) return;
  DeviceGuard guard(c->device);
  destroy_ctx(c);
}

cf_status cf_rope_reposition(const cf_ctx* c, const void* k_store, const void* v_store, int64_t sls,
                             int32_t store_rows, void* k_blend, void* v_blend, int64_t bls, int32_t blend_rows,
                             const int32_t* tab, int32_t m, int32_t lb, int32_t le, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  const int64_t kvd = (int64_t)c->cfg.n_kv_heads * c->cfg.head_dim;
  CF_CHECK(lb >= 0 && lb <= le && le <= c->cfg.n_layers, CF_EINVAL, "layer range [%d, %d) outside [0, %d]", lb, le,
           c->cfg.n_layers);
  CF_CHECK(store_rows >= 0 && blend_rows >= 0, CF_EINVAL, "negative row count");
  if (cf_status s = check_chunks(c, tab, m, store_rows, blend_rows, -1)) return s;
  if (m == 0 || lb == le) return CF_OK;
  CF_CHECK(k_store && v_store && k_blend && v_blend, CF_EINVAL, "null cache pointer");
  CF_CHECK(aligned16(k_store) && aligned16(v_store) && aligned16(k_blend) && aligned16(v_blend), CF_EINVAL,
           "cache pointers must be 16-byte aligned");
  CF_CHECK(sls >= store_rows * kvd && bls >= blend_rows * kvd && sls % 8 == 0 && bls % 8 == 0, CF_ESHAPE,
           "layer strides must hold rows * kvd elements and be multiples of 8");
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  return enqueue_reposition(c, k_store, v_store, sls, k_blend, v_blend, bls, tab, m, lb, le, st);
}

cf_status cf_kv_deviation(const void* k_new, int32_t new_dtype, int64_t ld_new, const void* k_ref, int32_t ref_dtype,
                          int64_t ld_ref, float* dev, int32_t n_tok, int32_t kv_dim, hipStream_t st) {
  g_err.clear();
  CF_CHECK((new_dtype == CF_F32 || new_dtype == CF_BF16) && (ref_dtype == CF_F32 || ref_dtype == CF_BF16), CF_EDTYPE,
           "unknown dtype");
  CF_CHECK(n_tok >= 0 && kv_dim > 0 && kv_dim % 8 == 0, CF_ESHAPE, "kv_dim must be a positive multiple of 8");
  if (n_tok == 0) return CF_OK;
  CF_CHECK(k_new && k_ref && dev, CF_EINVAL, "null pointer");
  CF_CHECK(aligned16(k_new) && aligned16(k_ref), CF_EINVAL, "key pointers must be 16-byte aligned");
  CF_CHECK(ld_new >= kv_dim && ld_ref >= kv_dim && ld_new % 8 == 0 && ld_ref % 8 == 0, CF_ESHAPE,
           "row strides must be >= kv_dim and multiples of 8");
  CF_RUN("deviation", cf::launch_deviation(new_dtype == CF_BF16 ? cf::BF16 : cf::F32, k_new, ld_new,
                              ref_dtype == CF_BF16 ? cf::BF16 : cf::F32, k_ref, ld_ref, dev, n_tok, kv_dim, st));
  return CF_OK;
}

size_t cf_topk_workspace_size(int32_t n, int32_t mode) {
  if (n < 0) return 0;
  if (mode == CF_SEL_DOC_SPANS) return al((size_t)(n + 1) * 8);
  return mode == CF_SEL_TOKEN_TOPK ? al(cf::topk_token_ws_bytes(n)) : 0;
}

size_t cf_topk_workspace_min_size(int32_t n, int32_t mode) {
  if (n < 0) return 0;
  return mode == CF_SEL_TOKEN_TOPK ? cf::topk_token_ws_min_bytes(n) : cf_topk_workspace_size(n, mode);
}

cf_status cf_topk_select(const float* dev, int32_t n, int32_t k, int32_t mode, const int32_t* bounds, int32_t ns,
                         int32_t* out, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  CF_CHECK(mode == CF_SEL_TOKEN_TOPK || span_mode(mode), CF_EINVAL, "mode %d is not a selection mode", mode);
  CF_CHECK(n >= 0 && k >= 0 && k <= n, CF_EINVAL, "need 0 <= k <= n (k=%d, n=%d)", k, n);
  if (span_mode(mode))
    if (cf_status s = check_spans(bounds, ns, n, mode)) return s;
  const size_t need = cf_topk_workspace_min_size(n, mode);
  CF_CHECK(k == 0 || need == 0 || (ws && ws_bytes >= need), CF_EWORKSPACE,
           "this selection needs at least %zu workspace bytes", need);
  if (k == 0) return CF_OK;
  CF_CHECK(dev && out, CF_EINVAL, "null pointer");
  return enqueue_select(dev, n, k, mode, bounds, ns, out, reinterpret_cast<double*>(ws), ws_bytes, st);
}

cf_status cf_topk_select_noalloc(const float* dev, int32_t n, int32_t k, int32_t mode, const int32_t* bounds,
                                 int32_t ns, int32_t* out, hipStream_t st) {
  g_err.clear();
  CF_CHECK(mode == CF_SEL_TOKEN_TOPK || span_mode(mode), CF_EINVAL, "mode %d is not a selection mode", mode);
  CF_CHECK(n >= 0 && k >= 0 && k <= n, CF_EINVAL, "need 0 <= k <= n (k=%d, n=%d)", k, n);
  if (span_mode(mode))
    if (cf_status s = check_spans(bounds, ns, n, mode)) return s;
  // token mode's candidate list takes what the scratch holds beyond the minimum
  const size_t need = cf_topk_workspace_min_size(n, mode);
  CF_CHECK(need <= CF_NOALLOC_SCRATCH_BYTES, CF_EWORKSPACE,
           "this selection needs %zu scratch bytes; the fixed scratch holds %u", need, CF_NOALLOC_SCRATCH_BYTES);
  if (k == 0) return CF_OK;
  CF_CHECK(dev && out, CF_EINVAL, "null pointer");
  void* ws = nullptr;
  if (need > 0) CF_HIP(cf::noalloc_scratch(&ws));
  return enqueue_select(dev, n, k, mode, bounds, ns, out, reinterpret_cast<double*>(ws), CF_NOALLOC_SCRATCH_BYTES,
                        st);
}

size_t cf_blend_layer_workspace_size(const cf_ctx* c, int32_t L, int32_t n_sel) {
  if (!c || L <= 0 || n_sel < 0) return 0;
  return layer_ws(c, L, std::min(n_sel, L)).total;
}

cf_status cf_blend_layer(const cf_ctx* c, const cf_layer_weights* w, float* hidden, void* kc, void* vc,
                         const int32_t* sel, int32_t n_sel, int32_t L, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  CF_CHECK(L > 0 && L <= c->max_pos, CF_EINVAL, "L=%d outside [1, max_pos=%d]", L, c->max_pos);
  CF_CHECK(n_sel >= 0 && n_sel <= L, CF_EINVAL, "n_sel=%d outside [0, L=%d]", n_sel, L);
  if (cf_status s = check_layer(c, w, 0)) return s;
  if (n_sel == 0) return CF_OK;
  CF_CHECK(hidden && kc && vc && sel, CF_EINVAL, "null pointer");
  CF_CHECK(aligned16(hidden) && aligned16(kc) && aligned16(vc), CF_EINVAL, "buffers must be 16-byte aligned");
  LayerWs lw = layer_ws(c, L, n_sel);
  CF_CHECK(ws && aligned16(ws) && ws_bytes >= lw.total, CF_EWORKSPACE, "workspace: need %zu bytes, got %zu", lw.total,
           ws_bytes);
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  return run_layer(c, w, hidden, kc, vc, sel, n_sel, L, static_cast<char*>(ws), lw, st);
}

size_t cf_selection_deviation_workspace_size(const cf_ctx* c, int32_t N) {
  if (!c || N <= 0) return 0;
  const cf_model_cfg& m = c->cfg;
  const int kvd = m.n_kv_heads * m.head_dim;
  const cf::GemmPlan p = cf::gemm_plan(dt_of(c), N, kvd, m.d_model, false, true, c->n_cu);
  return al((size_t)N * m.d_model * esize(c)) + al((size_t)p.splits * N * kvd * 4);
}

cf_status cf_selection_deviation(const cf_ctx* c, const cf_layer_weights* w, const float* hidden, int32_t N,
                                 const void* k_ref, float* dev, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  CF_CHECK(N >= 0 && N <= c->max_pos, CF_EINVAL, "N=%d outside [0, max_pos=%d]", N, c->max_pos);
  if (cf_status s = check_layer(c, w, 0)) return s;
  if (N == 0) return CF_OK;
  CF_CHECK(hidden && k_ref && dev, CF_EINVAL, "null pointer");
  CF_CHECK(aligned16(hidden) && aligned16(k_ref), CF_EINVAL, "hidden and k_ref must be 16-byte aligned");
  const size_t need = cf_selection_deviation_workspace_size(c, N);
  CF_CHECK(ws && aligned16(ws) && ws_bytes >= need, CF_EWORKSPACE, "workspace: need %zu bytes, got %zu", need,
           ws_bytes);
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  const cf_model_cfg& m = c->cfg;
  const int kvd = m.n_kv_heads * m.head_dim;
  const cf::GemmPlan p = cf::gemm_plan(dt_of(c), N, kvd, m.d_model, false, true, c->n_cu);
  char* W = static_cast<char*>(ws);
  return enqueue_sel_deviation(c, w, hidden, N, N, k_ref, dev, W, reinterpret_cast<float*>(
                               W + al((size_t)N * m.d_model * esize(c))), p, st);
}

size_t cf_blend_prefill_workspace_size(const cf_ctx* c, int32_t N, int32_t U, int32_t k, int32_t mode) {
  if (!c || N < 0 || U < 0 || N + U <= 0) return 0;
  if (mode == CF_SEL_ALL) k = N;
  return prefill_ws(c, N, U, std::max(0, std::min(k, N)), mode).total;
}

}  // extern "C"

namespace {

// The blended prefill of cf_blend_prefill, and with ks (host, n_layers - s_layer counts) the
// gradual filtering of cf_blend_prefill_gradual: out_sel then receives every layer's set and
// out_dev the selection-layer deviation followed by each later layer's deviation over its set.
bool pinned_host(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // not a HIP allocation: clear the error so no later call reports it
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

// host_store: k_store/v_store are pinned host memory (cf_blend_prefill_streamed).
cf_status prefill(const cf_ctx* c, const cf_layer_weights* layers, const void* embed, const float* final_norm,
                  const int32_t* tokens, int32_t N, int32_t U, const void* k_store, const void* v_store, int64_t sls,
                  int32_t store_rows, const int32_t* tab, int32_t m, int32_t s_layer, int32_t k, int32_t mode,
                  const int32_t* bounds, int32_t ns, const int32_t* ks, void* k_out, void* v_out, int64_t ols,
                  float* out_hidden, int32_t* out_sel, float* out_dev, void* ws, size_t ws_bytes, hipStream_t st,
                  bool host_store = false) {
  if (cf_status s = check_ctx(c)) return s;
  const cf_model_cfg& mc = c->cfg;
  const int L = N + U;
  const int64_t kvd = (int64_t)mc.n_kv_heads * mc.head_dim;
  CF_CHECK(N >= 0 && U >= 0 && L > 0, CF_EINVAL, "need N, U >= 0 and N + U > 0");
  CF_CHECK(L <= c->max_pos, CF_EINVAL, "L=%d exceeds max_pos=%d", L, c->max_pos);
  CF_CHECK(mode == CF_SEL_TOKEN_TOPK || span_mode(mode) || mode == CF_SEL_ALL || mode == SEL_GIVEN, CF_EINVAL,
           "unknown mode %d", mode);
  CF_CHECK(mode != SEL_GIVEN || k == 0 || out_sel, CF_EINVAL, "mode CF_SEL_GIVEN reads the set from out_sel");
  CF_CHECK(layers, CF_EINVAL, "null layer array");
  for (int l = 0; l < mc.n_layers; ++l)
    if (cf_status s = check_layer(c, layers + l, l)) return s;
  CF_CHECK(embed && final_norm && tokens, CF_EINVAL, "null embed, final_norm or tokens");
  CF_CHECK(aligned16(embed), CF_EINVAL, "embedding must be 16-byte aligned");
  CF_CHECK(k_out && v_out && aligned16(k_out) && aligned16(v_out), CF_EINVAL, "k_out/v_out null or misaligned");
  CF_CHECK(ols >= L * kvd && ols % 8 == 0, CF_ESHAPE, "out_layer_stride must be >= L*kvd and a multiple of 8");
  CF_CHECK(U == 0 || out_hidden, CF_EINVAL, "out_hidden is NULL but U > 0");
  const bool full = mode == CF_SEL_ALL;
  if (!full) {
    CF_CHECK(s_layer >= 0 && s_layer < mc.n_layers, CF_EINVAL, "sel_layer %d outside [0, %d)", s_layer, mc.n_layers);
    CF_CHECK(k >= 0 && k <= N, CF_EINVAL, "k=%d outside [0, N=%d]", k, N);
    if (N > 0) {
      CF_CHECK(k_store && v_store && aligned16(k_store) && aligned16(v_store), CF_EINVAL,
               "chunk store null or misaligned");
      if (host_store)
        CF_CHECK(pinned_host(k_store) && pinned_host(v_store), CF_EINVAL,
                 "the chunk store must be pinned host memory (hipHostMalloc)");
      CF_CHECK(store_rows >= 0 && sls >= store_rows * kvd && sls % 8 == 0, CF_ESHAPE,
               "store_layer_stride must hold store_rows*kvd elements and be a multiple of 8");
    }
    if (cf_status s = check_chunks(c, tab, m, store_rows, N, N)) return s;
    if (span_mode(mode) && N > 0)
      if (cf_status s = check_spans(bounds, ns, N, mode)) return s;
  } else {
    k = N;
  }
  const int nks = mc.n_layers - s_layer;
  if (ks) {
    CF_CHECK(mode == CF_SEL_TOKEN_TOPK, CF_EINVAL, "gradual filtering ranks single tokens (token mode)");
    CF_CHECK(ks[0] == k, CF_EINVAL, "k_sched[0]=%d must equal k=%d", ks[0], k);
    for (int i = 1; i < nks; ++i)
      CF_CHECK(ks[i] >= 0 && ks[i] <= ks[i - 1], CF_EINVAL, "k_sched must be non-increasing and >= 0 (entry %d)", i);
  }
  const bool streamed = host_store && !full && N > 0;
  const PrefillWs pw = prefill_ws(c, N, U, k, mode, ks, ks ? nks : 0, streamed ? store_rows : 0);
  CF_CHECK(ws && aligned16(ws) && ws_bytes >= pw.total, CF_EWORKSPACE, "workspace: need %zu bytes, got %zu", pw.total,
           ws_bytes);
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");

  char* W = static_cast<char*>(ws);
  float* hidden = reinterpret_cast<float*>(W + pw.hidden);
  int* sel = reinterpret_cast<int*>(W + pw.sel);
  float* dev = reinterpret_cast<float*>(W + pw.dev);
  char* lws = W + pw.layer;
  int* ident = reinterpret_cast<int*>(W + pw.ident);
  const cf::Dt dt = dt_of(c);
  const LayerWs lw_full = layer_ws(c, L, L, full ? 0 : N);
  auto K_l = [&](int l) { return static_cast<char*>(k_out) + (size_t)l * ols * esize(c); };
  auto V_l = [&](int l) { return static_cast<char*>(v_out) + (size_t)l * ols * esize(c); };

  const int first_sel = full ? mc.n_layers : s_layer;
  if (!streamed && !full && N > 0 && first_sel < mc.n_layers)
    if (cf_status s = enqueue_reposition(c, k_store, v_store, sls, k_out, v_out, ols, tab, m, first_sel,
                                         mc.n_layers, st))
      return s;
  // Streamed store: on the copy stream, layer l's K/V go host -> slot (l - s) % 2 and are
  // re-positioned from there into k_out/v_out[l]; an event then marks layer l ready, and the
  // compute stream waits for it right before layer l. The copy stream's own order keeps a slot
  // from being refilled (layer l + 2) before its re-position has read it, so the compute stream
  // records nothing. The copy stream starts after the caller's earlier work on `st` (the slots
  // and k_out may still be in use by a previous call) and runs up to two layers ahead of the
  // compute. If the call fails after the copy stream has started, the guard below makes `st`
  // wait for everything queued on it, so the caller's buffers are stream-ordered either way.
  struct CopyJoin {
    const cf_ctx* c;
    hipStream_t st;
    bool on;
    ~CopyJoin() {
      if (on && hipEventRecord(c->start_ev, c->copy_st) == hipSuccess) (void)hipStreamWaitEvent(st, c->start_ev, 0);
    }
  } join{c, st, false};
  const size_t slot_bytes = (size_t)store_rows * kvd * esize(c);
  auto slot_k = [&](int l) { return W + pw.stage + (size_t)((l - first_sel) % 2) * 2 * slot_bytes; };
  auto load_layer = [&](int l) -> cf_status {
    const size_t layer_off = (size_t)l * sls * esize(c);
    CF_HIP(hipMemcpyAsync(slot_k(l), static_cast<const char*>(k_store) + layer_off, slot_bytes,
                          hipMemcpyHostToDevice, c->copy_st));
    CF_HIP(hipMemcpyAsync(slot_k(l) + slot_bytes, static_cast<const char*>(v_store) + layer_off, slot_bytes,
                          hipMemcpyHostToDevice, c->copy_st));
    if (cf_status s = enqueue_reposition(c, slot_k(l), slot_k(l) + slot_bytes, 0, K_l(l), V_l(l), ols, tab, m, 0, 1,
                                         c->copy_st))
      return s;
    CF_HIP(hipEventRecord(c->copied[(l - first_sel) % 2], c->copy_st));
    return CF_OK;
  };
  auto stitch_layer = [&](int l) -> cf_status {
    if (!streamed) return CF_OK;
    CF_HIP(hipStreamWaitEvent(st, c->copied[(l - first_sel) % 2], 0));
    if (l + 2 < mc.n_layers) return load_layer(l + 2);  // its record of this parity comes after the wait
    return CF_OK;
  };
  if (streamed) {
    // One streamed call of this context in flight at a time: a call waits on the host for the
    // previous one to finish before it enqueues anything. Copies queued behind the work of an
    // earlier, still running call have stalled the enqueueing thread inside the runtime and
    // slowed the running call by up to a third; waiting costs only the start of this call's
    // enqueue (its first kernels go out within microseconds).
    const long long n = c->streamed_calls;
    if (n >= 1) CF_HIP(hipEventSynchronize(c->done[(n - 1) % 2]));
    CF_HIP(hipEventRecord(c->start_ev, st));
    CF_HIP(hipStreamWaitEvent(c->copy_st, c->start_ev, 0));
    join.on = true;
    for (int l = first_sel; l < std::min(first_sel + 2, mc.n_layers); ++l)
      if (cf_status s = load_layer(l)) return s;
  }
  CF_RUN("embed", cf::launch_embed(dt, tokens, L, embed, mc.vocab, mc.d_model, hidden, st));
  CF_RUN("iota", cf::launch_iota(ident, L, 0, st));
  // consecutive layers on the same rows hand the next attention-norm input over (see run_layer)
  bool xr = false, sched_full = false;
  for (int l = 0; l < first_sel; ++l) {
    const float* nn = l + 1 < first_sel ? layers[l + 1].attn_norm : nullptr;
    bool xn = false;
    if (cf_status s = run_layer(c, layers + l, hidden, K_l(l), V_l(l), ident, L, L, lws, lw_full, st, xr, nn, &xn,
                                &sched_full))
      return s;
    xr = xn;
  }

  if (!full) {
    const cf_layer_weights* w = layers + s_layer;
    const int n_sel = k + U;
    if (cf_status s = stitch_layer(s_layer)) return s;
    if (mode == SEL_GIVEN) {
      if (k > 0) CF_RUN("copy", cf::launch_copy_i32(sel, out_sel, k, st));
    } else if (N > 0) {
      // current keys of the context rows at the selection layer and their deviation
      // (the full-row layout holds N rows of X and of K)
      if (cf_status s = enqueue_sel_deviation(c, w, hidden, N, L, K_l(s_layer), dev, lws + lw_full.x,
                                              reinterpret_cast<float*>(lws + lw_full.qkv), lw_full.plan.ksel, st))
        return s;
      if (cf_status s = enqueue_select(dev, N, k, mode, bounds, ns, sel, reinterpret_cast<double*>(W + pw.topk),
                                       pw.topk_bytes, st))
        return s;
      if (out_dev) CF_RUN("copy", cf::launch_copy_f32(out_dev, dev, N, st));
      if (out_sel) CF_RUN("copy", cf::launch_copy_i32(out_sel, sel, k, st));
    }
    CF_RUN("iota", cf::launch_iota(sel + k, U, N, st));
    xr = false;
    bool sched_sel = false;
    if (!ks) {
      const LayerWs lw_sel = layer_ws(c, L, n_sel);
      for (int l = s_layer; l < mc.n_layers; ++l) {
        const float* nn = l + 1 < mc.n_layers ? layers[l + 1].attn_norm : nullptr;
        bool xn = false;
        if (l > s_layer)
          if (cf_status s = stitch_layer(l)) return s;
        if (cf_status s = run_layer(c, layers + l, hidden, K_l(l), V_l(l), sel, n_sel, L, lws, lw_sel, st, xr, nn,
                                    &xn, &sched_sel))
          return s;
        xr = xn;
      }
    } else {
      // gradual filtering: layer s + i recomputes ks[i] context rows. Layers s < l < Ly - 1 also
      // measure the deviation of their set (fused into the key store); when the next count is
      // smaller, the next set is the top of that deviation (at layer s: of the full ranking).
      int* cur = sel;
      int* nxt = reinterpret_cast<int*>(W + pw.sel2);
      float* dev2 = reinterpret_cast<float*>(W + pw.dev2);
      float* devh = reinterpret_cast<float*>(W + pw.devh);
      double* tkws = reinterpret_cast<double*>(W + pw.topk);
      size_t set_off = k, dev_off = N;
      for (int i = 0; i < nks; ++i) {
        const int l = s_layer + i, kl = ks[i];
        const bool last = i + 1 == nks;
        const bool narrows = !last && ks[i + 1] < kl;
        const LayerWs lw = layer_ws(c, L, kl + U);
        const float* nn = last || narrows ? nullptr : layers[l + 1].attn_norm;
        float* dh = i > 0 && !last && kl > 0 ? devh : nullptr;
        if (i > 0)
          if (cf_status s = stitch_layer(l)) return s;
        if (i > 0 && out_sel && kl > 0) CF_RUN("copy", cf::launch_copy_i32(out_sel + set_off, cur, kl, st));
        if (i > 0) set_off += kl;
        bool xn = false;
        if (cf_status s = run_layer(c, layers + l, hidden, K_l(l), V_l(l), cur, kl + U, L, lws, lw, st, xr, nn, &xn,
                                    &sched_sel, dh, kl))
          return s;
        xr = xn;
        if (dh) {
          CF_RUN("dev_rows", cf::launch_dev_rows(devh, kl, mc.n_kv_heads, dev2, st));
          if (out_dev) CF_RUN("copy", cf::launch_copy_f32(out_dev + dev_off, dev2, kl, st));
          dev_off += kl;
        }
        if (narrows) {
          const int kn = ks[i + 1];
          if (i == 0) {
            if (cf_status s = enqueue_select(dev, N, kn, CF_SEL_TOKEN_TOPK, nullptr, 0, nxt, tkws, pw.topk_bytes, st))
              return s;
            CF_RUN("iota", cf::launch_iota(nxt + kn, U, N, st));
          } else {
            if (cf_status s = enqueue_select(dev2, kl, kn, CF_SEL_TOKEN_TOPK, nullptr, 0, nxt, tkws, pw.topk_bytes, st))
              return s;
            CF_RUN("sel_map", cf::launch_sel_map(nxt, cur, kn, U, N, st));
          }
          std::swap(cur, nxt);
          sched_sel = false;
        }
      }
    }
  }
  if (U > 0)
    CF_RUN("rmsnorm_rows", cf::launch_rmsnorm_rows(cf::F32, hidden + (size_t)N * mc.d_model, nullptr, U, U, mc.d_model, final_norm,
                                   mc.rms_eps, out_hidden, mc.d_model, st));
  if (streamed) {
    join.on = false;  // every layer the copy stream loaded has been waited for on `st`
    CF_HIP(hipEventRecord(c->done[c->streamed_calls % 2], st));
    ++c->streamed_calls;
  }
  return CF_OK;
}

}  // namespace

extern "C" {

cf_status cf_blend_prefill(const cf_ctx* c, const cf_layer_weights* layers, const void* embed, const float* final_norm,
                           const int32_t* tokens, int32_t N, int32_t U, const void* k_store, const void* v_store,
                           int64_t sls, int32_t store_rows, const int32_t* tab, int32_t m, int32_t s_layer, int32_t k,
                           int32_t mode, const int32_t* bounds, int32_t ns, void* k_out, void* v_out, int64_t ols,
                           float* out_hidden, int32_t* out_sel, float* out_dev, void* ws, size_t ws_bytes,
                           hipStream_t st) {
  g_err.clear();
  return prefill(c, layers, embed, final_norm, tokens, N, U, k_store, v_store, sls, store_rows, tab, m, s_layer, k, mode,
                 bounds, ns, nullptr, k_out, v_out, ols, out_hidden, out_sel, out_dev, ws, ws_bytes, st);
}

namespace {

struct ScoresWs {
  size_t hidden, sel, ml, part, layer, total;
};

ScoresWs scores_ws(const cf_ctx* c, int N, int U) {
  const int L = N + U;
  ScoresWs p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  p.hidden = take((size_t)L * c->cfg.d_model * 4);
  p.sel = take((size_t)U * 4);
  p.ml = take((size_t)U * c->cfg.n_q_heads * 2 * 4);
  p.part = take((size_t)c->cfg.n_kv_heads * N * 4);
  p.layer = take(layer_ws(c, L, U).total);
  p.total = off;
  return p;
}

}  // namespace

size_t cf_query_scores_workspace_size(const cf_ctx* c, int32_t N, int32_t U) {
  if (!c || N <= 0 || U <= 0) return 0;
  return scores_ws(c, N, U).total;
}

cf_status cf_query_scores(const cf_ctx* c, const cf_layer_weights* layers, const void* embed, const int32_t* tokens,
                          int32_t N, int32_t U, void* k_cache, void* v_cache, int64_t ols, const int32_t* layer_set,
                          int32_t n_set, float* scores, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  const cf_model_cfg& mc = c->cfg;
  const int L = N + U;
  const int64_t kvd = (int64_t)mc.n_kv_heads * mc.head_dim;
  CF_CHECK(N > 0 && U > 0, CF_EINVAL, "need N > 0 context rows and U > 0 query rows");
  CF_CHECK(L <= c->max_pos, CF_EINVAL, "L=%d exceeds max_pos=%d", L, c->max_pos);
  CF_CHECK(layer_set && n_set > 0, CF_EINVAL, "empty layer set");
  for (int i = 0; i < n_set; ++i)
    CF_CHECK(layer_set[i] >= 0 && layer_set[i] < mc.n_layers && (i == 0 || layer_set[i] > layer_set[i - 1]), CF_EINVAL,
             "layer set must be strictly increasing layer ids in [0, %d)", mc.n_layers);
  const int last = layer_set[n_set - 1];
  for (int l = 0; l <= last; ++l)
    if (cf_status s = check_layer(c, layers + l, l)) return s;
  CF_CHECK(embed && tokens && scores && aligned16(embed), CF_EINVAL, "null or misaligned embed, tokens or scores");
  CF_CHECK(k_cache && v_cache && aligned16(k_cache) && aligned16(v_cache), CF_EINVAL, "cache null or misaligned");
  CF_CHECK(ols >= L * kvd && ols % 8 == 0, CF_ESHAPE, "layer stride must be >= L*kvd and a multiple of 8");
  const ScoresWs pw = scores_ws(c, N, U);
  CF_CHECK(ws && aligned16(ws) && ws_bytes >= pw.total, CF_EWORKSPACE, "workspace: need %zu bytes, got %zu", pw.total,
           ws_bytes);
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  char* W = static_cast<char*>(ws);
  float* hidden = reinterpret_cast<float*>(W + pw.hidden);
  int* sel = reinterpret_cast<int*>(W + pw.sel);
  const LayerWs lw = layer_ws(c, L, U);
  const cf::Dt dt = dt_of(c);
  // the query rows only: embeddings into rows N.., positions N..L-1
  CF_RUN("embed", cf::launch_embed(dt, tokens + N, U, embed, mc.vocab, mc.d_model, hidden + (size_t)N * mc.d_model, st));
  CF_RUN("iota", cf::launch_iota(sel, U, N, st));
  bool xr = false, sched = false;
  int set_i = 0;
  for (int l = 0; l <= last; ++l) {
    char* kl = static_cast<char*>(k_cache) + (size_t)l * ols * esize(c);
    char* vl = static_cast<char*>(v_cache) + (size_t)l * ols * esize(c);
    MassHook mh{reinterpret_cast<float*>(W + pw.ml), reinterpret_cast<float*>(W + pw.part), scores, N, set_i == 0};
    const bool scored = set_i < n_set && layer_set[set_i] == l;
    const float* nn = l < last ? layers[l + 1].attn_norm : nullptr;
    bool xn = false;
    if (cf_status s = run_layer(c, layers + l, hidden, kl, vl, sel, U, L, W + pw.layer, lw, st, xr, nn, &xn, &sched,
                                nullptr, 0, scored ? &mh : nullptr))
      return s;
    xr = xn;
    if (scored) ++set_i;
  }
  return CF_OK;
}

cf_status cf_key_norms(const cf_ctx* c, const void* k_store, int64_t sls, int32_t store_rows, int32_t lb, int32_t le,
                       float* norms, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  const int64_t kvd = (int64_t)c->cfg.n_kv_heads * c->cfg.head_dim;
  CF_CHECK(lb >= 0 && lb < le && le <= c->cfg.n_layers, CF_EINVAL, "layer range [%d, %d) outside [0, %d] or empty", lb,
           le, c->cfg.n_layers);
  CF_CHECK(store_rows >= 0, CF_EINVAL, "negative row count");
  if (store_rows == 0) return CF_OK;
  CF_CHECK(k_store && norms, CF_EINVAL, "null pointer");
  CF_CHECK(sls >= store_rows * kvd, CF_ESHAPE, "store_layer_stride must hold store_rows * kvd elements");
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  CF_RUN("key_norms", cf::launch_key_norms(dt_of(c), k_store, sls, store_rows, (int)kvd, lb, le, norms, st));
  return CF_OK;
}

namespace {

struct AnchoredWs {
  size_t hidden, sel, pos, kc, vc, ml, part, sched, layer, total;
};

AnchoredWs anchored_ws(const cf_ctx* c, int N, int U, int n_a) {
  const int R = n_a + U;
  const size_t kvd = (size_t)c->cfg.n_kv_heads * c->cfg.head_dim;
  AnchoredWs p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  p.hidden = take((size_t)R * c->cfg.d_model * 4);
  p.sel = take((size_t)U * 4);
  p.pos = take((size_t)U * 4);
  p.kc = take((size_t)R * kvd * esize(c));
  p.vc = take((size_t)R * kvd * esize(c));
  p.ml = take((size_t)U * c->cfg.n_q_heads * 2 * 4);
  p.part = take((size_t)c->cfg.n_kv_heads * N * 4);
  p.sched = take(sizeof(cf::AttnSched));
  p.layer = take(layer_ws(c, R, U).total);
  p.total = off;
  return p;
}

}  // namespace

size_t cf_query_scores_anchored_workspace_size(const cf_ctx* c, int32_t N, int32_t U, int32_t n_anchors) {
  if (!c || N <= 0 || U <= 0 || n_anchors < 0 || n_anchors > N) return 0;
  return anchored_ws(c, N, U, n_anchors).total;
}

cf_status cf_query_scores_anchored(const cf_ctx* c, const cf_layer_weights* layers, const void* embed,
                                   const int32_t* tokens, int32_t N, int32_t U, void* k_cache, void* v_cache,
                                   int64_t ols, const int32_t* anchors, int32_t n_a, const int32_t* layer_set,
                                   int32_t n_set, float* scores, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  const cf_model_cfg& mc = c->cfg;
  const int L = N + U, R = n_a + U;
  const int64_t kvd = (int64_t)mc.n_kv_heads * mc.head_dim;
  const int qd = mc.n_q_heads * mc.head_dim;
  CF_CHECK(N > 0 && U > 0, CF_EINVAL, "need N > 0 context rows and U > 0 query rows");
  CF_CHECK(n_a >= 0 && n_a <= N, CF_EINVAL, "anchor count %d outside [0, N=%d]", n_a, N);
  CF_CHECK(n_a == 0 || anchors, CF_EINVAL, "null anchor array");
  CF_CHECK(L <= c->max_pos, CF_EINVAL, "L=%d exceeds max_pos=%d", L, c->max_pos);
  CF_CHECK(layer_set && n_set > 0, CF_EINVAL, "empty layer set");
  for (int i = 0; i < n_set; ++i)
    CF_CHECK(layer_set[i] >= 0 && layer_set[i] < mc.n_layers && (i == 0 || layer_set[i] > layer_set[i - 1]), CF_EINVAL,
             "layer set must be strictly increasing layer ids in [0, %d)", mc.n_layers);
  const int last = layer_set[n_set - 1];
  for (int l = 0; l <= last; ++l)
    if (cf_status s = check_layer(c, layers + l, l)) return s;
  CF_CHECK(embed && tokens && scores && aligned16(embed), CF_EINVAL, "null or misaligned embed, tokens or scores");
  CF_CHECK(k_cache && v_cache && aligned16(k_cache) && aligned16(v_cache), CF_EINVAL, "cache null or misaligned");
  CF_CHECK(ols >= L * kvd && ols % 8 == 0, CF_ESHAPE, "layer stride must be >= L*kvd and a multiple of 8");
  const AnchoredWs pw = anchored_ws(c, N, U, n_a);
  CF_CHECK(ws && aligned16(ws) && ws_bytes >= pw.total, CF_EWORKSPACE, "workspace: need %zu bytes, got %zu", pw.total,
           ws_bytes);
  DeviceGuard guard(c->device);
  CF_CHECK(guard.ok, CF_EHIP, "hipSetDevice failed");
  char* W = static_cast<char*>(ws);
  float* hidden = reinterpret_cast<float*>(W + pw.hidden);
  int* sel = reinterpret_cast<int*>(W + pw.sel);   // the query rows in the compact cache: n_a .. R-1
  int* pos = reinterpret_cast<int*>(W + pw.pos);   // their request positions: N .. L-1
  char* kc = W + pw.kc;
  char* vc = W + pw.vc;
  float* ml = reinterpret_cast<float*>(W + pw.ml);
  cf::AttnSched* sched2 = reinterpret_cast<cf::AttnSched*>(W + pw.sched);
  char* lws = W + pw.layer;
  const LayerWs lw = layer_ws(c, R, U);
  const cf::Dt dt = dt_of(c);
  const size_t es = esize(c);
  // the query rows: embeddings into compact rows n_a.., RoPE at their request positions N..
  CF_RUN("embed", cf::launch_embed(dt, tokens + N, U, embed, mc.vocab, mc.d_model, hidden + (size_t)n_a * mc.d_model,
                                   st));
  CF_RUN("iota", cf::launch_iota(sel, U, n_a, st));
  CF_RUN("iota", cf::launch_iota(pos, U, N, st));
  bool xr = false, sched = false, sched_score = false;
  int set_i = 0;
  for (int l = 0; l <= last; ++l) {
    char* kl = static_cast<char*>(k_cache) + (size_t)l * ols * es;
    char* vl = static_cast<char*>(v_cache) + (size_t)l * ols * es;
    // compact anchor cache of this layer (QCFuse Eq. 16): the stitched rows at the anchors, whose
    // keys already carry the anchors' request positions; the query rows follow them
    CF_RUN("gather_rows", cf::launch_gather_rows(dt, kl, kvd, N, anchors, n_a, (int)kvd, kc, kvd, st));
    CF_RUN("gather_rows", cf::launch_gather_rows(dt, vl, kvd, N, anchors, n_a, (int)kvd, vc, kvd, st));
    const bool scored = set_i < n_set && layer_set[set_i] == l;
    const float* nn = l < last ? layers[l + 1].attn_norm : nullptr;
    bool xn = false;
    // the probe (Eq. 17): the query rows over the anchors and themselves, positions N.. for RoPE
    if (cf_status s = run_layer(c, layers + l, hidden, kc, vc, sel, U, R, lws, lw, st, xr, nn, &xn, &sched, nullptr,
                                0, nullptr, N - n_a))
      return s;
    xr = xn;
    if (!scored) continue;
    ++set_i;
    // scoring (Eq. 18, Eq. 20): the probe's query states of this layer against the full stitched
    // context keys; the query rows' own keys go to rows N..L-1 of the caller's cache, as in the
    // full-view probe, and their softmax runs over the context rows and the query rows up to each
    CF_RUN("gather_rows", cf::launch_gather_rows(dt, kc + (size_t)n_a * kvd * es, kvd, U, nullptr, U, (int)kvd,
                                                 kl + (size_t)N * kvd * es, kvd, st));
    CF_RUN("gather_rows", cf::launch_gather_rows(dt, vc + (size_t)n_a * kvd * es, kvd, U, nullptr, U, (int)kvd,
                                                 vl + (size_t)N * kvd * es, kvd, st));
    cf::AttnArgs at{};
    at.dt = dt; at.q = lws + lw.q; at.ldq = qd; at.pos = pos; at.n = U; at.k = kl; at.v = vl; at.L = L;
    at.hq = mc.n_q_heads; at.hkv = mc.n_kv_heads; at.hd = mc.head_dim; at.out = lws + lw.ao; at.ldo = qd;
    at.o_part = reinterpret_cast<float*>(lws + lw.opart);
    at.ml_part = reinterpret_cast<float*>(lws + lw.mlpart);
    if (lw.plan.attn_P > 0) {
      at.P = lw.plan.attn_P;
      if (!sched_score) CF_RUN("attn_sched", cf::launch_attention_sched(at, sched2, st));
      sched_score = true;
      at.sched = sched2;
    }
    at.ml_out = ml;
    CF_RUN("attention", cf::launch_attention(at, st));
    if (at.sched) CF_RUN("attn_merge", cf::launch_attention_merge(at, st));
    cf::QMassArgs qm{};
    qm.q = lws + lw.q; qm.ldq = qd; qm.n = U; qm.k = kl; qm.n_ctx = N;
    qm.hq = mc.n_q_heads; qm.hkv = mc.n_kv_heads; qm.hd = mc.head_dim;
    qm.ml = ml; qm.part = reinterpret_cast<float*>(W + pw.part); qm.score = scores;
    CF_RUN("query_mass", cf::launch_query_mass(dt, qm, set_i == 1 ? 1 : 0, st));
  }
  return CF_OK;
}

size_t cf_blend_prefill_streamed_workspace_size(const cf_ctx* c, int32_t N, int32_t U, int32_t k, int32_t mode,
                                                int32_t store_rows) {
  if (!c || N < 0 || U < 0 || N + U <= 0 || store_rows < 0) return 0;
  if (mode == CF_SEL_ALL) return prefill_ws(c, N, U, N, mode).total;
  return prefill_ws(c, N, U, std::max(0, std::min(k, N)), mode, nullptr, 0, N > 0 ? store_rows : 0).total;
}

cf_status cf_blend_prefill_streamed(const cf_ctx* c, const cf_layer_weights* layers, const void* embed,
                                    const float* final_norm, const int32_t* tokens, int32_t N, int32_t U,
                                    const void* k_store, const void* v_store, int64_t sls, int32_t store_rows,
                                    const int32_t* tab, int32_t m, int32_t s_layer, int32_t k, int32_t mode,
                                    const int32_t* bounds, int32_t ns, void* k_out, void* v_out, int64_t ols,
                                    float* out_hidden, int32_t* out_sel, float* out_dev, void* ws, size_t ws_bytes,
                                    hipStream_t st) {
  g_err.clear();
  return prefill(c, layers, embed, final_norm, tokens, N, U, k_store, v_store, sls, store_rows, tab, m, s_layer, k, mode,
                 bounds, ns, nullptr, k_out, v_out, ols, out_hidden, out_sel, out_dev, ws, ws_bytes, st, true);
}

size_t cf_blend_prefill_gradual_workspace_size(const cf_ctx* c, int32_t N, int32_t U, int32_t s_layer,
                                               const int32_t* k_sched) {
  if (!c || !k_sched || N < 0 || U < 0 || N + U <= 0 || s_layer < 0 || s_layer >= c->cfg.n_layers) return 0;
  const int nks = c->cfg.n_layers - s_layer;
  for (int i = 0; i < nks; ++i)
    if (k_sched[i] < 0 || k_sched[i] > N || (i && k_sched[i] > k_sched[i - 1])) return 0;
  return prefill_ws(c, N, U, k_sched[0], CF_SEL_TOKEN_TOPK, k_sched, nks).total;
}

cf_status cf_blend_prefill_gradual(const cf_ctx* c, const cf_layer_weights* layers, const void* embed,
                                   const float* final_norm, const int32_t* tokens, int32_t N, int32_t U,
                                   const void* k_store, const void* v_store, int64_t sls, int32_t store_rows,
                                   const int32_t* tab, int32_t m, int32_t s_layer, const int32_t* k_sched,
                                   void* k_out, void* v_out, int64_t ols, float* out_hidden, int32_t* out_sets,
                                   float* out_devs, void* ws, size_t ws_bytes, hipStream_t st) {
  g_err.clear();
  if (cf_status s = check_ctx(c)) return s;
  CF_CHECK(k_sched, CF_EINVAL, "null k_sched");
  CF_CHECK(s_layer >= 0 && s_layer < c->cfg.n_layers, CF_EINVAL, "sel_layer %d outside [0, %d)", s_layer,
           c->cfg.n_layers);
  return prefill(c, layers, embed, final_norm, tokens, N, U, k_store, v_store, sls, store_rows, tab, m, s_layer,
                 k_sched[0], CF_SEL_TOKEN_TOPK, nullptr, 0, k_sched, k_out, v_out, ols, out_hidden, out_sets, out_devs,
                 ws, ws_bytes, st);
}

}  // extern "C"
