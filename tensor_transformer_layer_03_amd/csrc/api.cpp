// C ABI of the tensor-parallel layer-shard library: argument validation,
// the layout of the forward->backward `saved` buffer, and the sequence of
// kernel launches of each entry point (see include/tp_layer.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/tp_layer.h"
#include "kernels.h"

using namespace tpl;

namespace {

// ------------------------------------------------------------------ validation

struct Dims {
  int64_t N;          // rows = micro_batch * seq
  int h, hr, fr, vr;  // hidden, per-rank hidden (heads_r*head_dim), per-rank ffn, per-rank vocab
  int heads_r, d;
  int dt;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }

tpl_status check_desc(const tpl_desc* d, Dims* out) {
  if (!d) return TPL_ERR_INVALID_ARG;
  if (d->dtype != TPL_F32 && d->dtype != TPL_BF16) return TPL_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->heads <= 0 || d->head_dim <= 0 || d->ffn <= 0 || d->vocab <= 0)
    return TPL_ERR_INVALID_ARG;
  if ((int64_t)d->heads * d->head_dim != d->hidden) return TPL_ERR_INVALID_ARG;
  if (d->tp < 1 || d->rank < 0 || d->rank >= d->tp) return TPL_ERR_INVALID_ARG;
  if (d->heads % d->tp || d->ffn % d->tp || d->vocab % d->tp) return TPL_ERR_INVALID_ARG;
  if (d->seq < 1 || d->micro_batch < 1) return TPL_ERR_INVALID_ARG;
  if (d->causal != 0 && d->causal != 1) return TPL_ERR_INVALID_ARG;
  if (!(d->ln_eps >= 0.f) || !std::isfinite(d->ln_eps)) return TPL_ERR_INVALID_ARG;
  const int fr = d->ffn / d->tp, vr = d->vocab / d->tp;
  if (d->hidden % 8 || fr % 8 || vr % 8) return TPL_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128) return TPL_ERR_UNSUPPORTED;
  // LayerNorm caches a row in registers: at most 32 16-byte chunks per lane.
  if (d->hidden > 64 * 32 * (d->dtype == TPL_BF16 ? 8 : 4)) return TPL_ERR_UNSUPPORTED;
  const int64_t N = (int64_t)d->seq * d->micro_batch;
  const int hr = d->heads / d->tp * d->head_dim;
  const int64_t widest = std::max<int64_t>({(int64_t)d->hidden, 3LL * hr, fr, vr});
  if (N * widest >= (1LL << 31) || N >= (1LL << 31) / 64) return TPL_ERR_INVALID_ARG;
  if (out) {
    out->N = N;
    out->h = d->hidden;
    out->hr = hr;
    out->fr = fr;
    out->vr = vr;
    out->heads_r = d->heads / d->tp;
    out->d = d->head_dim;
    out->dt = d->dtype == TPL_BF16 ? DT_BF16 : DT_F32;
  }
  return TPL_OK;
}

tpl_status from_hip(hipError_t e) { return e == hipSuccess ? TPL_OK : TPL_ERR_HIP; }
#define TPL_TRY(expr)                                        \
  do {                                                       \
    hipError_t e_ = (expr);                                  \
    if (e_ != hipSuccess) return TPL_ERR_HIP;                \
  } while (0)

GemmDesc gemm(const Dims& m, bool ak, bool bk, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
              const void* B, int64_t ldb, void* C, int64_t ldc) {
  GemmDesc g{};
  g.dtype = m.dt;
  g.a_kmajor = ak;
  g.b_kmajor = bk;
  g.epi = EPI_NONE;
  g.c_f32 = false;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda;
  g.B = B; g.ldb = ldb;
  g.C = C; g.ldc = ldc;
  g.C2 = nullptr; g.ldc2 = 0;
  g.bias = nullptr;
  return g;
}

// Workspace floats of a block's paired activation- and weight-gradient
// products (dg: [dM x dN] over dK; wg: [wM x wN] fp32 over wK), whether or
// not the pair is taken (the plan's split is fixed either way).
size_t pair_ws_floats(const Dims& m, int64_t dM, int64_t dN, int64_t dK, int epi, int64_t wM, int64_t wN, int64_t wK) {
  if (m.dt != DT_BF16) return 0;
  GemmDesc dg = gemm(m, true, false, dM, dN, dK, nullptr, dK, nullptr, dN, nullptr, dN);
  dg.epi = epi;
  GemmDesc wg = gemm(m, false, false, wM, wN, wK, nullptr, wM, nullptr, wN, nullptr, wN);
  wg.c_f32 = true;
  PairPlan plan;
  (void)gemm_pair_plan(dg, wg, &plan);
  return gemm_pair_ws_floats(dg, wg, plan);
}

// ------------------------------------------------------------------ saved layout
// Regions are 256-byte aligned. ATTN: mu, rstd [N] f32; y [N][h]; qkv [N][3hr];
// ctx [N][hr]; lse [b][a_r][s] f32; then backward scratch: dctx [N][hr],
// dqkv [N][3hr], delta [b][a_r][s] f32, ws (column partials, f32).
// MLP: mu, rstd; z [N][h]; GeLU'(u) [N][fr]; act [N][fr]; then du [N][fr], ws.
enum { S_MU, S_RSTD, S_Y, S_QKV, S_CTX, S_LSE, S_DCTX, S_DQKV, S_DELTA, S_WS, S_COUNT };
enum { S_Z = S_Y, S_GP = S_QKV, S_ACT = S_CTX, S_DU = S_DCTX };

struct Saved {
  size_t off[S_COUNT];
  size_t total;
};

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

Saved saved_layout(const Dims& m, tpl_block block) {
  Saved s{};
  const size_t es = dtype_size(m.dt);
  size_t sz[S_COUNT] = {0};
  sz[S_MU] = sz[S_RSTD] = m.N * 4;
  sz[S_Y] = m.N * m.h * es;
  size_t ws = layernorm_bwd_ws_floats(m.N, m.h);
  if (block == TPL_BLOCK_ATTN) {
    sz[S_QKV] = m.N * 3 * m.hr * es;
    sz[S_CTX] = m.N * m.hr * es;
    sz[S_LSE] = m.N * m.heads_r * 4;
    sz[S_DCTX] = m.N * m.hr * es;
    sz[S_DQKV] = m.N * 3 * m.hr * es;
    sz[S_DELTA] = m.N * m.heads_r * 4;
    ws = std::max(ws, colsum_ws_floats(m.N, 3 * m.hr));
    ws = std::max(ws, gemm_ws_floats(m.dt, m.h, m.hr, m.N));       // dW_o
    ws = std::max(ws, gemm_ws_floats(m.dt, 3 * m.hr, m.h, m.N));   // dW_qkv
    ws = std::max(ws, gemm_dgrad_ws_floats(m.dt, m.N, m.hr, m.h));  // dctx split over K
    // d_ln + dW_qkv, then db_qkv's column partials past the pair's workspace
    ws = std::max(ws, pair_ws_floats(m, m.N, m.h, 3 * m.hr, EPI_NONE, 3 * m.hr, m.h, m.N) +
                          colsum_ws_floats(m.N, 3 * m.hr));
    ws = std::max(ws, pair_ws_floats(m, m.N, m.hr, m.h, EPI_NONE, m.h, m.hr, m.N));           // dctx + dW_o
  } else {
    sz[S_GP] = m.N * m.fr * es;
    sz[S_ACT] = m.N * m.fr * es;
    sz[S_DU] = m.N * m.fr * es;
    ws = std::max(ws, colsum_ws_floats(m.N, m.fr));
    ws = std::max(ws, (size_t)gemm_colpart_chunks(m.dt, m.N, m.fr) * m.fr);   // db_1 partials of the du product
    ws = std::max(ws, pair_ws_floats(m, m.N, m.fr, m.h, EPI_DGELU, m.h, m.fr, m.N));   // du + dW_2
    ws = std::max(ws, pair_ws_floats(m, m.N, m.h, m.fr, EPI_NONE, m.fr, m.h, m.N));    // d_ln + dW_1
    ws = std::max(ws, gemm_ws_floats(m.dt, m.h, m.fr, m.N));       // dW_2
    ws = std::max(ws, gemm_ws_floats(m.dt, m.fr, m.h, m.N));       // dW_1
  }
  sz[S_WS] = ws * 4;
  size_t at = 0;
  for (int i = 0; i < S_COUNT; ++i) {
    s.off[i] = at;
    at += round256(sz[i]);
  }
  s.total = at;
  return s;
}

template <typename P>
P* slot(void* base, const Saved& s, int i) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + s.off[i]);
}

// Row statistics [N][3] at the head of the xent statistics buffer, padded to 256 B.
size_t xent_head_floats(int64_t rows) { return (size_t)((rows * 3 + 63) / 64) * 64; }


// ------------------------------------------------------------------ tracing state

struct TraceRec { int id; double work; hipEvent_t start, stop; };
std::mutex g_trace_mu;
std::vector<TraceRec> g_trace;   // pre-created event pairs
int g_trace_cap = 0, g_trace_used = 0;

const char* const kKernelNames[K_COUNT] = {
    "gemm_nt", "gemm_nn", "gemm_tn", "attn_fwd", "attn_bwd_pre", "attn_bwd_dq", "attn_bwd_dkdv",
    "layernorm_fwd", "layernorm_bwd", "layernorm_bwd_cols", "colsum", "colsum_final", "partial_sum",
    "xent_stats", "xent_finish", "xent_dlogits", "xent_merge", "embedding_fwd", "embedding_sort", "embedding_bwd",
    "rows_gather", "rows_expand", "gemm_pair", "attn_bwd_pair"};

}  // namespace

namespace tpl {
const char* kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : "unknown"; }

TraceScope::TraceScope(int kernel_id, hipStream_t s, double work) : slot(-1), stream(s) {
  if (g_trace_cap == 0) return;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  if (g_trace_used >= g_trace_cap) return;
  slot = g_trace_used++;
  g_trace[slot].id = kernel_id;
  g_trace[slot].work = work;
  (void)hipEventRecord(g_trace[slot].start, s);
}
TraceScope::~TraceScope() {
  if (slot >= 0) (void)hipEventRecord(g_trace[slot].stop, stream);
}
}  // namespace tpl

extern "C" {

const char* tpl_status_string(tpl_status st) {
  switch (st) {
    case TPL_OK: return "ok";
    case TPL_ERR_INVALID_ARG: return "invalid argument";
    case TPL_ERR_UNSUPPORTED: return "unsupported configuration";
    case TPL_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int32_t tpl_trace_enable(int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  for (auto& r : g_trace) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_trace.clear();
  g_trace_cap = 0;
  g_trace_used = 0;
  if (capacity <= 0) return 0;
  g_trace.resize(capacity);
  for (auto& r : g_trace) {
    r.id = -1;
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) return -1;
  }
  g_trace_cap = capacity;
  return capacity;
}

int32_t tpl_trace_read(int32_t* ids, float* ms, double* work, int32_t max_n) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  const int n = std::min(g_trace_used, max_n);
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(g_trace[i].stop) != hipSuccess) return -1;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_trace[i].start, g_trace[i].stop) != hipSuccess) return -1;
    ids[i] = g_trace[i].id;
    ms[i] = t;
    if (work) work[i] = g_trace[i].work;
  }
  return n;
}

const char* tpl_trace_kernel_name(int32_t id) { return tpl::kernel_name(id); }

size_t tp_layer_saved_bytes(const tpl_desc* desc, tpl_block block) {
  Dims m;
  if (check_desc(desc, &m) != TPL_OK) return 0;
  if (block != TPL_BLOCK_ATTN && block != TPL_BLOCK_MLP) return 0;
  return saved_layout(m, block).total;
}

}  // extern "C"

namespace {
// The block's forward up to (not including) the row-parallel product: LN into
// `saved`, then ATTN: qkv = y W_qkv^T + b, attention -> ctx, LSE; MLP: u = z
// W_1^T + b, kept as GeLU'(u), and act = GeLU(u). Used by the forward and by the recomputing
// backward.
tpl_status fwd_stash(const Dims& m, const tpl_desc* desc, tpl_block block, const void* x, const tpl_block_params* p,
                     void* saved, const Saved& L, hipStream_t s) {
  float* mu = slot<float>(saved, L, S_MU);
  float* rstd = slot<float>(saved, L, S_RSTD);
  void* y = slot<char>(saved, L, S_Y);
  TPL_TRY(launch_layernorm_fwd(m.dt, x, p->ln_g, p->ln_b, y, mu, rstd, m.N, m.h, desc->ln_eps, s));
  if (block == TPL_BLOCK_ATTN) {
    void* qkv = slot<char>(saved, L, S_QKV);
    void* ctx = slot<char>(saved, L, S_CTX);
    GemmDesc g = gemm(m, true, true, m.N, 3 * m.hr, m.h, y, m.h, p->w_in, m.h, qkv, 3 * m.hr);
    g.epi = EPI_BIAS;
    g.bias = p->b_in;
    TPL_TRY(launch_gemm(g, s));
    AttnDesc a{};
    a.dtype = m.dt; a.batch = desc->micro_batch; a.heads = m.heads_r; a.seq = desc->seq;
    a.head_dim = m.d; a.causal = desc->causal;
    a.qkv = qkv; a.ld_qkv = 3 * m.hr; a.ctx = ctx; a.ld_ctx = m.hr;
    a.lse = slot<float>(saved, L, S_LSE);
    TPL_TRY(launch_attn_fwd(a, s));
  } else {
    void* gp = slot<char>(saved, L, S_GP);   // GeLU'(u), all the backward needs of u
    void* act = slot<char>(saved, L, S_ACT);
    GemmDesc g = gemm(m, true, true, m.N, m.fr, m.h, y, m.h, p->w_in, m.h, gp, m.fr);
    g.epi = EPI_BIAS_GELU;
    g.bias = p->b_in;
    g.C2 = act;
    g.ldc2 = m.fr;
    TPL_TRY(launch_gemm(g, s));
  }
  return TPL_OK;
}
}  // namespace

extern "C" {

tpl_status tp_layer_shard_fwd(const tpl_desc* desc, tpl_block block, const void* x,
                              const tpl_block_params* p, void* partial, void* saved, void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (block != TPL_BLOCK_ATTN && block != TPL_BLOCK_MLP) return TPL_ERR_INVALID_ARG;
  if (!p || !ok_ptr(x) || !ok_ptr(partial) || !ok_ptr(saved) || !ok_ptr(p->ln_g) || !ok_ptr(p->ln_b) ||
      !ok_ptr(p->w_in) || !ok_ptr(p->b_in) || !ok_ptr(p->w_out))
    return TPL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Saved L = saved_layout(m, block);
  st = fwd_stash(m, desc, block, x, p, saved, L, s);
  if (st != TPL_OK) return st;
  if (block == TPL_BLOCK_ATTN) {
    void* ctx = slot<char>(saved, L, S_CTX);
    TPL_TRY(launch_gemm(gemm(m, true, true, m.N, m.h, m.hr, ctx, m.hr, p->w_out, m.hr, partial, m.h), s));
  } else {
    void* act = slot<char>(saved, L, S_ACT);
    TPL_TRY(launch_gemm(gemm(m, true, true, m.N, m.h, m.fr, act, m.fr, p->w_out, m.fr, partial, m.h), s));
  }
  return TPL_OK;
}

tpl_status shard_partial_sum(const tpl_desc* desc, const void* const* partials, int32_t n, const void* bias,
                             const void* residual, void* out, int64_t rows, int32_t cols, void* stream) {
  if (!desc || (desc->dtype != TPL_F32 && desc->dtype != TPL_BF16)) return TPL_ERR_INVALID_ARG;
  if (!partials || n < 1 || n > 16 || rows < 0 || cols <= 0 || cols % 8 || !ok_ptr(out)) return TPL_ERR_INVALID_ARG;
  if (rows * (int64_t)cols >= (1LL << 40)) return TPL_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!ok_ptr(partials[i])) return TPL_ERR_INVALID_ARG;
  if ((bias && !aligned16(bias)) || (residual && !aligned16(residual))) return TPL_ERR_INVALID_ARG;
  if (rows == 0) return TPL_OK;
  const int dt = desc->dtype == TPL_BF16 ? DT_BF16 : DT_F32;
  return from_hip(launch_partial_sum(dt, partials, n, bias, residual, out, rows, cols,
                                     static_cast<hipStream_t>(stream)));
}

tpl_status tp_layer_shard_bwd(const tpl_desc* desc, tpl_block block, tpl_bwd_phase phase, const void* dy,
                              const void* d_ln_sum, const void* x, const tpl_block_params* p, void* saved,
                              void* d_ln_partial, void* dx, const tpl_block_grads* gr, void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (block != TPL_BLOCK_ATTN && block != TPL_BLOCK_MLP) return TPL_ERR_INVALID_ARG;
  if (phase != TPL_BWD_SHARD && phase != TPL_BWD_REPLICATED && phase != TPL_BWD_SHARD_RECOMPUTE)
    return TPL_ERR_INVALID_ARG;
  if (!p || !gr || !ok_ptr(dy) || !ok_ptr(saved)) return TPL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Saved L = saved_layout(m, block);
  float* ws = slot<float>(saved, L, S_WS);
  if (phase == TPL_BWD_SHARD_RECOMPUTE) {
    // activation recomputation: rebuild the forward stash from the block
    // input, then the shard backward as usual
    if (!ok_ptr(x) || !ok_ptr(p->ln_g) || !ok_ptr(p->ln_b) || !ok_ptr(p->b_in) || !ok_ptr(p->w_in))
      return TPL_ERR_INVALID_ARG;
    st = fwd_stash(m, desc, block, x, p, saved, L, s);
    if (st != TPL_OK) return st;
    phase = TPL_BWD_SHARD;
  }
  if (phase == TPL_BWD_REPLICATED) {
    if (!ok_ptr(d_ln_sum) || !ok_ptr(x) || !ok_ptr(dx) || !ok_ptr(p->ln_g) || !ok_ptr(gr->d_ln_g) ||
        !ok_ptr(gr->d_ln_b) || !ok_ptr(gr->d_b_out))
      return TPL_ERR_INVALID_ARG;
    return from_hip(launch_layernorm_bwd(m.dt, dy, d_ln_sum, x, slot<float>(saved, L, S_MU),
                                         slot<float>(saved, L, S_RSTD), p->ln_g, dx, gr->d_ln_g, gr->d_ln_b,
                                         gr->d_b_out, ws, m.N, m.h, s));
  }
  if (!ok_ptr(d_ln_partial) || !ok_ptr(p->w_in) || !ok_ptr(p->w_out) || !ok_ptr(gr->d_w_in) ||
      !ok_ptr(gr->d_b_in) || !ok_ptr(gr->d_w_out))
    return TPL_ERR_INVALID_ARG;
  const void* y = slot<char>(saved, L, S_Y);
  if (block == TPL_BLOCK_ATTN) {
    void* qkv = slot<char>(saved, L, S_QKV);
    void* ctx = slot<char>(saved, L, S_CTX);
    void* dctx = slot<char>(saved, L, S_DCTX);
    void* dqkv = slot<char>(saved, L, S_DQKV);
    // dctx = dy W_o (split over K through the workspace when its grid is
    // small: nothing else lives there yet) ; dW_o = dy^T ctx; the two in one
    // launch when that fills the CUs better (both may then split over K)
    GemmDesc gd = gemm(m, true, false, m.N, m.hr, m.h, dy, m.h, p->w_out, m.hr, dctx, m.hr);
    gd.ws = ws;
    gd.ws_floats = (L.total - L.off[S_WS]) / 4;   // the workspace is the last slot
    GemmDesc gw = gemm(m, false, false, m.h, m.hr, m.N, dy, m.h, ctx, m.hr, gr->d_w_out, m.hr);
    gw.c_f32 = true;
    gw.ws = ws;
    PairPlan po;
    if (gemm_pair_plan(gd, gw, &po)) {
      TPL_TRY(launch_gemm_pair(gd, gw, po, ws, s));
    } else {
      TPL_TRY(launch_gemm(gd, s));
      TPL_TRY(launch_gemm(gw, s));
    }
    AttnDesc a{};
    a.dtype = m.dt; a.batch = desc->micro_batch; a.heads = m.heads_r; a.seq = desc->seq;
    a.head_dim = m.d; a.causal = desc->causal;
    a.qkv = qkv; a.ld_qkv = 3 * m.hr; a.ctx = ctx; a.ld_ctx = m.hr;
    a.lse = slot<float>(saved, L, S_LSE);
    a.dctx = dctx; a.dqkv = dqkv; a.delta = slot<float>(saved, L, S_DELTA);
    TPL_TRY(launch_attn_bwd(a, s));
    // dW_qkv = dqkv^T y ; db_qkv = colsum(dqkv) ; d_ln = dqkv W_qkv (the two products
    // in one launch when that fills the CUs better)
    GemmDesc gq = gemm(m, false, false, 3 * m.hr, m.h, m.N, dqkv, 3 * m.hr, y, m.h, gr->d_w_in, m.h);
    gq.c_f32 = true;
    gq.ws = ws;
    const GemmDesc gqd = gemm(m, true, false, m.N, m.h, 3 * m.hr, dqkv, 3 * m.hr, p->w_in, m.h, d_ln_partial, m.h);
    PairPlan pq;
    if (gemm_pair_plan(gqd, gq, &pq)) {
      if (pq.wg_splits > 1) {
        // db_qkv's column partials in the launch that sums dW_qkv's split
        // slices, into the workspace past the pair's own
        float* wsc = ws + gemm_pair_ws_floats(gqd, gq, pq);
        const PairTail t{TAIL_COLSUM_PARTIALS, dqkv, 3 * m.hr, m.N, 0, (int)(3 * m.hr), wsc, nullptr};
        TPL_TRY(launch_gemm_pair(gqd, gq, pq, ws, s, &t));
        const int64_t nch = (int64_t)(colsum_ws_floats(m.N, 3 * m.hr) / (size_t)(3 * m.hr));
        TPL_TRY(launch_colsum_final(wsc, nch, 3 * m.hr, gr->d_b_in, s));
      } else {
        TPL_TRY(launch_gemm_pair(gqd, gq, pq, ws, s));
        TPL_TRY(launch_colsum(m.dt, dqkv, 3 * m.hr, m.N, 3 * m.hr, gr->d_b_in, ws, s));
      }
    } else {
      TPL_TRY(launch_gemm(gq, s));
      TPL_TRY(launch_colsum(m.dt, dqkv, 3 * m.hr, m.N, 3 * m.hr, gr->d_b_in, ws, s));
      TPL_TRY(launch_gemm(gqd, s));
    }
  } else {
    void* gp = slot<char>(saved, L, S_GP);
    void* act = slot<char>(saved, L, S_ACT);
    void* du = slot<char>(saved, L, S_DU);
    // du = (dy W_2) * GeLU'(u) (stored by the forward); db_1 = colsum(du) from the product's column
    // partials when it provides them (bf16), else a separate pass below
    GemmDesc g = gemm(m, true, false, m.N, m.fr, m.h, dy, m.h, p->w_out, m.fr, du, m.fr);
    g.epi = EPI_DGELU;
    g.C2 = gp;
    g.ldc2 = m.fr;
    GemmDesc g2 = gemm(m, false, false, m.h, m.fr, m.N, dy, m.h, act, m.fr, gr->d_w_out, m.fr);
    g2.c_f32 = true;
    g2.ws = ws;
    // the fc2 activation and weight gradients in one launch when that fills the
    // CUs better (the column partials then come in the paired tile's row blocks)
    PairPlan p2;
    const bool pair2 = gemm_pair_plan(g, g2, &p2);
    const int64_t cp = pair2 ? gemm_pair_colpart_chunks(m.N) : gemm_colpart_chunks(m.dt, m.N, m.fr);
    if (cp > 0) g.colpart = ws;
    if (pair2) {
      // db_1's final column sum in the launch that sums dW_2's split slices
      // when there is one
      const bool merge = cp > 0 && p2.wg_splits > 1;
      const PairTail t{TAIL_COLSUM_FINAL, nullptr, 0, 0, cp, (int)m.fr, ws, gr->d_b_in};
      TPL_TRY(launch_gemm_pair(g, g2, p2, ws, s, merge ? &t : nullptr));
      if (cp > 0 && !merge) TPL_TRY(launch_colsum_final(ws, cp, m.fr, gr->d_b_in, s));
    } else {
      TPL_TRY(launch_gemm(g, s));
      if (cp > 0) TPL_TRY(launch_colsum_final(ws, cp, m.fr, gr->d_b_in, s));
      TPL_TRY(launch_gemm(g2, s));
    }
    GemmDesc g1 = gemm(m, false, false, m.fr, m.h, m.N, du, m.fr, y, m.h, gr->d_w_in, m.h);
    g1.c_f32 = true;
    g1.ws = ws;
    const GemmDesc g1d = gemm(m, true, false, m.N, m.h, m.fr, du, m.fr, p->w_in, m.h, d_ln_partial, m.h);
    PairPlan p1;
    if (gemm_pair_plan(g1d, g1, &p1)) {
      TPL_TRY(launch_gemm_pair(g1d, g1, p1, ws, s));
      if (cp == 0) TPL_TRY(launch_colsum(m.dt, du, m.fr, m.N, m.fr, gr->d_b_in, ws, s));
    } else {
      TPL_TRY(launch_gemm(g1, s));
      if (cp == 0) TPL_TRY(launch_colsum(m.dt, du, m.fr, m.N, m.fr, gr->d_b_in, ws, s));
      TPL_TRY(launch_gemm(g1d, s));
    }
  }
  return TPL_OK;
}

size_t vocab_parallel_xent_stats_bytes(const tpl_desc* desc) {
  Dims m;
  if (check_desc(desc, &m) != TPL_OK) return 0;
  size_t floats = xent_head_floats(m.N);
  if (xent_gemm_tile_cols(m.dt, m.N, m.vr) > 0) floats += xent_part_floats(m.N, m.vr);
  return floats * sizeof(float);
}

tpl_status vocab_parallel_xent_fwd(const tpl_desc* desc, tpl_xent_phase phase, const void* hidden, const void* emb,
                                   const int32_t* targets, const uint8_t* loss_mask, void* logits, float* stats,
                                   const float* const* all_stats, float* lse, float* loss_rows, float* loss,
                                   void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (phase == TPL_XENT_LOCAL) {
    if (!ok_ptr(hidden) || !ok_ptr(emb) || !ok_ptr(targets) || !ok_ptr(logits) || !ok_ptr(stats))
      return TPL_ERR_INVALID_ARG;
    GemmDesc g = gemm(m, true, true, m.N, m.vr, m.h, hidden, m.h, emb, m.h, logits, m.vr);
    const int tcols = xent_gemm_tile_cols(m.dt, m.N, m.vr);
    if (tcols > 0) {
      // statistics fused into the product's epilogue, per tile column, then
      // merged per row; the tile statistics live behind the row statistics
      g.epi = EPI_XENT;
      g.targets = targets;
      g.v0 = (int64_t)desc->rank * m.vr;
      g.xpart = stats + xent_head_floats(m.N);
      TPL_TRY(launch_gemm(g, s));
      return from_hip(launch_xent_merge(m.dt, g.xpart, tcols, m.N, logits, m.vr, targets, g.v0, stats, s));
    }
    TPL_TRY(launch_gemm(g, s));
    return from_hip(launch_xent_stats(m.dt, logits, m.N, m.vr, targets, (int64_t)desc->rank * m.vr, stats, s));
  }
  if (phase != TPL_XENT_FINISH) return TPL_ERR_INVALID_ARG;
  if (!all_stats || desc->tp > 64 || !ok_ptr(lse) || !ok_ptr(loss_rows) || !ok_ptr(loss)) return TPL_ERR_INVALID_ARG;
  for (int i = 0; i < desc->tp; ++i)
    if (!ok_ptr(all_stats[i])) return TPL_ERR_INVALID_ARG;
  if (loss_mask && !aligned16(loss_mask)) return TPL_ERR_INVALID_ARG;
  return from_hip(launch_xent_finish(all_stats, desc->tp, m.N, loss_mask, lse, loss_rows, loss, s));
}

tpl_status vocab_parallel_xent_bwd(const tpl_desc* desc, const void* hidden, const void* emb, const int32_t* targets,
                                   const uint8_t* loss_mask, void* logits, const float* lse, const float* loss,
                                   float dloss, void* d_hidden_partial, float* d_emb, void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (!ok_ptr(hidden) || !ok_ptr(emb) || !ok_ptr(targets) || !ok_ptr(logits) || !ok_ptr(lse) || !ok_ptr(loss) ||
      !ok_ptr(d_hidden_partial) || !ok_ptr(d_emb) || !std::isfinite(dloss))
    return TPL_ERR_INVALID_ARG;
  if (loss_mask && !aligned16(loss_mask)) return TPL_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPL_TRY(launch_xent_dlogits(m.dt, logits, m.N, m.vr, targets, (int64_t)desc->rank * m.vr, loss_mask, lse, loss,
                              dloss, s));
  // dH first: it may use d_emb (written by dE right after) as split-K scratch
  GemmDesc gh = gemm(m, true, false, m.N, m.h, m.vr, logits, m.vr, emb, m.h, d_hidden_partial, m.h);
  gh.ws = d_emb;
  gh.ws_floats = (size_t)m.vr * m.h;
  TPL_TRY(launch_gemm(gh, s));
  GemmDesc ge = gemm(m, false, false, m.vr, m.h, m.N, logits, m.vr, hidden, m.h, d_emb, m.h);
  ge.c_f32 = true;
  return from_hip(launch_gemm(ge, s));
}

size_t vocab_parallel_embedding_ws_bytes(const tpl_desc* desc) {
  Dims m;
  if (check_desc(desc, &m) != TPL_OK) return 0;
  return round256(embedding_ws_bytes(m.N, (int)m.vr));
}

tpl_status vocab_parallel_embedding_fwd(const tpl_desc* desc, const int32_t* tokens, const void* emb_in,
                                        void* x_partial, void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (!ok_ptr(tokens) || !ok_ptr(emb_in) || !ok_ptr(x_partial)) return TPL_ERR_INVALID_ARG;
  return from_hip(launch_embedding_fwd(m.dt, tokens, emb_in, x_partial, m.N, (int)m.h, (int64_t)desc->rank * m.vr,
                                       (int)m.vr, static_cast<hipStream_t>(stream)));
}

tpl_status vocab_parallel_embedding_bwd(const tpl_desc* desc, const int32_t* tokens, const void* d_out,
                                        float* d_emb_in, void* workspace, void* stream) {
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (!ok_ptr(tokens) || !ok_ptr(d_out) || !ok_ptr(d_emb_in) || !ok_ptr(workspace)) return TPL_ERR_INVALID_ARG;
  return from_hip(launch_embedding_bwd(m.dt, tokens, d_out, d_emb_in, m.N, (int)m.h, (int64_t)desc->rank * m.vr,
                                       (int)m.vr, workspace, static_cast<hipStream_t>(stream)));
}

tpl_status vocab_parallel_embedding_bwd_noalloc(const tpl_desc* desc, const int32_t* tokens, const void* d_out,
                                                float* d_emb_in, void* stream) {
  static_assert(TPL_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "header and library disagree on the limit");
  Dims m;
  tpl_status st = check_desc(desc, &m);
  if (st != TPL_OK) return st;
  if (!ok_ptr(tokens) || !ok_ptr(d_out) || !ok_ptr(d_emb_in)) return TPL_ERR_INVALID_ARG;
  if (round256(embedding_ws_bytes(m.N, (int)m.vr)) > kNoAllocScratchBytes) return TPL_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return TPL_ERR_HIP;
  return from_hip(launch_embedding_bwd(m.dt, tokens, d_out, d_emb_in, m.N, (int)m.h, (int64_t)desc->rank * m.vr,
                                       (int)m.vr, ws, static_cast<hipStream_t>(stream)));
}

static bool ok_ptr4(const void* p) { return p != nullptr && reinterpret_cast<uintptr_t>(p) % 4 == 0; }

tpl_status tpl_rows_gather(const void* src, int64_t n_src, const int32_t* rows, int64_t n, int64_t row_bytes, void* dst,
                           void* stream) {
  if (n < 0 || n_src < 0 || row_bytes <= 0 || row_bytes % 4 || n >= (1LL << 40) / row_bytes) return TPL_ERR_INVALID_ARG;
  if (n > 0 && (!ok_ptr4(rows) || !ok_ptr4(dst) || (n_src > 0 && !ok_ptr4(src)))) return TPL_ERR_INVALID_ARG;
  return from_hip(tpl::launch_rows_gather(src, rows, n, n_src, row_bytes, dst, static_cast<hipStream_t>(stream)));
}

tpl_status tpl_rows_expand(const void* src, int64_t n_src, const int32_t* pos, int64_t n_dst, int64_t row_bytes,
                           void* dst, void* stream) {
  if (n_dst < 0 || n_src < 0 || row_bytes <= 0 || row_bytes % 4 || n_dst >= (1LL << 40) / row_bytes)
    return TPL_ERR_INVALID_ARG;
  if (n_dst > 0 && (!ok_ptr4(pos) || !ok_ptr4(dst) || (n_src > 0 && !ok_ptr4(src)))) return TPL_ERR_INVALID_ARG;
  return from_hip(tpl::launch_rows_expand(src, pos, n_dst, n_src, row_bytes, dst, static_cast<hipStream_t>(stream)));
}

tpl_status tpl_gemm(int32_t dtype, int32_t a_kmajor, int32_t b_kmajor, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, const void* B, int64_t ldb, const void* bias, void* C, int64_t ldc, int32_t c_f32,
                    void* stream) {
  if (dtype != TPL_F32 && dtype != TPL_BF16) return TPL_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0 || M >= (1LL << 31) || N >= (1LL << 31) || K >= (1LL << 31)) return TPL_ERR_INVALID_ARG;
  if (N % 8 || (a_kmajor ? K % 8 : M % 8) || !ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C)) return TPL_ERR_INVALID_ARG;
  if (lda % 8 || ldb % 8 || ldc % 8) return TPL_ERR_INVALID_ARG;
  if (a_kmajor ? lda < K : lda < M) return TPL_ERR_INVALID_ARG;
  if (b_kmajor ? ldb < K : ldb < N) return TPL_ERR_INVALID_ARG;
  if (ldc < N || (bias && !aligned16(bias))) return TPL_ERR_INVALID_ARG;
  if (b_kmajor && !a_kmajor) return TPL_ERR_UNSUPPORTED;
  if (a_kmajor && b_kmajor && c_f32) return TPL_ERR_UNSUPPORTED;
  if (a_kmajor && !b_kmajor && (c_f32 || bias)) return TPL_ERR_UNSUPPORTED;
  if (!a_kmajor && !b_kmajor && (!c_f32 || bias)) return TPL_ERR_UNSUPPORTED;
  GemmDesc g{};
  g.dtype = dtype == TPL_BF16 ? DT_BF16 : DT_F32;
  g.a_kmajor = a_kmajor != 0;
  g.b_kmajor = b_kmajor != 0;
  g.epi = bias ? EPI_BIAS : EPI_NONE;
  g.c_f32 = c_f32 != 0;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc; g.bias = bias;
  return from_hip(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
