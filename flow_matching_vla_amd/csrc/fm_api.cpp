// Runtime behind the C ABI: validation, weight layout, the K/V pool, the schedule table,
// the per-step launch sequence and its capture into one hipGraph per (steps, batch,
// prefix length).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fm.h"
#include "fm_kernels.h"
#include "fm_xloop.h"

using namespace fm;

namespace {

thread_local std::string g_err;

std::string fmt(const char* f, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

long round_up(long x, long m) { return (x + m - 1) / m * m; }

struct Spec {
  std::string name;
  std::vector<int64_t> shape;
};

int n_sites(const fm_config& c) { return c.arch == FM_ARCH_PREFIX_JOINT ? 2 * c.n_layers + 1 : c.n_layers + 1; }

std::vector<Spec> weight_specs(const fm_config& c) {
  const int64_t D = c.hidden, F = c.mlp_dim, S = n_sites(c);
  std::vector<Spec> v = {
      {"time_in.w", {D, D}}, {"time_in.b", {D}}, {"time_out.w", {D, D}}, {"time_out.b", {D}},
      {"mod.w", {S, 3 * D, D}}, {"mod.b", {S, 3 * D}}, {"action_in.w", {D, c.action_dim}},
      {"action_in.b", {D}}, {"action_out.w", {c.action_dim, D}}, {"action_out.b", {c.action_dim}},
  };
  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    const int64_t qd = (int64_t)c.n_heads * c.head_dim, kd = (int64_t)c.n_kv_heads * c.head_dim;
    for (int l = 0; l < c.n_layers; ++l) {
      const std::string p = "layers." + std::to_string(l) + ".";
      v.push_back({p + "q.w", {qd, D}});
      v.push_back({p + "k.w", {kd, D}});
      v.push_back({p + "v.w", {kd, D}});
      v.push_back({p + "o.w", {D, qd}});
      v.push_back({p + "gate.w", {F, D}});
      if (c.mlp_gated) v.push_back({p + "up.w", {F, D}});
      v.push_back({p + "down.w", {D, F}});
    }
  } else {
    v.push_back({"time_bias.w", {D, D}});
    v.push_back({"time_bias.b", {D}});
    v.push_back({"state_in.w", {D, c.state_dim}});
    v.push_back({"state_in.b", {D}});
    for (int i = 0; i < c.n_layers; ++i) {
      const std::string p = "blocks." + std::to_string(i) + ".";
      const int64_t kin = (i % 2 == 0) ? c.ctx_dim : D;
      v.push_back({p + "q.w", {D, D}});
      v.push_back({p + "k.w", {D, kin}});
      v.push_back({p + "v.w", {D, kin}});
      v.push_back({p + "o.w", {D, D}});
      v.push_back({p + "ff1.w", {F, D}});
      v.push_back({p + "ff2.w", {D, F}});
    }
  }
  return v;
}

// Config validation (host only).
fm_status check_config(const fm_config* c, std::string& msg) {
  if (!c) { msg = "config is NULL"; return FM_ERR_INVALID_ARG; }
  if (c->arch != FM_ARCH_PREFIX_JOINT && c->arch != FM_ARCH_DIT_CROSS) { msg = fmt("arch %d unknown", c->arch); return FM_ERR_INVALID_ARG; }
  if (c->dtype != FM_F32 && c->dtype != FM_BF16) { msg = fmt("dtype %d unknown", c->dtype); return FM_ERR_INVALID_ARG; }
  if (c->n_layers < 1 || c->hidden < 64 || c->n_heads < 1 || c->head_dim < 1 || c->mlp_dim < 1 ||
      c->action_horizon < 1 || c->action_dim < 1 || c->max_batch < 1 || c->max_steps < 1 || c->n_kv_heads < 1) {
    msg = "n_layers, hidden (>= 64), heads, head_dim, mlp_dim, action_horizon, action_dim, n_kv_heads, max_batch and max_steps must be positive";
    return FM_ERR_INVALID_ARG;
  }
  // upper limits far above any expert the pages describe, so that every derived count and size
  // (weight list, pool and buffer bytes, products of fields) stays small and within range
  if (c->n_layers > 1024 || c->n_heads > 256 || c->n_kv_heads > 256 || c->mlp_dim > (1 << 16) ||
      c->action_horizon > 4096 || c->action_dim > 4096 || c->max_batch > 4096 || c->max_steps > 4096 ||
      c->max_prefix_len > (1 << 20) || c->state_tokens > 8 || c->state_dim > (1 << 16) || c->ctx_len_max > (1 << 20) ||
      c->ctx_dim > (1 << 16) || c->mlp_gated < 0) {
    msg = "a config field is out of range (n_layers <= 1024, heads <= 256, mlp_dim, state_dim, ctx_dim <= 65536, "
          "action_horizon, action_dim, max_batch, max_steps <= 4096, max_prefix_len, ctx_len_max <= 2^20)";
    return FM_ERR_INVALID_ARG;
  }
  if (c->hidden % 64 != 0 || c->hidden / kStatCols > kMaxStatSlots) { msg = fmt("hidden %d must be a multiple of 64 and at most %d", c->hidden, kStatCols * kMaxStatSlots); return FM_ERR_UNSUPPORTED; }
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) {
    msg = fmt("head_dim %d not in {64, 128, 256}", c->head_dim);
    return FM_ERR_UNSUPPORTED;
  }
  if (c->dtype == FM_F32 && c->head_dim == 256) { msg = "fp32 head_dim 256 is not built"; return FM_ERR_UNSUPPORTED; }
  const int kq = c->dtype == FM_BF16 ? 32 : 16;
  if (c->mlp_dim % kq != 0) { msg = fmt("mlp_dim %d must be a multiple of %d", c->mlp_dim, kq); return FM_ERR_UNSUPPORTED; }
  if (!(c->norm_eps >= 0.f) || !(c->rope_base >= 0.f)) { msg = "norm_eps and rope_base must be >= 0"; return FM_ERR_INVALID_ARG; }
  if (c->arch == FM_ARCH_PREFIX_JOINT) {
    if (c->n_kv_heads != 1) {
      msg = fmt("prefix-joint expert needs exactly one K/V head (got %d): the pool is one flat [capacity, head_dim] plane per request", c->n_kv_heads);
      return FM_ERR_UNSUPPORTED;
    }
    if (c->max_prefix_len < 0) { msg = "max_prefix_len must be >= 0"; return FM_ERR_INVALID_ARG; }
    if (c->state_tokens != 0 || c->ctx_len_max != 0) { msg = "state_tokens and ctx_len_max must be 0 for the prefix-joint expert"; return FM_ERR_INVALID_ARG; }
  } else {
    if (c->n_kv_heads != c->n_heads) { msg = fmt("DiT head needs n_kv_heads == n_heads (%d vs %d)", c->n_kv_heads, c->n_heads); return FM_ERR_UNSUPPORTED; }
    if (c->n_heads * c->head_dim != c->hidden) { msg = fmt("n_heads * head_dim (%d) must equal hidden (%d)", c->n_heads * c->head_dim, c->hidden); return FM_ERR_INVALID_ARG; }
    if (c->state_tokens < 0 || c->state_tokens > 8 || (c->state_tokens > 0 && c->state_dim < 1)) { msg = "state_tokens in [0, 8] with state_dim >= 1"; return FM_ERR_INVALID_ARG; }
    if (c->ctx_len_max < 1 || c->ctx_dim < 1 || c->ctx_dim % kq != 0) { msg = fmt("ctx_len_max >= 1 and ctx_dim a multiple of %d", kq); return FM_ERR_INVALID_ARG; }
    if (c->rope_base != 0.f) { msg = "RoPE is not used by the DiT head"; return FM_ERR_UNSUPPORTED; }
    if (c->mlp_gated) { msg = "the DiT feed-forward is not gated"; return FM_ERR_UNSUPPORTED; }
  }
  if (c->arch == FM_ARCH_PREFIX_JOINT && c->mlp_gated != 0 && c->mlp_gated != 1) { msg = "mlp_gated must be 0 or 1"; return FM_ERR_INVALID_ARG; }
  const int qcols = c->n_heads * c->head_dim;
  if (qcols % kq != 0) { msg = "n_heads * head_dim must be a multiple of the k chunk"; return FM_ERR_UNSUPPORTED; }
  return FM_OK;
}

int pool_capacity(const fm_config& c) { return (int)round_up((long)c.max_prefix_len + c.action_horizon, 256); }

struct Op {
  enum Kind { GEMM, ATTN, INPROJ, TRACE } kind;
  int role;  // FM_OP_* of include/fm.h
  GemmArgs g;
  AttnArgs at;
  InProjArgs ip;
  int trace_layer;
};

}  // namespace

struct fm_ctx {
  fm_config c;
  hipStream_t stream = nullptr, cap_stream = nullptr;
  int device = 0, num_cus = 256, elem = ET_BF16, esz = 2;
  std::string err;
  bool poisoned = false;

  // device memory owned by the context
  std::vector<void*> allocs;
  bool loaded = false;
  struct Layer {
    void *qkv = nullptr, *q = nullptr, *kx = nullptr, *vx = nullptr, *o = nullptr, *gu = nullptr, *down = nullptr;
    // FP8 weights (FM_WEIGHTS_FP8_E4M3): codes fragment-major and per-row scales of the same
    // matrices, streamed by the loop kernel and by the skinny GEMMs of the per-operation graph;
    // q, qkv .. down then hold the dequantized bf16 (for the large-M GEMMs and the schedule)
    void *q8 = nullptr, *qkv8 = nullptr, *o8 = nullptr, *gu8 = nullptr, *down8 = nullptr;
    float *sq = nullptr, *sqkv = nullptr, *so = nullptr, *sgu = nullptr, *sdown = nullptr;
  };
  std::vector<Layer> L;
  void *w_tin = nullptr, *w_tout = nullptr, *w_mod = nullptr, *w_tb = nullptr, *w_in = nullptr, *w_out = nullptr, *w_state = nullptr;
  float *b_tin = nullptr, *b_tout = nullptr, *b_mod = nullptr, *b_tb = nullptr, *b_in = nullptr, *b_out = nullptr, *b_state = nullptr;

  // schedule
  int steps = -1, sched_batch = 0;
  std::vector<float> tau;
  float *table = nullptr, *tbias = nullptr;
  void *e_buf = nullptr, *c1_buf = nullptr, *c_buf = nullptr, *row_buf = nullptr;
  // per step and norm site: c = shift W^T and (LayerNorm) d = (1 + scale) W^T of the
  // site's consumer weights, [max_steps][csum]; site s starts at c_off[s]
  float *cbuf = nullptr, *dbuf = nullptr, *dff = nullptr;
  std::vector<long> c_off;
  long csum = 0;

  // binding
  int bound_batch = 0, prefix_len = -1;
  int cap = 0, spad = 0, tpad = 0;
  void* pool = nullptr;       // PREFIX_JOINT: [L][2][Bmax][cap][dh]; K plane RoPE-interleaved, V plane transposed
  // DIT: cross block ci's K plane holds [batch][ctx_len][D] packed (the bound length), its V
  // plane [Bmax][D][spad] transposed; both written at bind by one GEMM over all cross blocks
  void* cross_k = nullptr;    // [ceil(L/2)][Bmax * ctx_max * D]
  void* cross_vt = nullptr;   // [ceil(L/2)][Bmax][D][spad]
  void *wkx_all = nullptr, *wvx_all = nullptr;   // DIT: every cross block's W_K (W_V), stacked
  float* state_tok = nullptr; // DIT: [Bmax*st][D]
  float2* rope_cs = nullptr;  // [Bmax][H][dh/2]: cos/sin at each request's chunk positions P_b + i
  std::vector<float2> rope_pos;   // host [max_prefix_len + H][dh/2]: cos/sin of every position
  // per-request visibility: PREFIX_JOINT compact prefix lengths, DIT text / image masks
  int* plens = nullptr;       // [Bmax]
  std::vector<int> plens_host;   // the same, on the host
  uint32_t* kmask = nullptr;  // [2][Bmax][ctx_words]: bit j % 32 of word j / 32 = key j visible
  int ctx_words = 0;
  // whether a request sees less than the whole binding (some P_b < P; a text / image mask
  // with a hidden token): the attention then runs its visibility variant
  bool ragged = false, masked[2] = {false, false};

  // activations
  float *h = nullptr, *x = nullptr;
  void* hs = nullptr;         // T copy of h scaled by (1 + scale) of the next norm site
  float2* stats = nullptr;
  float *zeros = nullptr, *ones = nullptr;   // kVecPad each: stand-ins for absent vectors
  void *qbuf = nullptr, *obuf = nullptr, *abuf = nullptr, *kself = nullptr, *vtself = nullptr;

  // split-K / split-key workspace
  float* ws = nullptr;
  size_t ws_bytes = 0;
  unsigned* counters = nullptr;

  // the loop kernel: XCD-local buffers (one region per XCD), the cross-XCD partial sums and
  // norm operands, flag words and their counter bases, per-step dt
  int loop_mode = FM_LOOP_AUTO;
  char* xl = nullptr;
  size_t xl_bytes = 0;
  long xl_zeroed_stride = -1;   // layout the XCD-local buffers were last zeroed for
  int xl_zeroed_batch = -1;
  char* xag = nullptr;          // norm operands of every (step, site)
  size_t xag_bytes = 0;
  float* xpart = nullptr;       // [2][8][64][hidden] partial sums
  uint32_t* pflags = nullptr;
  float* dts = nullptr;
  uint32_t xb_base = 0, ag_base = 0, pe_base = 0;   // counter values at the next launch's start
  XLoopArgs* loop_dev = nullptr;      // the loop description the kernel reads, and its host copy
  XLoopArgs loop_host;
  bool loop_uploaded = false;
  int wformat = FM_WEIGHTS_AS_GIVEN;   // for the next fm_load_weights
  bool w8 = false;                     // the loaded per-layer weights have FP8 copies
  XLayerW* lw_dev = nullptr;         // [n_layers] weight pointers
  std::vector<XLayerW> lw_host;

  // the step after the path: action statistics of the robot's share of the chunk
  int unnorm_kind = -1, robot_h = 0, robot_d = 0;
  float *q01 = nullptr, *q99 = nullptr;   // [action_dim] each

  // captured loop
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  bool graph_valid = false;

  int rows_per_req() const { return c.state_tokens + c.action_horizon; }
};

namespace {

fm_status fail(fm_ctx* x, fm_status s, const std::string& m) {
  x->err = m;
  if (s == FM_ERR_DEVICE) x->poisoned = true;
  return s;
}

#define HIPCK(call)                                                                       \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(ctx, FM_ERR_DEVICE, fmt("%s failed: %s (%s:%d)", #call, \
                                                              hipGetErrorString(e_), __FILE__, __LINE__)); \
  } while (0)

fm_status dalloc(fm_ctx* ctx, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return FM_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(ctx, FM_ERR_OOM, fmt("hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e)));
  }
  ctx->allocs.push_back(*p);
  return FM_OK;
}

void dfree(fm_ctx* ctx, void* p) {
  if (!p) return;
  for (size_t i = 0; i < ctx->allocs.size(); ++i)
    if (ctx->allocs[i] == p) { ctx->allocs.erase(ctx->allocs.begin() + i); break; }
  (void)hipFree(p);
}

void invalidate_graph(fm_ctx* ctx) {
  if (ctx->gexec) { (void)hipGraphExecDestroy(ctx->gexec); ctx->gexec = nullptr; }
  if (ctx->graph) { (void)hipGraphDestroy(ctx->graph); ctx->graph = nullptr; }
  ctx->graph_valid = false;
}

GemmArgs gemm_base(int M, int N, int K, const void* W) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.M = M; a.N = N; a.K = K; a.W = W;
  a.row_group = 1 << 30; a.row_gstride = 0; a.row_off = 0;
  a.splits = 1; a.k_split = K;
  return a;
}

// Consumer of norm site s at step k: A = hs, per-row (mu, rinv) from the statistics,
// epilogue y = rinv (acc - mu d) + c.
void set_consumer(fm_ctx* ctx, GemmArgs& a, int kind, int k, int s, const float* dvec_override, int rows_h) {
  a.A = ctx->hs; a.lda = ctx->c.hidden;
  a.norm = kind;
  a.stats = ctx->stats; a.nparts = ctx->c.hidden / kStatCols; a.stats_ld = ctx->c.hidden / kStatCols;
  (void)rows_h;
  a.eps = ctx->c.norm_eps;
  if (s >= 0) {
    a.cvec = ctx->cbuf + (size_t)k * ctx->csum + ctx->c_off[s];
    a.dvec = kind == NORM_LN ? ctx->dbuf + (size_t)k * ctx->csum + ctx->c_off[s] : nullptr;
  } else {
    a.cvec = nullptr;
    a.dvec = dvec_override;
  }
}

// Weights consuming norm site s (the output of that norm), and their row count.
std::pair<const void*, int> site_consumer(fm_ctx* ctx, int s) {
  const fm_config& c = ctx->c;
  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    if (s == 2 * c.n_layers) return {ctx->w_out, c.action_dim};
    const auto& W = ctx->L[s / 2];
    if (s % 2 == 0) return {W.qkv, c.n_heads * c.head_dim + 2 * c.head_dim};
    return {W.gu, c.mlp_gated ? 2 * c.mlp_dim : c.mlp_dim};
  }
  if (s == c.n_layers) return {ctx->w_out, c.action_dim};
  const auto& W = ctx->L[s];
  return s % 2 == 0 ? std::pair<const void*, int>{W.q, c.hidden} : std::pair<const void*, int>{W.qkv, 3 * c.hidden};
}

// The launch sequence of Euler step k. vout: velocity output (then x is not updated);
// trace: residual stream copies after the in-projection and after every layer.
std::vector<Op> build_step(fm_ctx* ctx, int k, float* vout, float* trace) {
  const fm_config& c = ctx->c;
  const int B = ctx->bound_batch, H = c.action_horizon, D = c.hidden, F = c.mlp_dim;
  const int st = c.state_tokens, Mh = B * (st + H), Ma = B * H;
  const int S = n_sites(c);
  const float* row = ctx->table + (size_t)k * S * 3 * D;
  auto site = [&](int s, int part) { return row + (size_t)s * 3 * D + (size_t)part * D; };
  std::vector<Op> ops;
  Op op;
  memset(&op, 0, sizeof op);

  // action (and state) tokens -> h
  op.kind = Op::INPROJ;
  InProjArgs& ip = op.ip;
  ip.x = ctx->x; ip.da = c.action_dim; ip.w = ctx->w_in; ip.b = ctx->b_in;
  ip.tb = c.arch == FM_ARCH_DIT_CROSS ? ctx->tbias + (size_t)k * D : nullptr;
  ip.state_tok = ctx->state_tok; ip.B = B; ip.Ha = H; ip.st = st; ip.D = D;
  ip.h = ctx->h; ip.stats = ctx->stats; ip.stats_ld = D / kStatCols; ip.zeros = ctx->zeros;
  ip.hs = ctx->hs; ip.hscale = site(0, 0);
  op.role = FM_OP_INPROJ;
  ops.push_back(op);
  if (trace) { Op t; memset(&t, 0, sizeof t); t.kind = Op::TRACE; t.trace_layer = 0; ops.push_back(t); }

  for (int l = 0; l < c.n_layers; ++l) {
    const auto& W = ctx->L[l];
    if (c.arch == FM_ARCH_PREFIX_JOINT) {
      const int nq = c.n_heads, dh = c.head_dim, qd = nq * dh;
      const size_t plane = (size_t)c.max_batch * ctx->cap * dh * ctx->esz;
      char* kpl = (char*)ctx->pool + (size_t)(2 * l) * plane;
      char* vpl = (char*)ctx->pool + (size_t)(2 * l + 1) * plane;
      // QKV + RoPE + append into pool slots [P, P+H)
      GemmArgs g = gemm_base(Ma, qd + 2 * dh, D, W.qkv);
      g.w8 = W.qkv8; g.wscale = W.sqkv;
      set_consumer(ctx, g, NORM_RMS, k, 2 * l, nullptr, Mh);
      g.epi = EPI_QKV; g.out = ctx->qbuf; g.ldo = qd;
      g.q_cols = qd; g.kv_cols = dh; g.tq = H; g.kv_off = ctx->prefix_len;
      g.rope = c.rope_base > 0.f; g.half_dh = dh / 2; g.rope_cs = ctx->rope_cs;
      g.kdst = kpl; g.k_bs = (long)ctx->cap * dh; g.k_rs = dh;
      g.vdst = vpl; g.v_bs = (long)dh * ctx->cap; g.v_ds = ctx->cap;
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_QKV; op.g = g; ops.push_back(op);
      // attention over [prefix ; suffix]
      AttnArgs at;
      memset(&at, 0, sizeof at);
      at.q = ctx->qbuf; at.q_bs = (long)H * qd; at.q_rs = qd;
      at.k = kpl; at.k_bs = (long)ctx->cap * dh; at.k_rs = dh; at.k_hs = 0;
      at.vt = vpl; at.v_bs = (long)dh * ctx->cap; at.v_hs = 0; at.v_ds = ctx->cap;
      at.k_len = at.v_len = (long)c.max_batch * ctx->cap * dh;
      at.o = ctx->obuf; at.o_bs = (long)H * qd; at.o_rs = qd;
      at.B = B; at.Tq = H; at.n_heads = nq; at.heads_per_kv = nq; at.n_keys = ctx->prefix_len + H; at.dh = dh;
      if (ctx->ragged) { at.seg_len = ctx->plens; at.seg_end = ctx->prefix_len; }   // request b: its first P_b prefix keys, then its chunk
      at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
      memset(&op, 0, sizeof op); op.kind = Op::ATTN; op.role = FM_OP_ATTN; op.at = at; ops.push_back(op);
      // O projection + gated residual
      g = gemm_base(Ma, D, qd, W.o);
      g.w8 = W.o8; g.wscale = W.so;
      g.A = ctx->obuf; g.lda = qd;
      g.epi = EPI_RESID; g.h = ctx->h; g.ldh_out = D; g.gate = site(2 * l, 2); g.stats_out = ctx->stats; g.stats_out_ld = D / kStatCols;
      g.hs = ctx->hs; g.hscale = site(2 * l + 1, 0);
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_OPROJ; op.g = g; ops.push_back(op);
      // gate/up + GELU * up
      g = gemm_base(Ma, c.mlp_gated ? 2 * F : F, D, W.gu);
      g.w8 = W.gu8; g.wscale = W.sgu;
      set_consumer(ctx, g, NORM_RMS, k, 2 * l + 1, nullptr, Mh);
      g.out = ctx->abuf; g.ldo = F;
      if (c.mlp_gated) g.epi = EPI_GELU_MUL; else { g.epi = EPI_STORE; g.act = ACT_GELU; }
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_MLP_UP; op.g = g; ops.push_back(op);
      // down + gated residual
      g = gemm_base(Ma, D, F, W.down);
      g.w8 = W.down8; g.wscale = W.sdown;
      g.A = ctx->abuf; g.lda = F;
      g.epi = EPI_RESID; g.h = ctx->h; g.ldh_out = D; g.gate = site(2 * l + 1, 2); g.stats_out = ctx->stats; g.stats_out_ld = D / kStatCols;
      g.hs = ctx->hs; g.hscale = site(2 * l + 2, 0);
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_MLP_DOWN; op.g = g; ops.push_back(op);
    } else {
      const int nh = c.n_heads, dh = c.head_dim, Tq = st + H;
      const bool cross = (l % 2) == 0;
      AttnArgs at;
      memset(&at, 0, sizeof at);
      at.q = ctx->qbuf; at.q_bs = (long)Tq * D; at.q_rs = D;
      at.o = ctx->obuf; at.o_bs = (long)Tq * D; at.o_rs = D;
      at.B = B; at.Tq = Tq; at.n_heads = nh; at.heads_per_kv = 1; at.dh = dh;
      at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
      GemmArgs g;
      if (cross) {
        const int ci = l / 2;
        g = gemm_base(Mh, D, D, W.q);
        g.w8 = W.q8; g.wscale = W.sq;
        set_consumer(ctx, g, NORM_LN, k, l, nullptr, Mh);
        g.epi = EPI_STORE; g.out = ctx->qbuf; g.ldo = D;
        memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_QKV; op.g = g; ops.push_back(op);
        at.k = (char*)ctx->cross_k + (size_t)ci * c.max_batch * c.ctx_len_max * D * ctx->esz;
        at.k_bs = (long)ctx->prefix_len * D; at.k_rs = D; at.k_hs = dh;   // packed at the bound length
        at.vt = (char*)ctx->cross_vt + (size_t)ci * c.max_batch * D * ctx->spad * ctx->esz;
        at.v_bs = (long)D * ctx->spad; at.v_hs = (long)dh * ctx->spad; at.v_ds = ctx->spad;
        at.k_len = (long)c.max_batch * c.ctx_len_max * D; at.v_len = (long)c.max_batch * D * ctx->spad;
        at.n_keys = ctx->prefix_len;
        // the text mask on cross blocks whose index is a multiple of 4, the image mask on the others
        const int mi = l % 4 == 0 ? 0 : 1;
        if (ctx->masked[mi]) { at.kmask = ctx->kmask + (size_t)mi * c.max_batch * ctx->ctx_words; at.km_bs = ctx->ctx_words; }
      } else {
        g = gemm_base(Mh, 3 * D, D, W.qkv);
        g.w8 = W.qkv8; g.wscale = W.sqkv;
        set_consumer(ctx, g, NORM_LN, k, l, nullptr, Mh);
        g.epi = EPI_QKV; g.out = ctx->qbuf; g.ldo = D;
        g.q_cols = D; g.kv_cols = D; g.tq = Tq; g.kv_off = 0; g.rope = 0;
        g.kdst = ctx->kself; g.k_bs = (long)Tq * D; g.k_rs = D;
        g.vdst = ctx->vtself; g.v_bs = (long)D * ctx->tpad; g.v_ds = ctx->tpad;
        memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_QKV; op.g = g; ops.push_back(op);
        at.k = ctx->kself; at.k_bs = (long)Tq * D; at.k_rs = D; at.k_hs = dh;
        at.vt = ctx->vtself; at.v_bs = (long)D * ctx->tpad; at.v_hs = (long)dh * ctx->tpad; at.v_ds = ctx->tpad;
        at.k_len = (long)c.max_batch * Tq * D; at.v_len = (long)c.max_batch * D * ctx->tpad;
        at.n_keys = Tq;
      }
      memset(&op, 0, sizeof op); op.kind = Op::ATTN; op.role = FM_OP_ATTN; op.at = at; ops.push_back(op);
      g = gemm_base(Mh, D, D, W.o);
      g.w8 = W.o8; g.wscale = W.so;
      g.A = ctx->obuf; g.lda = D;
      g.epi = EPI_RESID; g.h = ctx->h; g.ldh_out = D; g.gate = site(l, 2); g.stats_out = ctx->stats; g.stats_out_ld = D / kStatCols;
      g.hs = ctx->hs; g.hscale = nullptr;  // the feed-forward LayerNorm carries no modulation
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_OPROJ; op.g = g; ops.push_back(op);
      g = gemm_base(Mh, F, D, W.gu);
      g.w8 = W.gu8; g.wscale = W.sgu;
      set_consumer(ctx, g, NORM_LN, k, -1, ctx->dff + (size_t)l * F, Mh);
      g.epi = EPI_STORE; g.act = ACT_GELU; g.out = ctx->abuf; g.ldo = F;
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_MLP_UP; op.g = g; ops.push_back(op);
      g = gemm_base(Mh, D, F, W.down);
      g.w8 = W.down8; g.wscale = W.sdown;
      g.A = ctx->abuf; g.lda = F;
      g.epi = EPI_RESID; g.h = ctx->h; g.ldh_out = D; g.gate = nullptr; g.stats_out = ctx->stats; g.stats_out_ld = D / kStatCols;
      g.hs = ctx->hs; g.hscale = site(l + 1, 0);
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_MLP_DOWN; op.g = g; ops.push_back(op);
    }
    if (trace) { Op t; memset(&t, 0, sizeof t); t.kind = Op::TRACE; t.trace_layer = l + 1; ops.push_back(t); }
  }
  // final modulated norm + velocity projection + Euler update
  GemmArgs g = gemm_base(Ma, c.action_dim, D, ctx->w_out);
  set_consumer(ctx, g, c.arch == FM_ARCH_PREFIX_JOINT ? NORM_RMS : NORM_LN, k, S - 1, nullptr, Mh);
  if (st > 0) { g.row_group = H; g.row_gstride = st + H; g.row_off = st; }
  g.epi = EPI_EULER; g.bias = ctx->b_out; g.ldo = c.action_dim;
  if (vout) { g.vout = vout; g.x = nullptr; g.dt = 0.f; }
  else { g.x = ctx->x; g.dt = ctx->tau[k + 1] - ctx->tau[k]; g.vout = nullptr; }
  memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.role = FM_OP_OUT; op.g = g; ops.push_back(op);
  return ops;
}

// Plan tile shapes / splits and make sure the shared workspace covers every op.
fm_status plan_ops(fm_ctx* ctx, std::vector<Op>& ops) {
  size_t need = 0;
  for (auto& op : ops) {
    if (op.kind == Op::GEMM) {
      gemm_plan(op.g, ctx->elem, ctx->num_cus);
      need = std::max(need, gemm_ws_bytes(op.g));
      if (op.g.splits > 1 && gemm_num_tiles(op.g) > kGemmCounters) return fail(ctx, FM_ERR_UNSUPPORTED, "too many split tiles");
    } else if (op.kind == Op::ATTN) {
      attn_plan(op.at, ctx->elem, ctx->num_cus);
      need = std::max(need, attn_ws_bytes(op.at));
    }
  }
  if (need > ctx->ws_bytes) {
    HIPCK(hipStreamSynchronize(ctx->stream));
    dfree(ctx, ctx->ws);
    ctx->ws = nullptr;
    ctx->ws_bytes = 0;
    void* p;
    fm_status s = dalloc(ctx, &p, need);
    if (s != FM_OK) return s;
    ctx->ws = (float*)p;
    ctx->ws_bytes = need;
  }
  for (auto& op : ops) {
    if (op.kind == Op::GEMM) { op.g.ws = ctx->ws; op.g.counters = ctx->counters; op.g.zeros = ctx->zeros; op.g.ones = ctx->ones; }
    else if (op.kind == Op::ATTN) op.at.ws = ctx->ws;
  }
  return FM_OK;
}

fm_status enqueue_ops(fm_ctx* ctx, const std::vector<Op>& ops, hipStream_t s, float* trace) {
  const size_t hsz = (size_t)ctx->bound_batch * ctx->rows_per_req() * ctx->c.hidden;
  for (const auto& op : ops) {
    switch (op.kind) {
      case Op::GEMM: HIPCK(gemm_launch(op.g, ctx->elem, s)); break;
      case Op::ATTN: HIPCK(attn_launch(op.at, ctx->elem, s)); break;
      case Op::INPROJ: HIPCK(inproj_launch(op.ip, ctx->elem, s)); break;
      case Op::TRACE:
        HIPCK(hipMemcpyAsync(trace + (size_t)op.trace_layer * hsz, ctx->h, hsz * sizeof(float), hipMemcpyDeviceToDevice, s));
        break;
    }
  }
  return FM_OK;
}

fm_status check_ready(fm_ctx* ctx) {
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!ctx->loaded) return fail(ctx, FM_ERR_STATE, "weights are not loaded");
  if (ctx->steps < 0) return fail(ctx, FM_ERR_STATE, "no schedule: call fm_set_schedule first");
  if (ctx->prefix_len < 0) return fail(ctx, FM_ERR_STATE, "nothing bound: call fm_bind_prefix_kv first");
  if (ctx->sched_batch != ctx->bound_batch)
    return fail(ctx, FM_ERR_SCHEDULE, fmt("scheduled batch %d differs from bound batch %d", ctx->sched_batch, ctx->bound_batch));
  return FM_OK;
}

// ---------------------------------------------------------------------------------------
// The loop kernel (fm_xloop.hip)
// ---------------------------------------------------------------------------------------
XShape loop_shape(const fm_ctx* ctx) {
  const fm_config& c = ctx->c;
  XShape sh;
  sh.bf16 = c.dtype == FM_BF16;
  sh.B = ctx->bound_batch; sh.H = c.action_horizon; sh.D = c.hidden; sh.nq = c.n_heads; sh.dh = c.head_dim;
  sh.F = c.mlp_dim; sh.da = c.action_dim; sh.L = c.n_layers;
  sh.npairs = 0;
  for (int b = 0; b < ctx->bound_batch && b < (int)ctx->plens_host.size(); ++b)
    sh.npairs += ((ctx->plens_host[b] + 31) / 32 + (c.action_horizon + 31) / 32 + 1) / 2;
  return sh;
}

// nullptr when the loop kernel serves the current weights / schedule / binding, else why not
const char* loop_unsupported(const fm_ctx* ctx) {
  const fm_config& c = ctx->c;
  if (ctx->loop_mode != FM_LOOP_AUTO) return "loop mode is FM_LOOP_GRAPH";
  if (c.arch != FM_ARCH_PREFIX_JOINT || !c.mlp_gated || c.n_kv_heads != 1) return "not a pi0.5-family expert";
  if (!ctx->pflags) return "no loop-kernel workspace (bf16, head_dim 256 only)";
  if (ctx->steps < 1 || ctx->prefix_len < 0) return "no schedule or binding";
  return xloop_check(loop_shape(ctx), ctx->num_cus);
}

// the buffers for `steps` steps of the current binding; the XCD-local ones are zeroed whenever
// their layout changes: key slots past the horizon in the chunk's last key tile are never
// written, and their zero softmax weight must not meet a stale NaN or Inf left by another layout
fm_status loop_buffers(fm_ctx* ctx, int steps) {
  const fm_config& c = ctx->c;
  const XShape sh = loop_shape(ctx);
  const XLayout r = xloop_layout(sh.B, sh.H, sh.D, sh.F, sh.da, sh.npairs);
  const size_t need_xl = 8 * (size_t)r.xl_stride;
  const size_t need_ag = (size_t)steps * (2 * c.n_layers + 1) * r.ag_site;
  if (need_xl > ctx->xl_bytes || need_ag > ctx->xag_bytes) HIPCK(hipStreamSynchronize(ctx->stream));
  if (need_xl > ctx->xl_bytes) {
    dfree(ctx, ctx->xl);
    ctx->xl = nullptr;
    ctx->xl_bytes = 0;
    void* p;
    fm_status s = dalloc(ctx, &p, need_xl);
    if (s != FM_OK) return s;
    ctx->xl = (char*)p;
    ctx->xl_bytes = need_xl;
    ctx->xl_zeroed_stride = -1;
  }
  if (need_ag > ctx->xag_bytes) {
    dfree(ctx, ctx->xag);
    ctx->xag = nullptr;
    ctx->xag_bytes = 0;
    void* p;
    fm_status s = dalloc(ctx, &p, need_ag);
    if (s != FM_OK) return s;
    ctx->xag = (char*)p;
    ctx->xag_bytes = need_ag;
  }
  if (ctx->xl_zeroed_stride != r.xl_stride || ctx->xl_zeroed_batch != ctx->bound_batch) {
    HIPCK(hipMemsetAsync(ctx->xl, 0, ctx->xl_bytes, ctx->stream));
    ctx->xl_zeroed_stride = r.xl_stride;
    ctx->xl_zeroed_batch = ctx->bound_batch;
  }
  return FM_OK;
}

// one launch of the loop kernel: steps k0 .. k0 + nsteps - 1 on ctx->x (or, with vout, the
// velocity of step k0 without the update)
fm_status loop_run(fm_ctx* ctx, int k0, int nsteps, float* vout) {
  const fm_config& c = ctx->c;
  fm_status s = loop_buffers(ctx, ctx->steps);
  if (s != FM_OK) return s;
  const XShape sh = loop_shape(ctx);
  const XLayout r = xloop_layout(sh.B, sh.H, sh.D, sh.F, sh.da, sh.npairs);
  XLoopArgs a;
  memset(&a, 0, sizeof a);
  a.B = ctx->bound_batch; a.H = c.action_horizon; a.M = a.B * a.H; a.D = c.hidden; a.nq = c.n_heads;
  a.F = c.mlp_dim; a.da = c.action_dim; a.L = c.n_layers; a.P = ctx->prefix_len; a.cap = ctx->cap;
  a.Hp = r.Hp; a.S = n_sites(c); a.csum = ctx->csum;
  const int nqkv = c.n_heads * c.head_dim + 2 * c.head_dim;
  a.cq4 = (int)round_up(nqkv, 4); a.cg4 = (int)round_up(2 * a.F, 4); a.cout4 = (int)round_up(a.da, 4);
  a.eps = c.norm_eps; a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  a.rope = c.rope_base > 0.f;
  a.max_steps = std::max(c.max_steps, 1); a.dts = ctx->dts;
  // attention key-tile pairs of one head: request b's prefix tiles, then its chunk's tiles, two
  // by two
  a.npairs = 0;
  for (int b = 0; b < a.B; ++b) {
    a.poff[b] = a.npairs;
    a.plen[b] = ctx->plens_host[b];
    const int nt = (a.plen[b] + 31) / 32 + (a.H + 31) / 32;
    for (int j = 0; j < nt; j += 2) a.pair[a.npairs++] = XPair{b, j};
  }
  a.poff[a.B] = a.npairs;
  a.w_in = ctx->w_in; a.b_in = ctx->b_in; a.w_out = ctx->w_out; a.b_out = ctx->b_out;
  std::vector<XLayerW> lw(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const auto& W = ctx->L[l];
    lw[l] = ctx->w8 ? XLayerW{W.qkv8, W.o8, W.gu8, W.down8, W.sqkv, W.so, W.sgu, W.sdown}
                    : XLayerW{W.qkv, W.o, W.gu, W.down, nullptr, nullptr, nullptr, nullptr};
  }
  a.lw = ctx->lw_dev;
  auto wbytes = [&](int N, int K) { return (uint32_t)(ctx->w8 ? swizzled_fp8_bytes(N, K) : swizzled_bytes(N, K, ET_BF16)); };
  a.wb_qkv = wbytes(nqkv, a.D);
  a.wb_o = wbytes(a.D, c.n_heads * c.head_dim);
  a.wb_gu = wbytes(2 * a.F, a.D);
  a.wb_down = wbytes(a.D, a.F);
  a.wb_out = (uint32_t)swizzled_bytes(a.da, a.D, ET_BF16);
  a.table = ctx->table; a.cbuf = ctx->cbuf; a.rope_cs = ctx->rope_cs;
  a.pool = (const __bf16*)ctx->pool; a.plane = (long)c.max_batch * ctx->cap * c.head_dim;
  a.xl = ctx->xl; a.xl_stride = r.xl_stride;
  a.o_xx = r.o_xx; a.o_q = r.o_q; a.o_sk = r.o_sk; a.o_svt = r.o_svt; a.o_ap = r.o_ap; a.o_ml = r.o_ml;
  a.o_ax = r.o_ax; a.o_act = r.o_act;
  a.part = ctx->xpart;
  a.ag = ctx->xag; a.ag_site = r.ag_site; a.ag_step = (long)(2 * c.n_layers + 1) * r.ag_site; a.o_agst = r.o_agst;
  a.flags = ctx->pflags;
  // the description lives in device memory; it is uploaded again only when it changed
  if (!ctx->loop_uploaded || memcmp(&a, &ctx->loop_host, sizeof a) != 0 || lw.size() != ctx->lw_host.size() ||
      memcmp(lw.data(), ctx->lw_host.data(), lw.size() * sizeof(XLayerW)) != 0) {
    HIPCK(hipStreamSynchronize(ctx->stream));
    ctx->loop_host = a;
    ctx->lw_host = lw;
    HIPCK(hipMemcpy(ctx->loop_dev, &ctx->loop_host, sizeof a, hipMemcpyHostToDevice));
    HIPCK(hipMemcpy(ctx->lw_dev, ctx->lw_host.data(), lw.size() * sizeof(XLayerW), hipMemcpyHostToDevice));
    ctx->loop_uploaded = true;
  }
  uint32_t nxb, nag, npe;
  xloop_counts(c.n_layers, nsteps, &nxb, &nag, &npe);
  if (ctx->xb_base > 0x70000000u - 32u * nxb || ctx->ag_base > 0x70000000u - 32u * nag || ctx->pe_base > 0x70000000u - npe) {
    // counters only grow within a flag generation: start a new one
    HIPCK(hipMemsetAsync(ctx->pflags, 0, kXFlagWords * sizeof(uint32_t), ctx->stream));
    ctx->xb_base = ctx->ag_base = ctx->pe_base = 0;
  }
  XLaunch la;
  la.k0 = k0; la.nsteps = nsteps;
  la.xb0 = ctx->xb_base; la.ag0 = ctx->ag_base; la.pe0 = ctx->pe_base;
  la.xin = ctx->x; la.xout = ctx->x; la.vout = vout;
  ctx->xb_base += 32u * nxb;
  ctx->ag_base += 32u * nag;
  ctx->pe_base += npe;
  HIPCK(xloop_launch(ctx->loop_dev, la, ctx->w8, ctx->stream));
  return FM_OK;
}

}  // namespace

// =======================================================================================
// C ABI
// =======================================================================================
extern "C" {

fm_status fm_device_supported(const char* gcn_arch, int32_t num_xcc, int32_t num_cus, char* msg, int32_t msg_len) {
  std::string m;
  fm_status s = FM_OK;
  if (!gcn_arch) { m = "gcn_arch is NULL"; s = FM_ERR_INVALID_ARG; }
  else if (strncmp(gcn_arch, "gfx950", 6) != 0) { m = fmt("device is %s; this library is built for gfx950", gcn_arch); s = FM_ERR_UNSUPPORTED; }
  else if (num_xcc != 8) {
    m = fmt("the device reports %d XCDs; the split-K and loop-kernel exchanges assume the 8 XCDs of a whole MI355X "
            "partition (workgroup b on XCD b mod 8)", num_xcc);
    s = FM_ERR_UNSUPPORTED;
  } else if (num_cus < 8 || num_cus % 8 != 0) {
    m = fmt("the device reports %d CUs, not a multiple of its 8 XCDs", num_cus);
    s = FM_ERR_UNSUPPORTED;
  }
  if (msg && msg_len > 0) { strncpy(msg, m.c_str(), msg_len - 1); msg[msg_len - 1] = 0; }
  if (s != FM_OK) g_err = m;
  return s;
}

fm_status fm_query(const fm_config* cfg, fm_plan_info* info, char* msg, int32_t msg_len) {
  std::string m;
  fm_status s = check_config(cfg, m);
  if (msg && msg_len > 0) { strncpy(msg, m.c_str(), msg_len - 1); msg[msg_len - 1] = 0; }
  if (s != FM_OK) { g_err = m; return s; }
  if (info) {
    const fm_config& c = *cfg;
    const int esz = c.dtype == FM_BF16 ? 2 : 4;
    memset(info, 0, sizeof *info);
    info->n_sites = n_sites(c);
    info->pool_capacity = c.arch == FM_ARCH_PREFIX_JOINT ? pool_capacity(c) : 0;
    auto specs = weight_specs(c);
    info->n_weights = (int32_t)specs.size();
    int64_t wb = 0;
    for (auto& sp : specs) {
      int64_t n = 1;
      for (auto d : sp.shape) n *= d;
      wb += n * esz;
    }
    info->weight_bytes = wb;
    if (c.arch == FM_ARCH_PREFIX_JOINT)
      info->pool_bytes = (int64_t)c.n_layers * 2 * c.max_batch * pool_capacity(c) * c.head_dim * esz;
    else
      info->pool_bytes = (int64_t)((c.n_layers + 1) / 2) * c.max_batch * c.hidden * (c.ctx_len_max + round_up(c.ctx_len_max, 8)) * esz;
  }
  return FM_OK;
}

fm_status fm_weight_spec(const fm_config* cfg, int32_t i, const char** name, int32_t* ndim, int64_t shape[4]) {
  std::string m;
  fm_status s = check_config(cfg, m);
  if (s != FM_OK) { g_err = m; return s; }
  static thread_local std::vector<Spec> cache;
  cache = weight_specs(*cfg);
  if (i < 0 || i >= (int32_t)cache.size()) { g_err = fmt("weight index %d out of range [0, %zu)", i, cache.size()); return FM_ERR_INVALID_ARG; }
  if (name) *name = cache[i].name.c_str();
  if (ndim) *ndim = (int32_t)cache[i].shape.size();
  if (shape) for (size_t d = 0; d < 4; ++d) shape[d] = d < cache[i].shape.size() ? cache[i].shape[d] : 0;
  return FM_OK;
}

const char* fm_last_error(const fm_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

fm_status fm_create(const fm_config* cfg, void* stream, fm_ctx** out) {
  std::string m;
  if (!out) { g_err = "out is NULL"; return FM_ERR_INVALID_ARG; }
  *out = nullptr;
  fm_status s = check_config(cfg, m);
  if (s != FM_OK) { g_err = m; return s; }
  fm_ctx* ctx = new fm_ctx();
  ctx->c = *cfg;
  ctx->stream = (hipStream_t)stream;
  ctx->elem = cfg->dtype == FM_BF16 ? ET_BF16 : ET_F32;
  ctx->esz = cfg->dtype == FM_BF16 ? 2 : 4;
  auto bail = [&](fm_status st) { g_err = ctx->err; fm_destroy(ctx); return st; };
  hipError_t e = hipGetDevice(&ctx->device);
  if (e != hipSuccess) { ctx->err = fmt("hipGetDevice: %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, ctx->device);
  if (e != hipSuccess) { ctx->err = fmt("hipGetDeviceProperties: %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }
  int n_xcc = 0;
  e = hipDeviceGetAttribute(&n_xcc, hipDeviceAttributeNumberOfXccs, ctx->device);
  if (e != hipSuccess) { ctx->err = fmt("hipDeviceGetAttribute(NumberOfXccs): %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }
  {
    char msg[256];
    fm_status ds = fm_device_supported(prop.gcnArchName, n_xcc, prop.multiProcessorCount, msg, (int32_t)sizeof msg);
    if (ds != FM_OK) { ctx->err = msg; return bail(ds); }
  }
  ctx->num_cus = prop.multiProcessorCount;
  {
    // The XCD-local exchanges need each residue of blockIdx mod 8 on one XCD: check that the
    // dispatcher deals a launch round-robin over the XCDs (from whichever XCD it starts on).
    const int n = 2048;
    uint32_t* d = nullptr;
    std::vector<uint32_t> h(n);
    e = hipMalloc(&d, n * sizeof(uint32_t));
    if (e == hipSuccess) e = xcc_probe(d, n, ctx->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h.data(), d, n * sizeof(uint32_t), hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    if (d) (void)hipFree(d);
    if (e != hipSuccess) { ctx->err = fmt("workgroup placement probe: %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }
    for (int b = 0; b < n; ++b)
      if (h[b] >= 8u || ((h[b] - (uint32_t)b) & 7u) != (h[0] & 7u)) {
        ctx->err = fmt("workgroup %d of a %d-workgroup launch ran on XCD %u: the dispatch is not round-robin over the 8 XCDs, "
                       "which the split-K and loop-kernel exchanges need", b, n, h[b]);
        return bail(FM_ERR_UNSUPPORTED);
      }
  }
  e = hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) { ctx->err = fmt("hipStreamCreate: %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }

  const fm_config& c = *cfg;
  const size_t B = c.max_batch, D = c.hidden, F = c.mlp_dim, H = c.action_horizon, st = c.state_tokens;
  const size_t rows = B * (st + H);
  const size_t esz = ctx->esz;
  const size_t qd = (size_t)c.n_heads * c.head_dim;
  void* p;
#define ALLOC(field, bytes, type)                               \
  do {                                                          \
    if ((s = dalloc(ctx, &p, (bytes))) != FM_OK) return bail(s); \
    ctx->field = (type)p;                                       \
  } while (0)
  ALLOC(h, rows * D * 4, float*);
  ALLOC(hs, rows * D * esz, void*);
  ALLOC(x, B * H * c.action_dim * 4 + 64, float*);  // padded: the Euler epilogue reads 4 floats at a time
  // [row][slot]; the tail pads the consumers' fixed-width slot reads past the last row
  ALLOC(stats, ((D / kStatCols) * rows + 2 * kMaxStatSlots) * sizeof(float2), float2*);
  ALLOC(zeros, kVecPad * sizeof(float), float*);
  ALLOC(ones, kVecPad * sizeof(float), float*);
  ALLOC(qbuf, rows * std::max(qd, D) * esz, void*);
  ALLOC(obuf, rows * std::max(qd, D) * esz, void*);
  ALLOC(abuf, rows * F * esz, void*);
  ALLOC(table, (size_t)c.max_steps * n_sites(c) * 3 * D * 4, float*);
  ALLOC(e_buf, (size_t)c.max_steps * D * esz, void*);
  ALLOC(c1_buf, (size_t)c.max_steps * D * esz, void*);
  ALLOC(c_buf, (size_t)c.max_steps * D * esz, void*);
  ALLOC(row_buf, (size_t)std::max(c.max_steps, 1) * D * esz, void*);
  {
    // consumer row counts per norm site, in site order
    const int S = n_sites(c);
    ctx->c_off.assign(S, 0);
    long off = 0;
    for (int s2 = 0; s2 < S; ++s2) {
      int n;
      if (c.arch == FM_ARCH_PREFIX_JOINT)
        n = s2 == 2 * c.n_layers ? c.action_dim : (s2 % 2 == 0 ? c.n_heads * c.head_dim + 2 * c.head_dim : (c.mlp_gated ? 2 : 1) * c.mlp_dim);
      else
        n = s2 == c.n_layers ? c.action_dim : (s2 % 2 == 0 ? c.hidden : 3 * c.hidden);
      ctx->c_off[s2] = off;
      off += round_up(n, 4);
    }
    ctx->csum = off;
  }
  ALLOC(cbuf, (size_t)c.max_steps * ctx->csum * 4, float*);
  if (c.arch == FM_ARCH_DIT_CROSS) {
    ALLOC(dbuf, (size_t)c.max_steps * ctx->csum * 4, float*);
    ALLOC(dff, (size_t)c.n_layers * F * 4, float*);
  }
  ALLOC(counters, kGemmCounters * sizeof(unsigned), unsigned*);
  if (c.arch == FM_ARCH_PREFIX_JOINT && c.dtype == FM_BF16 && c.head_dim == 256 && c.n_layers <= kXMaxLayers) {
    ALLOC(pflags, kXFlagWords * sizeof(uint32_t), uint32_t*);
    ALLOC(xpart, 2 * 8 * 64 * D * sizeof(float), float*);
    ALLOC(dts, (size_t)std::max(c.max_steps, 1) * sizeof(float), float*);
    ALLOC(loop_dev, sizeof(XLoopArgs), XLoopArgs*);
    ALLOC(lw_dev, (size_t)c.n_layers * sizeof(XLayerW), XLayerW*);
  }
  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    ctx->cap = pool_capacity(c);
    ALLOC(pool, (size_t)c.n_layers * 2 * B * ctx->cap * c.head_dim * esz, void*);
    ALLOC(rope_cs, B * H * (c.head_dim / 2) * sizeof(float2), float2*);
    ALLOC(plens, B * sizeof(int), int*);
  } else {
    const size_t nc = (c.n_layers + 1) / 2;
    // transposed V planes hold whole key tiles (and the permuted slots of each)
    ctx->spad = (int)round_up(c.ctx_len_max, 64);
    ctx->tpad = (int)round_up(st + H, 64);
    ALLOC(cross_k, nc * B * c.ctx_len_max * D * esz, void*);
    ALLOC(cross_vt, nc * B * D * ctx->spad * esz, void*);
    ALLOC(kself, rows * D * esz, void*);
    ALLOC(vtself, B * D * ctx->tpad * esz, void*);
    ALLOC(tbias, (size_t)c.max_steps * D * 4, float*);
    if (st > 0) ALLOC(state_tok, B * st * D * 4, float*);
    ctx->ctx_words = (int)((c.ctx_len_max + 31) / 32);
    ALLOC(kmask, 2 * B * ctx->ctx_words * sizeof(uint32_t), uint32_t*);
  }
#undef ALLOC
  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    // cos/sin of positions 0 .. max_prefix_len + H - 1 (rotate_half pairs j, j + dh/2), in
    // double; a request's chunk rows take positions P_b .. P_b + H - 1 of it
    const int dh = c.head_dim, np = c.max_prefix_len + H;
    ctx->rope_pos.resize((size_t)np * (dh / 2));
    for (int j = 0; j < dh / 2; ++j) {
      const double th = c.rope_base > 0.f ? std::pow((double)c.rope_base, -2.0 * j / dh) : 0.0;
      for (int p = 0; p < np; ++p)
        ctx->rope_pos[(size_t)p * (dh / 2) + j] = make_float2((float)std::cos(p * th), (float)std::sin(p * th));
    }
  }
  e = hipMemsetAsync(ctx->counters, 0, kGemmCounters * sizeof(unsigned), ctx->stream);
  if (e == hipSuccess) e = hipMemsetAsync(ctx->zeros, 0, kVecPad * sizeof(float), ctx->stream);
  if (e == hipSuccess) e = fill_f32(ctx->ones, 1.f, kVecPad, ctx->stream);
  if (e == hipSuccess) e = hipMemsetAsync(ctx->stats, 0, ((D / kStatCols) * rows + 2 * kMaxStatSlots) * sizeof(float2), ctx->stream);
  if (e == hipSuccess && ctx->pflags) e = hipMemsetAsync(ctx->pflags, 0, kXFlagWords * sizeof(uint32_t), ctx->stream);
  if (e == hipSuccess && ctx->pool) e = hipMemsetAsync(ctx->pool, 0, (size_t)c.n_layers * 2 * B * ctx->cap * c.head_dim * esz, ctx->stream);
  if (e == hipSuccess && ctx->vtself) e = hipMemsetAsync(ctx->vtself, 0, B * D * ctx->tpad * esz, ctx->stream);
  if (e == hipSuccess && ctx->cross_vt) e = hipMemsetAsync(ctx->cross_vt, 0, ((c.n_layers + 1) / 2) * B * D * ctx->spad * esz, ctx->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) { ctx->err = fmt("initial clear: %s", hipGetErrorString(e)); return bail(FM_ERR_DEVICE); }
  ctx->L.resize(c.n_layers);
  *out = ctx;
  return FM_OK;
}

fm_status fm_destroy(fm_ctx* ctx) {
  if (!ctx) return FM_OK;
  (void)hipStreamSynchronize(ctx->stream);
  invalidate_graph(ctx);
  for (void* p : ctx->allocs) (void)hipFree(p);
  ctx->allocs.clear();
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  delete ctx;
  return FM_OK;
}

fm_status fm_load_weights(fm_ctx* ctx, const fm_tensor* t, int32_t n) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!t || n < 0) return fail(ctx, FM_ERR_INVALID_ARG, "tensor table is NULL");
  const fm_config& c = ctx->c;
  auto specs = weight_specs(c);
  std::map<std::string, const fm_tensor*> byname;
  for (int i = 0; i < n; ++i) {
    if (!t[i].name) return fail(ctx, FM_ERR_INVALID_ARG, fmt("tensor %d has no name", i));
    if (byname.count(t[i].name)) return fail(ctx, FM_ERR_SHAPE, fmt("tensor '%s' given twice", t[i].name));
    byname[t[i].name] = &t[i];
  }
  for (auto& sp : specs) {
    auto it = byname.find(sp.name);
    if (it == byname.end()) return fail(ctx, FM_ERR_SHAPE, fmt("missing weight '%s'", sp.name.c_str()));
    const fm_tensor* w = it->second;
    if (w->dtype != c.dtype) return fail(ctx, FM_ERR_SHAPE, fmt("weight '%s': dtype %d, expected %d", sp.name.c_str(), w->dtype, c.dtype));
    bool ok = w->ndim == (int)sp.shape.size();
    for (size_t d = 0; ok && d < sp.shape.size(); ++d) ok = w->shape[d] == sp.shape[d];
    if (!ok) {
      std::string got = "[", exp = "[";
      for (int d = 0; d < w->ndim && d < 4; ++d) got += std::to_string(w->shape[d]) + (d + 1 < w->ndim ? "," : "");
      for (size_t d = 0; d < sp.shape.size(); ++d) exp += std::to_string(sp.shape[d]) + (d + 1 < sp.shape.size() ? "," : "");
      return fail(ctx, FM_ERR_SHAPE, fmt("weight '%s': shape %s], expected %s]", sp.name.c_str(), got.c_str(), exp.c_str()));
    }
    if (!w->data) return fail(ctx, FM_ERR_INVALID_ARG, fmt("weight '%s' has no data", sp.name.c_str()));
    byname.erase(it);
  }
  if (!byname.empty()) return fail(ctx, FM_ERR_SHAPE, fmt("unexpected weight '%s'", byname.begin()->first.c_str()));
  for (int i = 0; i < n; ++i) byname[t[i].name] = &t[i];

  HIPCK(hipStreamSynchronize(ctx->stream));
  invalidate_graph(ctx);
  // drop previous weights
  auto drop = [&](void*& p) { dfree(ctx, p); p = nullptr; };
  for (auto& l : ctx->L) {
    drop(l.qkv); drop(l.q); l.kx = l.vx = nullptr; drop(l.o); drop(l.gu); drop(l.down);
    drop(l.q8); drop(l.qkv8); drop(l.o8); drop(l.gu8); drop(l.down8);
    { void* sp[] = {l.sq, l.sqkv, l.so, l.sgu, l.sdown}; for (void* q : sp) dfree(ctx, q); }
    l.sq = l.sqkv = l.so = l.sgu = l.sdown = nullptr;
  }
  ctx->w8 = false;
  drop(ctx->wkx_all); drop(ctx->wvx_all);   // kx / vx point into these
  drop(ctx->w_tin); drop(ctx->w_tout); drop(ctx->w_mod); drop(ctx->w_tb); drop(ctx->w_in); drop(ctx->w_out); drop(ctx->w_state);
  { void* bp[] = {ctx->b_tin, ctx->b_tout, ctx->b_mod, ctx->b_tb, ctx->b_in, ctx->b_out, ctx->b_state}; for (void* q : bp) dfree(ctx, q); }
  ctx->b_tin = ctx->b_tout = ctx->b_mod = ctx->b_tb = ctx->b_in = ctx->b_out = ctx->b_state = nullptr;
  ctx->loaded = false;
  ctx->steps = -1;

  const int elem = ctx->elem;
  const size_t esz = ctx->esz;
  const int D = c.hidden, F = c.mlp_dim;
  fm_status s;
  auto data = [&](const char* nm) { return byname[nm]->data; };
  auto swz = [&](void** dst, const void* src, const int* rows, int N, int K) -> fm_status {
    fm_status st2 = dalloc(ctx, dst, swizzled_bytes(N, K, elem));
    if (st2 != FM_OK) return st2;
    HIPCK(swizzle_weight(*dst, src, rows, N, K, K, elem, ctx->stream));
    return FM_OK;
  };
  auto bias = [&](float** dst, const void* src, long nel) -> fm_status {
    void* p;
    fm_status st2 = dalloc(ctx, &p, round_up(nel, 4) * 4);  // padded: epilogues read 4 floats at a time
    if (st2 != FM_OK) return st2;
    *dst = (float*)p;
    HIPCK(convert_to_f32(*dst, src, nel, elem, ctx->stream));
    return FM_OK;
  };
  auto plain = [&](void** dst, const void* src, size_t bytes) -> fm_status {
    fm_status st2 = dalloc(ctx, dst, bytes);
    if (st2 != FM_OK) return st2;
    HIPCK(hipMemcpyAsync(*dst, src, bytes, hipMemcpyDeviceToDevice, ctx->stream));
    return FM_OK;
  };
  const int S = n_sites(c);
  if ((s = swz(&ctx->w_tin, data("time_in.w"), nullptr, D, D)) != FM_OK) return s;
  if ((s = swz(&ctx->w_tout, data("time_out.w"), nullptr, D, D)) != FM_OK) return s;
  if ((s = swz(&ctx->w_mod, data("mod.w"), nullptr, S * 3 * D, D)) != FM_OK) return s;
  if ((s = swz(&ctx->w_out, data("action_out.w"), nullptr, c.action_dim, D)) != FM_OK) return s;
  if ((s = plain(&ctx->w_in, data("action_in.w"), (size_t)D * c.action_dim * esz)) != FM_OK) return s;
  if ((s = bias(&ctx->b_tin, data("time_in.b"), D)) != FM_OK) return s;
  if ((s = bias(&ctx->b_tout, data("time_out.b"), D)) != FM_OK) return s;
  if ((s = bias(&ctx->b_mod, data("mod.b"), (long)S * 3 * D)) != FM_OK) return s;
  if ((s = bias(&ctx->b_in, data("action_in.b"), D)) != FM_OK) return s;
  if ((s = bias(&ctx->b_out, data("action_out.b"), c.action_dim)) != FM_OK) return s;

  // staging buffer for concatenated row blocks, and device row-index lists
  size_t stage_rows = 0;
  if (c.arch == FM_ARCH_PREFIX_JOINT) stage_rows = std::max((size_t)(c.n_heads + 2) * c.head_dim, (size_t)2 * F);
  else stage_rows = 3 * (size_t)D;
  void* stage = nullptr;
  int* rowidx = nullptr;
  std::vector<int> rows;
  if ((s = dalloc(ctx, &stage, stage_rows * D * esz)) != FM_OK) return s;
  // FP8 weights: the matrix quantized row by row (codes, row scales, dequantized bf16), then
  // the dequantized matrix laid out for the per-operation kernels and the schedule, and the
  // codes and scales for the loop kernel, all in the same output-row order (rows)
  const bool w8 = ctx->wformat == FM_WEIGHTS_FP8_E4M3;
  void *st8 = nullptr, *stsc = nullptr, *stdq = nullptr;
  // the largest quantized matrix: the staged row blocks, or a feed-forward matrix (F x D or
  // D x F), or the pi0.5 output projection (D x n_heads head_dim)
  const size_t qrows = std::max({stage_rows, (size_t)F, (size_t)D});
  size_t qelems = std::max(stage_rows * D, (size_t)F * D);
  if (c.arch == FM_ARCH_PREFIX_JOINT) qelems = std::max(qelems, (size_t)D * c.n_heads * c.head_dim);
  if (w8) {
    if ((s = dalloc(ctx, &st8, qelems)) != FM_OK) return s;
    if ((s = dalloc(ctx, &stsc, qrows * 4)) != FM_OK) return s;
    if ((s = dalloc(ctx, &stdq, qelems * esz)) != FM_OK) return s;
  }
  auto q8 = [&](void** dbf, void** d8, float** dsc, const void* src, const int* rws, int N, int K) -> fm_status {
    if ((size_t)N > qrows || (size_t)N * K > qelems) return fail(ctx, FM_ERR_SHAPE, "FP8 staging smaller than a matrix");
    HIPCK(quantize_fp8_rows(src, K, N, K, (uint8_t*)st8, (float*)stsc, stdq, ctx->stream));
    fm_status st2 = swz(dbf, stdq, rws, N, K);
    if (st2 != FM_OK) return st2;
    if ((st2 = dalloc(ctx, d8, swizzled_fp8_bytes(N, K))) != FM_OK) return st2;
    HIPCK(swizzle_fp8(*d8, (const uint8_t*)st8, rws, N, K, ctx->stream));
    const int Np = (int)round_up(N, 4);
    void* p;
    if ((st2 = dalloc(ctx, &p, (size_t)Np * 4)) != FM_OK) return st2;
    *dsc = (float*)p;
    HIPCK(gather_f32(*dsc, (const float*)stsc, rws, N, Np, ctx->stream));
    return FM_OK;
  };

  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    const int nq = c.n_heads, dh = c.head_dim, qd = nq * dh, N = qd + 2 * dh;
    const bool rope = c.rope_base > 0.f;
    // QKV rows: within each q / k head, output row 2j <- j and 2j+1 <- j + dh/2 (RoPE pairs
    // adjacent); v rows unchanged. Gate/up rows interleaved: 2f <- gate f, 2f+1 <- up f.
    rows.assign(N + 2 * F, 0);
    for (int r = 0; r < N; ++r) {
      const int head0 = (r / dh) * dh, dp = r % dh;
      rows[r] = (r < qd + dh && rope) ? head0 + ((dp & 1) ? dp / 2 + dh / 2 : dp / 2) : r;
    }
    for (int f = 0; f < F; ++f) { rows[N + 2 * f] = f; rows[N + 2 * f + 1] = F + f; }
    {
      void* p;
      if ((s = dalloc(ctx, &p, rows.size() * sizeof(int))) != FM_OK) return s;
      rowidx = (int*)p;
    }
    HIPCK(hipMemcpyAsync(rowidx, rows.data(), rows.size() * sizeof(int), hipMemcpyHostToDevice, ctx->stream));
    HIPCK(hipStreamSynchronize(ctx->stream));
    for (int l = 0; l < c.n_layers; ++l) {
      const std::string p = "layers." + std::to_string(l) + ".";
      auto& W = ctx->L[l];
      HIPCK(hipMemcpyAsync(stage, data((p + "q.w").c_str()), (size_t)qd * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
      HIPCK(hipMemcpyAsync((char*)stage + (size_t)qd * D * esz, data((p + "k.w").c_str()), (size_t)dh * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
      HIPCK(hipMemcpyAsync((char*)stage + (size_t)(qd + dh) * D * esz, data((p + "v.w").c_str()), (size_t)dh * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
      if ((s = w8 ? q8(&W.qkv, &W.qkv8, &W.sqkv, stage, rowidx, N, D) : swz(&W.qkv, stage, rowidx, N, D)) != FM_OK) return s;
      const void* ow = data((p + "o.w").c_str());
      if ((s = w8 ? q8(&W.o, &W.o8, &W.so, ow, nullptr, D, qd) : swz(&W.o, ow, nullptr, D, qd)) != FM_OK) return s;
      const void* dw = data((p + "down.w").c_str());
      if ((s = w8 ? q8(&W.down, &W.down8, &W.sdown, dw, nullptr, D, F) : swz(&W.down, dw, nullptr, D, F)) != FM_OK) return s;
      if (c.mlp_gated) {
        HIPCK(hipMemcpyAsync(stage, data((p + "gate.w").c_str()), (size_t)F * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
        HIPCK(hipMemcpyAsync((char*)stage + (size_t)F * D * esz, data((p + "up.w").c_str()), (size_t)F * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
        if ((s = w8 ? q8(&W.gu, &W.gu8, &W.sgu, stage, rowidx + N, 2 * F, D) : swz(&W.gu, stage, rowidx + N, 2 * F, D)) != FM_OK) return s;
      } else {
        const void* gw = data((p + "gate.w").c_str());
        if ((s = w8 ? q8(&W.gu, &W.gu8, &W.sgu, gw, nullptr, F, D) : swz(&W.gu, gw, nullptr, F, D)) != FM_OK) return s;
      }
    }
  } else {
    if ((s = swz(&ctx->w_tb, data("time_bias.w"), nullptr, D, D)) != FM_OK) return s;
    if ((s = bias(&ctx->b_tb, data("time_bias.b"), D)) != FM_OK) return s;
    if ((s = plain(&ctx->w_state, data("state_in.w"), (size_t)D * c.state_dim * esz)) != FM_OK) return s;
    if ((s = bias(&ctx->b_state, data("state_in.b"), D)) != FM_OK) return s;
    // the cross blocks' K and V weights stacked: the fragment-major [nc D, ctx_dim] matrix is
    // the blocks' [D, ctx_dim] matrices one after another (D is a multiple of 16)
    const size_t xb = swizzled_bytes(D, c.ctx_dim, elem);
    const int nc = (c.n_layers + 1) / 2;
    if ((s = dalloc(ctx, &ctx->wkx_all, nc * xb)) != FM_OK) return s;
    if ((s = dalloc(ctx, &ctx->wvx_all, nc * xb)) != FM_OK) return s;
    for (int i = 0; i < c.n_layers; ++i) {
      const std::string p = "blocks." + std::to_string(i) + ".";
      auto& W = ctx->L[i];
      if (i % 2 == 0) {
        const void* qw = data((p + "q.w").c_str());
        if ((s = w8 ? q8(&W.q, &W.q8, &W.sq, qw, nullptr, D, D) : swz(&W.q, qw, nullptr, D, D)) != FM_OK) return s;
        W.kx = (char*)ctx->wkx_all + (size_t)(i / 2) * xb;
        W.vx = (char*)ctx->wvx_all + (size_t)(i / 2) * xb;
        HIPCK(swizzle_weight(W.kx, data((p + "k.w").c_str()), nullptr, D, c.ctx_dim, c.ctx_dim, elem, ctx->stream));
        HIPCK(swizzle_weight(W.vx, data((p + "v.w").c_str()), nullptr, D, c.ctx_dim, c.ctx_dim, elem, ctx->stream));
      } else {
        HIPCK(hipMemcpyAsync(stage, data((p + "q.w").c_str()), (size_t)D * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
        HIPCK(hipMemcpyAsync((char*)stage + (size_t)D * D * esz, data((p + "k.w").c_str()), (size_t)D * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
        HIPCK(hipMemcpyAsync((char*)stage + (size_t)2 * D * D * esz, data((p + "v.w").c_str()), (size_t)D * D * esz, hipMemcpyDeviceToDevice, ctx->stream));
        if ((s = w8 ? q8(&W.qkv, &W.qkv8, &W.sqkv, stage, nullptr, 3 * D, D) : swz(&W.qkv, stage, nullptr, 3 * D, D)) != FM_OK) return s;
        HIPCK(hipStreamSynchronize(ctx->stream));
      }
      const void* ow = data((p + "o.w").c_str());
      const void* f1 = data((p + "ff1.w").c_str());
      const void* f2 = data((p + "ff2.w").c_str());
      if ((s = w8 ? q8(&W.o, &W.o8, &W.so, ow, nullptr, D, D) : swz(&W.o, ow, nullptr, D, D)) != FM_OK) return s;
      if ((s = w8 ? q8(&W.gu, &W.gu8, &W.sgu, f1, nullptr, F, D) : swz(&W.gu, f1, nullptr, F, D)) != FM_OK) return s;
      if ((s = w8 ? q8(&W.down, &W.down8, &W.sdown, f2, nullptr, D, F) : swz(&W.down, f2, nullptr, D, F)) != FM_OK) return s;
    }
  }
  if (c.arch == FM_ARCH_DIT_CROSS) {
    // d of the feed-forward LayerNorm (no modulation): row sums of the FF1 weights
    HIPCK(fill_f32((float*)stage, 1.f, D, ctx->stream));
    HIPCK(rows_from_f32(ctx->row_buf, D, (const float*)stage, D, 1, D, 0.f, elem, ctx->stream));
    for (int i = 0; i < c.n_layers; ++i) {
      std::vector<Op> one(1);
      memset(&one[0], 0, sizeof(Op));
      one[0].kind = Op::GEMM;
      GemmArgs& gg = one[0].g;
      gg = gemm_base(1, F, D, ctx->L[i].gu);
      gg.A = ctx->row_buf; gg.lda = D; gg.epi = EPI_STORE; gg.out_f32 = 1; gg.ldo = F;
      gg.out = ctx->dff + (size_t)i * F;
      if ((s = plan_ops(ctx, one)) != FM_OK) return s;
      if ((s = enqueue_ops(ctx, one, ctx->stream, nullptr)) != FM_OK) return s;
    }
  }
  HIPCK(hipStreamSynchronize(ctx->stream));
  dfree(ctx, stage);
  dfree(ctx, rowidx);
  dfree(ctx, st8); dfree(ctx, stsc); dfree(ctx, stdq);
  ctx->w8 = w8;
  ctx->loaded = true;
  ctx->prefix_len = -1;  // a binding may depend on the previous weights (DiT projections)
  return FM_OK;
}

fm_status fm_set_weight_format(fm_ctx* ctx, int32_t format) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  const fm_config& c = ctx->c;
  if (format != FM_WEIGHTS_AS_GIVEN && format != FM_WEIGHTS_FP8_E4M3)
    return fail(ctx, FM_ERR_INVALID_ARG, fmt("weight format %d", format));
  if (format == FM_WEIGHTS_FP8_E4M3 &&
      (c.dtype != FM_BF16 || c.mlp_dim % 64 != 0 || (c.arch == FM_ARCH_DIT_CROSS && c.hidden % 64 != 0)))
    return fail(ctx, FM_ERR_UNSUPPORTED, "FP8 weights need bf16, mlp_dim a multiple of 64 and (DiT head) hidden a multiple of 64");
  ctx->wformat = format;
  return FM_OK;
}

fm_status fm_op_quantize_fp8(int32_t N, int32_t K, const void* src, void* codes, float* scale, void* deq, void* hip_stream) {
  if (N < 0 || K < 2 || K % 2 || !src || !codes || !scale || !deq) { g_err = "fm_op_quantize_fp8: bad arguments"; return FM_ERR_INVALID_ARG; }
  hipStream_t st = (hipStream_t)hip_stream;
  hipError_t e = quantize_fp8_rows(src, K, N, K, (uint8_t*)codes, scale, deq, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) { g_err = fmt("fm_op_quantize_fp8: %s", hipGetErrorString(e)); return FM_ERR_DEVICE; }
  return FM_OK;
}

fm_status fm_set_schedule(fm_ctx* ctx, int32_t steps, int32_t batch, const float* tau_host) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!ctx->loaded) return fail(ctx, FM_ERR_STATE, "weights are not loaded");
  const fm_config& c = ctx->c;
  if (steps < 0 || steps > c.max_steps) return fail(ctx, FM_ERR_INVALID_ARG, fmt("steps %d outside [0, %d]", steps, c.max_steps));
  if (batch < 1 || batch > c.max_batch) return fail(ctx, FM_ERR_INVALID_ARG, fmt("batch %d outside [1, %d]", batch, c.max_batch));
  std::vector<float> tau(steps + 1);
  for (int k = 0; k <= steps; ++k) {
    tau[k] = tau_host ? tau_host[k] : (steps > 0 ? (float)(1.0 - (double)k / steps) : 1.f);
    if (!std::isfinite(tau[k])) return fail(ctx, FM_ERR_INVALID_ARG, fmt("tau[%d] is not finite", k));
  }
  HIPCK(hipStreamSynchronize(ctx->stream));
  invalidate_graph(ctx);
  ctx->tau = tau;
  ctx->steps = steps;
  ctx->sched_batch = batch;
  if (steps == 0) return FM_OK;
  if (ctx->dts) {
    std::vector<float> dts(steps);
    for (int k = 0; k < steps; ++k) dts[k] = tau[k + 1] - tau[k];
    HIPCK(hipMemcpyAsync(ctx->dts, dts.data(), dts.size() * sizeof(float), hipMemcpyHostToDevice, ctx->stream));
  }
  const int D = c.hidden, S = n_sites(c), T = steps;
  // sinusoidal time embedding of tau_0..tau_{T-1}, evaluated in double on the host:
  // [sin(2 pi tau / p_j)] ++ [cos(2 pi tau / p_j)], periods geometric from 4e-3 to 4
  std::vector<float> e((size_t)T * D);
  const int half = D / 2;
  for (int k = 0; k < T; ++k)
    for (int j = 0; j < half; ++j) {
      const double frac = half > 1 ? (double)j / (half - 1) : 0.0;
      const double period = 4e-3 * std::pow(4.0 / 4e-3, frac);
      const double arg = (double)tau[k] * 2.0 * 3.14159265358979323846 / period;
      e[(size_t)k * D + j] = (float)std::sin(arg);
      e[(size_t)k * D + half + j] = (float)std::cos(arg);
    }
  float* e32 = nullptr;
  {
    void* p;
    fm_status s = dalloc(ctx, &p, e.size() * 4);
    if (s != FM_OK) return s;
    e32 = (float*)p;
  }
  HIPCK(hipMemcpyAsync(e32, e.data(), e.size() * 4, hipMemcpyHostToDevice, ctx->stream));
  HIPCK(convert_from_f32(ctx->e_buf, e32, (long)T * D, ctx->elem, ctx->stream));
  std::vector<Op> ops;
  Op op;
  auto add = [&](GemmArgs g) { memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.g = g; ops.push_back(op); };
  GemmArgs g = gemm_base(T, D, D, ctx->w_tin);
  g.A = ctx->e_buf; g.lda = D; g.epi = EPI_STORE; g.bias = ctx->b_tin; g.act = ACT_SILU; g.out = ctx->c1_buf; g.ldo = D;
  add(g);
  g = gemm_base(T, D, D, ctx->w_tout);
  g.A = ctx->c1_buf; g.lda = D; g.epi = EPI_STORE; g.bias = ctx->b_tout; g.act = ACT_SILU; g.out = ctx->c_buf; g.ldo = D;
  add(g);
  g = gemm_base(T, S * 3 * D, D, ctx->w_mod);
  g.A = ctx->c_buf; g.lda = D; g.epi = EPI_STORE; g.bias = ctx->b_mod; g.out = ctx->table; g.ldo = (long)S * 3 * D; g.out_f32 = 1;
  add(g);
  if (c.arch == FM_ARCH_DIT_CROSS) {
    g = gemm_base(T, D, D, ctx->w_tb);
    g.A = ctx->c_buf; g.lda = D; g.epi = EPI_STORE; g.bias = ctx->b_tb; g.out = ctx->tbias; g.ldo = D; g.out_f32 = 1;
    add(g);
  }
  fm_status s = plan_ops(ctx, ops);
  if (s != FM_OK) return s;
  if ((s = enqueue_ops(ctx, ops, ctx->stream, nullptr)) != FM_OK) return s;
  // per site: c = shift W^T and, for LayerNorm, d = (1 + scale) W^T of the consumer weights
  for (int site = 0; site < S; ++site) {
    auto cw = site_consumer(ctx, site);
    for (int which = 0; which < (c.arch == FM_ARCH_DIT_CROSS ? 2 : 1); ++which) {
      const float* src = ctx->table + (size_t)site * 3 * D + (which == 0 ? D : 0);
      HIPCK(rows_from_f32(ctx->row_buf, D, src, (long)S * 3 * D, T, D, which == 0 ? 0.f : 1.f, ctx->elem, ctx->stream));
      std::vector<Op> one(1);
      memset(&one[0], 0, sizeof(Op));
      one[0].kind = Op::GEMM;
      GemmArgs& gg = one[0].g;
      gg = gemm_base(T, cw.second, D, cw.first);
      gg.A = ctx->row_buf; gg.lda = D; gg.epi = EPI_STORE; gg.out_f32 = 1; gg.ldo = ctx->csum;
      gg.out = (which == 0 ? ctx->cbuf : ctx->dbuf) + ctx->c_off[site];
      if ((s = plan_ops(ctx, one)) != FM_OK) return s;
      if ((s = enqueue_ops(ctx, one, ctx->stream, nullptr)) != FM_OK) return s;
    }
  }
  HIPCK(hipStreamSynchronize(ctx->stream));
  dfree(ctx, e32);
  return FM_OK;
}

// Per-request compact prefix lengths and the cos/sin rows of each request's chunk positions
// P_b + i. Device copies on the context stream (ordered after any loop still running on it),
// then a wait, so the host vectors may go.
static fm_status upload_lengths(fm_ctx* ctx, const std::vector<int>& lens, int P) {
  const int H = ctx->c.action_horizon, hd = ctx->c.head_dim / 2, B = (int)lens.size();
  std::vector<float2> cs((size_t)B * H * hd);
  for (int b = 0; b < B; ++b)
    memcpy(&cs[(size_t)b * H * hd], &ctx->rope_pos[(size_t)lens[b] * hd], (size_t)H * hd * sizeof(float2));
  HIPCK(hipMemcpyAsync(ctx->rope_cs, cs.data(), cs.size() * sizeof(float2), hipMemcpyHostToDevice, ctx->stream));
  HIPCK(hipMemcpyAsync(ctx->plens, lens.data(), (size_t)B * sizeof(int), hipMemcpyHostToDevice, ctx->stream));
  ctx->plens_host = lens;
  HIPCK(hipStreamSynchronize(ctx->stream));
  bool ragged = false;
  for (int b = 0; b < B; ++b) ragged |= lens[b] != P;
  if (ragged != ctx->ragged) { ctx->ragged = ragged; invalidate_graph(ctx); }   // the attention variant changes
  return FM_OK;
}

// Text and image masks of the DiT cross blocks, bit-packed per request (NULL: every token of
// the bound context visible). A mask that some cross block reads must show each request at
// least one token: softmax over no visible key has no value.
static fm_status upload_masks(fm_ctx* ctx, int batch, int S, const uint8_t* text, const uint8_t* image) {
  const fm_config& c = ctx->c;
  const int W = ctx->ctx_words;
  std::vector<uint32_t> bits((size_t)2 * c.max_batch * W, 0u);
  const uint8_t* src[2] = {text, image};
  const bool read[2] = {c.n_layers >= 1, c.n_layers >= 3};   // block 0 reads text, block 2 image
  const char* name[2] = {"text", "image"};
  bool hidden[2] = {false, false};
  for (int m = 0; m < 2; ++m)
    for (int b = 0; b < batch; ++b) {
      uint32_t* w = &bits[((size_t)m * c.max_batch + b) * W];
      int seen = 0;
      for (int j = 0; j < S; ++j)
        if (!src[m] || src[m][(size_t)b * S + j]) { w[j / 32] |= 1u << (j % 32); ++seen; }
      if (read[m] && seen == 0)
        return fail(ctx, FM_ERR_INVALID_ARG, fmt("the %s mask shows request %d no context token", name[m], b));
      hidden[m] |= seen < S;
    }
  HIPCK(hipMemcpyAsync(ctx->kmask, bits.data(), bits.size() * sizeof(uint32_t), hipMemcpyHostToDevice, ctx->stream));
  HIPCK(hipStreamSynchronize(ctx->stream));
  if (hidden[0] != ctx->masked[0] || hidden[1] != ctx->masked[1]) {   // the attention variant changes
    ctx->masked[0] = hidden[0]; ctx->masked[1] = hidden[1];
    invalidate_graph(ctx);
  }
  return FM_OK;
}

fm_status fm_bind_prefix_kv(fm_ctx* ctx, int32_t batch, int32_t plen, const void* const* k_dev,
                            const void* const* v_dev, const void* ctx_dev, const void* state_dev) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!ctx->loaded) return fail(ctx, FM_ERR_STATE, "weights are not loaded");
  const fm_config& c = ctx->c;
  if (batch < 1 || batch > c.max_batch) return fail(ctx, FM_ERR_INVALID_ARG, fmt("batch %d outside [1, %d]", batch, c.max_batch));
  const int D = c.hidden;
  if (c.arch == FM_ARCH_PREFIX_JOINT) {
    if (plen < 0 || plen > c.max_prefix_len) return fail(ctx, FM_ERR_INVALID_ARG, fmt("prefix_len %d outside [0, %d]", plen, c.max_prefix_len));
    if (ctx_dev || state_dev) return fail(ctx, FM_ERR_INVALID_ARG, "ctx_dev / state_dev must be NULL for the prefix-joint expert");
    if (plen > 0 && (!k_dev || !v_dev)) return fail(ctx, FM_ERR_INVALID_ARG, "k_dev / v_dev are NULL");
    for (int l = 0; plen > 0 && l < c.n_layers; ++l)
      if (!k_dev[l] || !v_dev[l]) return fail(ctx, FM_ERR_INVALID_ARG, fmt("prefix K/V of layer %d is NULL", l));
    HIPCK(hipStreamSynchronize(ctx->stream));
    invalidate_graph(ctx);
    const int dh = c.head_dim;
    const size_t plane = (size_t)c.max_batch * ctx->cap * dh * ctx->esz;
    for (int l = 0; plen > 0 && l < c.n_layers; ++l) {
      HIPCK(prefix_k_copy((char*)ctx->pool + 2 * l * plane, (long)ctx->cap * dh, k_dev[l], batch, plen, dh, c.rope_base > 0.f, ctx->elem, ctx->stream));
      HIPCK(prefix_v_copy_t((char*)ctx->pool + (2 * l + 1) * plane, (long)dh * ctx->cap, ctx->cap, v_dev[l], batch, plen, dh, ctx->elem, ctx->stream));
    }
    // every request sees the whole bound prefix until fm_bind_prefix_lengths says otherwise
    std::vector<int> lens(batch, plen);
    fm_status s = upload_lengths(ctx, lens, plen);
    if (s != FM_OK) return s;
  } else {
    if (plen < 1 || plen > c.ctx_len_max) return fail(ctx, FM_ERR_INVALID_ARG, fmt("context length %d outside [1, %d]", plen, c.ctx_len_max));
    if (k_dev || v_dev) return fail(ctx, FM_ERR_INVALID_ARG, "k_dev / v_dev must be NULL for the DiT head");
    if (!ctx_dev) return fail(ctx, FM_ERR_INVALID_ARG, "ctx_dev is NULL");
    if (c.state_tokens > 0 && !state_dev) return fail(ctx, FM_ERR_INVALID_ARG, "state_dev is NULL");
    HIPCK(hipStreamSynchronize(ctx->stream));
    invalidate_graph(ctx);
    std::vector<Op> ops;
    Op op;
    // K_c = Z W_K^T and V_c = Z W_V^T of every cross block as two GEMMs over the stacked
    // weights (GR00T N1.7, "vl_backbone": projected once per observation), each output column
    // block of width D going to its cross block's plane
    const int nc = (c.n_layers + 1) / 2;
    if (nc > 0) {
      GemmArgs g = gemm_base(batch * plen, nc * D, c.ctx_dim, ctx->wkx_all);
      g.A = ctx_dev; g.lda = c.ctx_dim;
      g.epi = EPI_STORE; g.out = ctx->cross_k; g.ldo = D;   // rows b*plen + s: packed per request
      g.col_group = D; g.col_gstride = (long)c.max_batch * c.ctx_len_max * D;
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.g = g; ops.push_back(op);
      g = gemm_base(batch * plen, nc * D, c.ctx_dim, ctx->wvx_all);
      g.A = ctx_dev; g.lda = c.ctx_dim;
      g.epi = EPI_VT; g.out = ctx->cross_vt;
      g.vt_group = plen; g.vt_bs = (long)D * ctx->spad; g.vt_ds = ctx->spad;
      g.col_group = D; g.col_gstride = (long)c.max_batch * D * ctx->spad;
      memset(&op, 0, sizeof op); op.kind = Op::GEMM; op.g = g; ops.push_back(op);
    }
    if (c.state_tokens > 0) {
      memset(&op, 0, sizeof op);
      op.kind = Op::INPROJ;
      op.ip.x = (const float*)state_dev; op.ip.da = c.state_dim; op.ip.w = ctx->w_state; op.ip.b = ctx->b_state;
      op.ip.B = batch * c.state_tokens; op.ip.Ha = 1; op.ip.st = 0; op.ip.D = D; op.ip.h = ctx->state_tok; op.ip.stats = nullptr; op.ip.zeros = ctx->zeros;
      ops.push_back(op);
    }
    fm_status s = plan_ops(ctx, ops);
    if (s != FM_OK) return s;
    if ((s = enqueue_ops(ctx, ops, ctx->stream, nullptr)) != FM_OK) return s;
    // every context token visible until fm_bind_context_masks says otherwise
    if ((s = upload_masks(ctx, batch, plen, nullptr, nullptr)) != FM_OK) return s;
  }
  ctx->bound_batch = batch;
  ctx->prefix_len = plen;
  return FM_OK;
}

fm_status fm_prefix_kv_slot(fm_ctx* ctx, int32_t layer, void** k_dev, void** v_dev) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  const fm_config& c = ctx->c;
  if (c.arch != FM_ARCH_PREFIX_JOINT) return fail(ctx, FM_ERR_UNSUPPORTED, "the prefix K/V pool belongs to the prefix-joint expert");
  if (layer < 0 || layer >= c.n_layers || !k_dev || !v_dev)
    return fail(ctx, FM_ERR_INVALID_ARG, fmt("fm_prefix_kv_slot: layer %d outside [0, %d) or a NULL output", layer, c.n_layers));
  const size_t plane = (size_t)c.max_batch * ctx->cap * c.head_dim * ctx->esz;
  *k_dev = (char*)ctx->pool + (size_t)(2 * layer) * plane;
  *v_dev = (char*)ctx->pool + (size_t)(2 * layer + 1) * plane;
  return FM_OK;
}

fm_status fm_bind_prefix_inplace(fm_ctx* ctx, int32_t batch, int32_t plen) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!ctx->loaded) return fail(ctx, FM_ERR_STATE, "weights are not loaded");
  const fm_config& c = ctx->c;
  if (c.arch != FM_ARCH_PREFIX_JOINT) return fail(ctx, FM_ERR_UNSUPPORTED, "an in-place binding belongs to the prefix-joint expert");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, FM_ERR_INVALID_ARG, fmt("batch %d outside [1, %d]", batch, c.max_batch));
  if (plen < 0 || plen > c.max_prefix_len) return fail(ctx, FM_ERR_INVALID_ARG, fmt("prefix_len %d outside [0, %d]", plen, c.max_prefix_len));
  HIPCK(hipStreamSynchronize(ctx->stream));   // the producer's writes on this stream are done
  invalidate_graph(ctx);
  std::vector<int> lens(batch, plen);
  fm_status s = upload_lengths(ctx, lens, plen);
  if (s != FM_OK) return s;
  ctx->bound_batch = batch;
  ctx->prefix_len = plen;
  return FM_OK;
}

fm_status fm_bind_prefix_lengths(fm_ctx* ctx, const int32_t* lens_host) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (ctx->c.arch != FM_ARCH_PREFIX_JOINT) return fail(ctx, FM_ERR_UNSUPPORTED, "per-request prefix lengths belong to the prefix-joint expert");
  if (ctx->prefix_len < 0) return fail(ctx, FM_ERR_STATE, "nothing bound: call fm_bind_prefix_kv first");
  std::vector<int> lens(ctx->bound_batch, ctx->prefix_len);
  for (int b = 0; lens_host && b < ctx->bound_batch; ++b) {
    if (lens_host[b] < 0 || lens_host[b] > ctx->prefix_len)
      return fail(ctx, FM_ERR_INVALID_ARG, fmt("prefix length %d of request %d outside [0, %d]", lens_host[b], b, ctx->prefix_len));
    lens[b] = lens_host[b];
  }
  return upload_lengths(ctx, lens, ctx->prefix_len);
}

fm_status fm_bind_context_masks(fm_ctx* ctx, const uint8_t* text_host, const uint8_t* image_host) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (ctx->c.arch != FM_ARCH_DIT_CROSS) return fail(ctx, FM_ERR_UNSUPPORTED, "context masks belong to the DiT head");
  if (ctx->prefix_len < 0) return fail(ctx, FM_ERR_STATE, "nothing bound: call fm_bind_prefix_kv first");
  return upload_masks(ctx, ctx->bound_batch, ctx->prefix_len, text_host, image_host);
}

static fm_status capture_loop(fm_ctx* ctx) {
  invalidate_graph(ctx);
  std::vector<std::vector<Op>> steps;
  for (int k = 0; k < ctx->steps; ++k) {
    steps.push_back(build_step(ctx, k, nullptr, nullptr));
    fm_status s = plan_ops(ctx, steps.back());
    if (s != FM_OK) return s;
  }
  HIPCK(hipStreamBeginCapture(ctx->cap_stream, hipStreamCaptureModeThreadLocal));
  for (auto& ops : steps) {
    fm_status s = enqueue_ops(ctx, ops, ctx->cap_stream, nullptr);
    if (s != FM_OK) {
      hipGraph_t g;
      (void)hipStreamEndCapture(ctx->cap_stream, &g);
      if (g) (void)hipGraphDestroy(g);
      return s;
    }
  }
  HIPCK(hipStreamEndCapture(ctx->cap_stream, &ctx->graph));
  HIPCK(hipGraphInstantiate(&ctx->gexec, ctx->graph, nullptr, nullptr, 0));
  ctx->graph_valid = true;
  return FM_OK;
}

fm_status fm_denoise(fm_ctx* ctx, const float* x0, int32_t steps, float* out) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  fm_status s = check_ready(ctx);
  if (s != FM_OK) return s;
  if (!x0 || !out) return fail(ctx, FM_ERR_INVALID_ARG, "x0 / out is NULL");
  if (steps != ctx->steps)
    return fail(ctx, FM_ERR_SCHEDULE, fmt("steps %d differs from the scheduled %d", steps, ctx->steps));
  const size_t xbytes = (size_t)ctx->bound_batch * ctx->c.action_horizon * ctx->c.action_dim * sizeof(float);
  if (steps == 0) {
    if (out != x0) HIPCK(hipMemcpyAsync(out, x0, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    return FM_OK;
  }
  if (!loop_unsupported(ctx)) {
    HIPCK(hipMemcpyAsync(ctx->x, x0, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    if ((s = loop_run(ctx, 0, steps, nullptr)) != FM_OK) return s;
    HIPCK(hipMemcpyAsync(out, ctx->x, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    return FM_OK;
  }
  if (!ctx->graph_valid && (s = capture_loop(ctx)) != FM_OK) return s;
  HIPCK(hipMemcpyAsync(ctx->x, x0, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
  HIPCK(hipGraphLaunch(ctx->gexec, ctx->stream));
  HIPCK(hipMemcpyAsync(out, ctx->x, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
  return FM_OK;
}

static fm_status step_eager(fm_ctx* ctx, const float* xin, int32_t k, float* v, float* trace) {
  fm_status s = check_ready(ctx);
  if (s != FM_OK) return s;
  if (!xin || !v) return fail(ctx, FM_ERR_INVALID_ARG, "x / v is NULL");
  if (k < 0 || k >= ctx->steps) return fail(ctx, FM_ERR_SCHEDULE, fmt("step %d outside the scheduled [0, %d)", k, ctx->steps));
  const size_t xbytes = (size_t)ctx->bound_batch * ctx->c.action_horizon * ctx->c.action_dim * sizeof(float);
  if (!trace && !loop_unsupported(ctx)) {
    HIPCK(hipMemcpyAsync(ctx->x, xin, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    return loop_run(ctx, k, 1, v);
  }
  std::vector<Op> ops = build_step(ctx, k, v, trace);
  if ((s = plan_ops(ctx, ops)) != FM_OK) return s;
  HIPCK(hipMemcpyAsync(ctx->x, xin, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
  return enqueue_ops(ctx, ops, ctx->stream, trace);
}

fm_status fm_step_velocity(fm_ctx* ctx, const float* x, int32_t k, float* v) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  return step_eager(ctx, x, k, v, nullptr);
}

fm_status fm_set_action_stats(fm_ctx* ctx, int32_t kind, int32_t robot_horizon, int32_t robot_dim,
                              const float* q01_host, const float* q99_host) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  const fm_config& c = ctx->c;
  if ((kind != FM_UNNORM_QUANTILE_EPS && kind != FM_UNNORM_QUANTILE_CLIP) || robot_horizon < 1 ||
      robot_horizon > c.action_horizon || robot_dim < 1 || robot_dim > c.action_dim || !q01_host || !q99_host)
    return fail(ctx, FM_ERR_INVALID_ARG,
                fmt("fm_set_action_stats: kind %d, robot horizon %d (1..%d), robot dim %d (1..%d), q01/q99 %s", kind,
                    robot_horizon, c.action_horizon, robot_dim, c.action_dim, q01_host && q99_host ? "given" : "missing"));
  if (!ctx->q01) {
    void* p;
    fm_status s = dalloc(ctx, &p, 2 * (size_t)c.action_dim * sizeof(float));
    if (s != FM_OK) return s;
    ctx->q01 = (float*)p;
    ctx->q99 = ctx->q01 + c.action_dim;
  }
  HIPCK(hipMemcpyAsync(ctx->q01, q01_host, (size_t)robot_dim * sizeof(float), hipMemcpyHostToDevice, ctx->stream));
  HIPCK(hipMemcpyAsync(ctx->q99, q99_host, (size_t)robot_dim * sizeof(float), hipMemcpyHostToDevice, ctx->stream));
  // the host arrays may be reused once this returns
  HIPCK(hipStreamSynchronize(ctx->stream));
  ctx->unnorm_kind = kind; ctx->robot_h = robot_horizon; ctx->robot_d = robot_dim;
  return FM_OK;
}

fm_status fm_unnormalize(fm_ctx* ctx, const float* x, float* out) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  if (!x || !out) return fail(ctx, FM_ERR_INVALID_ARG, "fm_unnormalize: x or out is NULL");
  if (ctx->unnorm_kind < 0) return fail(ctx, FM_ERR_STATE, "fm_unnormalize before fm_set_action_stats");
  if (ctx->bound_batch < 1) return fail(ctx, FM_ERR_STATE, "fm_unnormalize before a binding");
  const fm_config& c = ctx->c;
  HIPCK(unnormalize_launch(x, out, ctx->q01, ctx->q99, ctx->bound_batch, c.action_horizon, c.action_dim, ctx->robot_h,
                           ctx->robot_d, ctx->unnorm_kind, ctx->stream));
  return FM_OK;
}

fm_status fm_step_trace(fm_ctx* ctx, const float* x, int32_t k, float* v, float* trace) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (!trace) return fail(ctx, FM_ERR_INVALID_ARG, "h_trace is NULL");
  return step_eager(ctx, x, k, v, trace);
}

fm_status fm_profile_loop(fm_ctx* ctx, const float* x0, int32_t steps, float* out, int32_t role, float* ms,
                          int32_t* launches) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  fm_status s = check_ready(ctx);
  if (s != FM_OK) return s;
  if (!x0 || !out || !ms || !launches || role < FM_OP_INPROJ || role > FM_OP_LOOP)
    return fail(ctx, FM_ERR_INVALID_ARG, "fm_profile_loop: bad arguments");
  if (steps != ctx->steps || steps < 1)
    return fail(ctx, FM_ERR_SCHEDULE, fmt("steps %d differs from the scheduled %d", steps, ctx->steps));
  const size_t xbytes = (size_t)ctx->bound_batch * ctx->c.action_horizon * ctx->c.action_dim * sizeof(float);
  if (role == FM_OP_LOOP) {
    const char* why = loop_unsupported(ctx);
    if (why) return fail(ctx, FM_ERR_UNSUPPORTED, fmt("the loop kernel does not serve this loop: %s", why));
    hipEvent_t e0, e1;
    HIPCK(hipEventCreate(&e0));
    HIPCK(hipEventCreate(&e1));
    HIPCK(hipMemcpyAsync(ctx->x, x0, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    if ((s = loop_buffers(ctx, ctx->steps)) != FM_OK) return s;
    HIPCK(hipEventRecord(e0, ctx->stream));
    if ((s = loop_run(ctx, 0, steps, nullptr)) != FM_OK) return s;
    HIPCK(hipEventRecord(e1, ctx->stream));
    HIPCK(hipMemcpyAsync(out, ctx->x, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
    HIPCK(hipStreamSynchronize(ctx->stream));
    float e = 0;
    HIPCK(hipEventElapsedTime(&e, e0, e1));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms = e;
    *launches = 1;
    return FM_OK;
  }
  std::vector<std::vector<Op>> all;
  size_t count = 0;
  for (int k = 0; k < steps; ++k) {
    all.push_back(build_step(ctx, k, nullptr, nullptr));
    if ((s = plan_ops(ctx, all.back())) != FM_OK) return s;
    for (auto& op : all.back()) count += op.role == role;
  }
  std::vector<hipEvent_t> ev(2 * count);
  for (auto& e : ev) HIPCK(hipEventCreate(&e));
  HIPCK(hipMemcpyAsync(ctx->x, x0, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
  size_t i = 0;
  for (auto& ops : all)
    for (auto& op : ops) {
      const bool hit = op.role == role;
      if (hit) HIPCK(hipEventRecord(ev[2 * i], ctx->stream));
      std::vector<Op> one(1, op);
      if ((s = enqueue_ops(ctx, one, ctx->stream, nullptr)) != FM_OK) return s;
      if (hit) { HIPCK(hipEventRecord(ev[2 * i + 1], ctx->stream)); ++i; }
    }
  HIPCK(hipMemcpyAsync(out, ctx->x, xbytes, hipMemcpyDeviceToDevice, ctx->stream));
  HIPCK(hipStreamSynchronize(ctx->stream));
  double tot = 0;
  for (size_t j = 0; j < count; ++j) {
    float e = 0;
    HIPCK(hipEventElapsedTime(&e, ev[2 * j], ev[2 * j + 1]));
    tot += e;
  }
  for (auto& e : ev) (void)hipEventDestroy(e);
  *ms = (float)tot;
  *launches = (int32_t)count;
  return FM_OK;
}

fm_status fm_set_loop_mode(fm_ctx* ctx, int32_t mode) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (mode != FM_LOOP_AUTO && mode != FM_LOOP_GRAPH) return fail(ctx, FM_ERR_INVALID_ARG, fmt("loop mode %d", mode));
  ctx->loop_mode = mode;
  return FM_OK;
}

fm_status fm_loop_status(fm_ctx* ctx, int32_t* persistent, uint32_t* fault) {
  if (!ctx) { g_err = "ctx is NULL"; return FM_ERR_INVALID_ARG; }
  if (ctx->poisoned) return FM_ERR_DEVICE;
  HIPCK(hipStreamSynchronize(ctx->stream));
  if (persistent) *persistent = (ctx->loaded && !loop_unsupported(ctx)) ? 1 : 0;
  uint32_t f = 0;
  if (ctx->pflags) HIPCK(hipMemcpy(&f, ctx->pflags + kXErr, sizeof f, hipMemcpyDeviceToHost));
  if (fault) *fault = f;
  if (f != 0) {
    (void)hipMemset(ctx->pflags, 0, kXFlagWords * sizeof(uint32_t));
    ctx->xb_base = ctx->ag_base = ctx->pe_base = 0;
    if (f == kXFaultSlot)
      return fail(ctx, FM_ERR_DEVICE, "loop kernel: two workgroups ran on one (XCD, rank) slot (the dispatch was not round-robin over the XCDs); results are invalid");
    return fail(ctx, FM_ERR_DEVICE, fmt("loop kernel: a bounded wait expired (fault word %u); results are invalid", f));
  }
  return FM_OK;
}

// ---------------------------------------------------------------------------------------
// Kernel-level entry points (own scratch, synchronous).
// ---------------------------------------------------------------------------------------
fm_status fm_op_linear(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, const void* W,
                       const float* bias, int32_t act, void* out, int32_t out_f32, void* stream) {
  const int elem = dtype == FM_BF16 ? ET_BF16 : ET_F32;
  const int kq = dtype == FM_BF16 ? 32 : 16;
  if ((dtype != FM_F32 && dtype != FM_BF16) || M < 0 || N < 1 || K < kq || K % kq != 0 || !A || !W || !out ||
      act < 0 || act > 2) {
    g_err = fmt("fm_op_linear: bad arguments (M %d N %d K %d, K a multiple of %d)", M, N, K, kq);
    return FM_ERR_INVALID_ARG;
  }
  if (M == 0) return FM_OK;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) { g_err = "no device"; return FM_ERR_DEVICE; }
  GemmArgs g = gemm_base(M, N, K, nullptr);
  g.A = A; g.lda = K; g.epi = EPI_STORE; g.bias = bias; g.act = act; g.out = out; g.ldo = N; g.out_f32 = out_f32;
  gemm_plan(g, elem, prop.multiProcessorCount);
  void *wsw = nullptr, *ws = nullptr, *cnt = nullptr, *bpad = nullptr, *zo = nullptr;
  hipError_t e = hipMalloc(&wsw, swizzled_bytes(N, K, elem));
  if (e == hipSuccess) e = hipMalloc(&zo, 2 * kVecPad * sizeof(float));
  if (e == hipSuccess) e = hipMemsetAsync(zo, 0, kVecPad * sizeof(float), s);
  if (e == hipSuccess) e = fill_f32((float*)zo + kVecPad, 1.f, kVecPad, s);
  g.zeros = (const float*)zo; g.ones = (const float*)zo + kVecPad;
  const size_t wsb = gemm_ws_bytes(g);
  if (e == hipSuccess && bias) {
    e = hipMalloc(&bpad, (size_t)round_up(N, 4) * 4);
    if (e == hipSuccess) e = hipMemsetAsync(bpad, 0, (size_t)round_up(N, 4) * 4, s);
    if (e == hipSuccess) e = hipMemcpyAsync(bpad, bias, (size_t)N * 4, hipMemcpyDeviceToDevice, s);
    g.bias = (const float*)bpad;
  }
  if (e == hipSuccess && wsb) e = hipMalloc(&ws, wsb);
  if (e == hipSuccess) e = hipMalloc(&cnt, kGemmCounters * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemsetAsync(cnt, 0, kGemmCounters * sizeof(unsigned), s);
  if (e == hipSuccess) e = swizzle_weight(wsw, W, nullptr, N, K, K, elem, s);
  g.W = wsw; g.ws = (float*)ws; g.counters = (unsigned*)cnt;
  if (e == hipSuccess && g.splits > 1 && gemm_num_tiles(g) > kGemmCounters) e = hipErrorInvalidValue;
  if (e == hipSuccess) e = gemm_launch(g, elem, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipError_t e2 = hipSuccess;
  if (wsw) e2 = hipFree(wsw);
  if (bpad) (void)hipFree(bpad);
  if (ws) (void)hipFree(ws);
  if (cnt) (void)hipFree(cnt);
  if (zo) (void)hipFree(zo);
  if (e == hipSuccess) e = e2;
  if (e != hipSuccess) { g_err = fmt("fm_op_linear: %s", hipGetErrorString(e)); return FM_ERR_DEVICE; }
  return FM_OK;
}

fm_status fm_op_attention(int32_t dtype, int32_t B, int32_t Tq, int32_t nh, int32_t nkv, int32_t nk, int32_t dh,
                          const void* q, const void* k, const void* v, void* o, void* stream) {
  const int elem = dtype == FM_BF16 ? ET_BF16 : ET_F32;
  if ((dtype != FM_F32 && dtype != FM_BF16) || B < 1 || Tq < 1 || nh < 1 || nk < 1 || (nkv != 1 && nkv != nh) ||
      !q || !k || !v || !o || (dh != 64 && dh != 128 && dh != 256) || (dtype == FM_F32 && dh == 256)) {
    g_err = "fm_op_attention: bad arguments";
    return FM_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) { g_err = "no device"; return FM_ERR_DEVICE; }
  const size_t esz = elem == ET_BF16 ? 2 : 4;
  const int kpad = (int)round_up(nk, 64);   // whole key tiles in the transposed V plane
  AttnArgs at;
  memset(&at, 0, sizeof at);
  at.q = q; at.q_bs = (long)Tq * nh * dh; at.q_rs = (long)nh * dh;
  at.k = k; at.k_bs = (long)nkv * nk * dh; at.k_rs = dh; at.k_hs = (long)nk * dh;
  at.o = o; at.o_bs = at.q_bs; at.o_rs = at.q_rs;
  at.v_bs = (long)nkv * dh * kpad; at.v_hs = (long)dh * kpad; at.v_ds = kpad;
  at.B = B; at.Tq = Tq; at.n_heads = nh; at.heads_per_kv = nh / nkv; at.n_keys = nk; at.dh = dh;
  at.k_len = (long)B * nkv * nk * dh; at.v_len = (long)B * nkv * dh * kpad;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  attn_plan(at, elem, prop.multiProcessorCount);
  void *vt = nullptr, *ws = nullptr;
  hipError_t e = hipMalloc(&vt, (size_t)B * nkv * dh * kpad * esz);
  const size_t wsb = attn_ws_bytes(at);
  if (e == hipSuccess && wsb) e = hipMalloc(&ws, wsb);
  if (e == hipSuccess) e = hipMemsetAsync(vt, 0, (size_t)B * nkv * dh * kpad * esz, s);
  if (e == hipSuccess) e = prefix_v_copy_t(vt, (long)dh * kpad, kpad, v, B * nkv, nk, dh, elem, s);
  at.vt = vt; at.ws = (float*)ws;
  if (e == hipSuccess) e = attn_launch(at, elem, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (vt) (void)hipFree(vt);
  if (ws) (void)hipFree(ws);
  if (e != hipSuccess) { g_err = fmt("fm_op_attention: %s", hipGetErrorString(e)); return FM_ERR_DEVICE; }
  return FM_OK;
}


}  // extern "C"

// ---------------------------------------------------------------------------------------
// Attention without allocation: the transposed V plane and the split partials of
// fm_op_attention live in one file-scope device array (one copy per GPU, held until the process
// ends). Host code never passes the array's name to a kernel: its address on the current device
// comes from hipGetSymbolAddress, taken once per device on the first call there.
// ---------------------------------------------------------------------------------------

namespace {
constexpr size_t kNoAllocScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];
int g_scratch_cus[kNoAllocMaxDevices];

// this device's copy of `scratch` and its CU count (hipGetSymbolAddress with the device current)
hipError_t scratch_of_current_device(void** ptr, int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_cus[dev] = prop.multiProcessorCount;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *cus = g_scratch_cus[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

fm_status fm_op_attention_noalloc(int32_t dtype, int32_t B, int32_t Tq, int32_t nh, int32_t nkv, int32_t nk,
                                  int32_t dh, const void* q, const void* k, const void* v, void* o, void* stream) {
  const int elem = dtype == FM_BF16 ? ET_BF16 : ET_F32;
  if ((dtype != FM_F32 && dtype != FM_BF16) || B < 1 || Tq < 1 || nh < 1 || nk < 1 || (nkv != 1 && nkv != nh) ||
      !q || !k || !v || !o || (dh != 64 && dh != 128 && dh != 256) || (dtype == FM_F32 && dh == 256)) {
    g_err = "fm_op_attention_noalloc: bad arguments";
    return FM_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  void* base = nullptr;
  int cus = 0;
  hipError_t e = scratch_of_current_device(&base, &cus);
  if (e != hipSuccess) { g_err = fmt("fm_op_attention_noalloc: scratch address: %s", hipGetErrorString(e)); return FM_ERR_DEVICE; }
  const size_t esz = elem == ET_BF16 ? 2 : 4;
  const int kpad = (int)round_up(nk, 64);
  AttnArgs at;
  memset(&at, 0, sizeof at);
  at.q = q; at.q_bs = (long)Tq * nh * dh; at.q_rs = (long)nh * dh;
  at.k = k; at.k_bs = (long)nkv * nk * dh; at.k_rs = dh; at.k_hs = (long)nk * dh;
  at.o = o; at.o_bs = at.q_bs; at.o_rs = at.q_rs;
  at.v_bs = (long)nkv * dh * kpad; at.v_hs = (long)dh * kpad; at.v_ds = kpad;
  at.B = B; at.Tq = Tq; at.n_heads = nh; at.heads_per_kv = nh / nkv; at.n_keys = nk; at.dh = dh;
  at.k_len = (long)B * nkv * nk * dh; at.v_len = (long)B * nkv * dh * kpad;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  attn_plan(at, elem, cus);
  // scratch layout: the V plane, then (256-byte aligned) the split partials
  const size_t vt_bytes = (size_t)B * nkv * dh * kpad * esz;
  const size_t ws_off = (size_t)round_up((long)vt_bytes, 256);
  const size_t need = ws_off + attn_ws_bytes(at);
  if (need > kNoAllocScratchBytes) {
    g_err = fmt("fm_op_attention_noalloc: needs %zu bytes of scratch, more than its fixed %zu", need,
                kNoAllocScratchBytes);
    return FM_ERR_INVALID_ARG;
  }
  char* sc = (char*)base;
  at.vt = sc;
  at.ws = attn_ws_bytes(at) ? (float*)(sc + ws_off) : nullptr;
  // the plane's padding keys must read zero (a fill kernel: this call may be captured in a graph)
  e = fill_f32((float*)sc, 0.f, (long)(vt_bytes / 4), s);
  if (e == hipSuccess) e = prefix_v_copy_t(sc, (long)dh * kpad, kpad, v, B * nkv, nk, dh, elem, s);
  if (e == hipSuccess) e = attn_launch(at, elem, s);
  if (e != hipSuccess) { g_err = fmt("fm_op_attention_noalloc: %s", hipGetErrorString(e)); return FM_ERR_DEVICE; }
  return FM_OK;
}

}  // extern "C"
