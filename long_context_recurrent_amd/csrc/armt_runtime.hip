// Runtime and C ABI of libarmt.so (declared in include/armt.h).
//
// Scheduling follows the pages: node (s, l) needs (s, l-1) and (s-1, l), so
// wave i = {(s, l) : s + l = i} and the S x L grid runs as S + L - 1 waves
// (Pith review of arXiv 2506.05229, "What carries the argument", Lemma 3.1);
// each wave is one grouped launch per step over the active layers' stacked
// weights (skill page "Diagonal Batching for Recurrent Memory Transformers",
// Architecture Overview: one grouped kernel launch per diagonal), and the
// per-layer memory state stays on the GPU between waves with no host
// synchronisation (same page, Practical Guidance).  The sequential baseline
// (Pith review, Figure 3) runs the same kernels one node at a time.
//
// Buffers.  Node outputs (the residual stream, fp32 in every workload; bf16
// workloads store only branch activations in bf16) live in two slots
// act[c & 1][L][n][d] (c = wave
// index; node (s, l) of wave c reads layer l-1's row of slot (c-1) & 1 and
// writes layer l's row of slot c & 1, so the nodes of one wave never touch a
// buffer another node of that wave writes).  Per-layer scratch (normalised
// activations, QKV, V^T, attention output, SwiGLU product, memory-write keys)
// is indexed by layer, so a node computes at the same addresses in either
// schedule.  The caller's x and y pointers and the running wave counter sit in
// a small device descriptor, which lets one captured hipGraph per wave shape
// (first layer, last layer, slot parity) be replayed for every call and every
// wave of that shape.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <map>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/armt.h"
#include "armt_kernels.h"

using namespace armt;

namespace {

// Message of the last non-OK status of this thread (a fixed buffer: setting
// it never allocates).
thread_local char g_last_error[512];

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  memcpy(g_last_error, buf, sizeof(buf));
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ARMT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t desc, rope, A, z, act0, act1, abuf, qkv, vt, attn, ubuf, qbuf, kbuf, pden, beta, moff, A2, total;
};

int validate_config(const armt_config* c) {
  if (!c) return fail(ARMT_E_INVALID, "config is NULL");
  if (c->n_layers <= 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->ffn_hidden <= 0 || c->seg_len <= 0 || c->n_mem <= 0 || c->d_key <= 0)
    return fail(ARMT_E_INVALID, "every size in the config must be positive");
  if (c->dtype != ARMT_F32 && c->dtype != ARMT_BF16) return fail(ARMT_E_INVALID, "dtype must be ARMT_F32 or ARMT_BF16");
  if (c->d_model != c->n_heads * c->head_dim)
    return fail(ARMT_E_INVALID, "d_model (%d) must equal n_heads * head_dim (%d)", c->d_model, c->n_heads * c->head_dim);
  if (c->n_heads % c->n_kv_heads) return fail(ARMT_E_INVALID, "n_heads must be a multiple of n_kv_heads");
  if (!(c->rms_eps > 0.f) || !(c->mem_eps > 0.f) || !(c->rope_theta > 0.f))
    return fail(ARMT_E_INVALID, "rms_eps, mem_eps and rope_theta must be positive");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(ARMT_E_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (c->d_key != 64) return fail(ARMT_E_UNSUPPORTED, "d_key must be 64");
  if (c->d_model % 64 || c->ffn_hidden % 64) return fail(ARMT_E_UNSUPPORTED, "d_model and ffn_hidden must be multiples of 64");
  if (c->n_mem > 64) return fail(ARMT_E_UNSUPPORTED, "n_mem must be <= 64");
  const int n = c->seg_len + c->n_mem;
  if (c->dtype == ARMT_BF16) {
    if (n > 4096) return fail(ARMT_E_UNSUPPORTED, "seg_len + n_mem must be <= 4096");
    if (c->d_model > 3072 || c->d_model % 128)
      return fail(ARMT_E_UNSUPPORTED, "bf16: d_model must be a multiple of 128 and <= 3072");
  } else {
    if (n > 2048) return fail(ARMT_E_UNSUPPORTED, "fp32: seg_len + n_mem must be <= 2048");
    if (c->d_model > 1024) return fail(ARMT_E_UNSUPPORTED, "fp32: d_model must be <= 1024");
  }
  return ARMT_OK;
}

// Buffers with a slab per (layer, sequence) problem: L * batch slabs.
Layout make_layout(const armt_config* c, int batch) {
  const size_t L = (size_t)c->n_layers * batch, d = c->d_model, n = c->seg_len + c->n_mem;
  const size_t n_pad = (n + 63) / 64 * 64;
  const size_t es = c->dtype == ARMT_BF16 ? 2 : 4;
  const size_t qkv_dim = (size_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  const size_t hhd = (size_t)c->n_heads * c->head_dim;
  const size_t M = c->n_mem, dk = c->d_key, F = c->ffn_hidden;
  Layout lo{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
  lo.desc = take(sizeof(CallDesc));
  lo.rope = take(n * (c->head_dim / 2) * 2 * sizeof(float));
  lo.A = take(L * d * dk * 4);
  lo.z = take(L * dk * 4);
  lo.act0 = take(L * n * d * 4);   // residual stream: fp32 in every workload
  lo.act1 = take(L * n * d * 4);
  lo.abuf = take(L * n * d * es);
  lo.qkv = take(L * n * qkv_dim * es);
  lo.vt = take(c->dtype == ARMT_BF16 ? L * c->n_kv_heads * c->head_dim * n_pad * 2 : 0);
  lo.attn = take(L * n * hhd * es);
  lo.ubuf = take(L * n * F * es);
  lo.qbuf = take(c->dtype == ARMT_BF16 ? L * n * dk * 4 : 0);
  lo.kbuf = take(L * M * dk * 4);
  lo.pden = take(L * M * 4 * 4);
  lo.beta = take(L * M * 4);
  lo.moff = take(L * 4);
  lo.A2 = take(c->dtype == ARMT_BF16 ? L * d * dk * 4 : 0);   // A as bf16 hi / lo pairs
  lo.total = off;
  return lo;
}

// Full-attention comparator: the layer geometry of the config (seg_len, n_mem,
// d_key and mem_eps unused) over up to max_tokens positions.
int validate_llama(const armt_config* c, int64_t max_tokens) {
  if (!c) return fail(ARMT_E_INVALID, "config is NULL");
  if (c->n_layers <= 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn_hidden <= 0)
    return fail(ARMT_E_INVALID, "every layer size in the config must be positive");
  if (max_tokens < 1) return fail(ARMT_E_INVALID, "max_tokens must be >= 1");
  if (c->dtype != ARMT_F32 && c->dtype != ARMT_BF16) return fail(ARMT_E_INVALID, "dtype must be ARMT_F32 or ARMT_BF16");
  if (c->d_model != c->n_heads * c->head_dim)
    return fail(ARMT_E_INVALID, "d_model (%d) must equal n_heads * head_dim (%d)", c->d_model, c->n_heads * c->head_dim);
  if (c->n_heads % c->n_kv_heads) return fail(ARMT_E_INVALID, "n_heads must be a multiple of n_kv_heads");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(ARMT_E_INVALID, "rms_eps and rope_theta must be positive");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(ARMT_E_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (c->d_model % 64 || c->ffn_hidden % 64 || c->d_model > 4096)
    return fail(ARMT_E_UNSUPPORTED, "d_model and ffn_hidden must be multiples of 64, d_model <= 4096");
  if (c->dtype == ARMT_BF16 && max_tokens > (1 << 18)) return fail(ARMT_E_UNSUPPORTED, "bf16: max_tokens must be <= 262144");
  // the bf16 attention addresses one sequence's keys with 32-bit offsets
  const int64_t qkv_bytes = (int64_t)max_tokens * (c->n_heads + 2 * c->n_kv_heads) * c->head_dim * 2;
  if (c->dtype == ARMT_BF16 && qkv_bytes > INT32_MAX)
    return fail(ARMT_E_UNSUPPORTED, "bf16: max_tokens * (n_heads + 2 n_kv_heads) * head_dim * 2 must be < 2^31");
  if (c->dtype == ARMT_F32 && max_tokens > 4096) return fail(ARMT_E_UNSUPPORTED, "fp32: max_tokens must be <= 4096");
  return ARMT_OK;
}

// One slab per buffer (the comparator runs one layer at a time over all
// positions): residual stream fp32 [N][d] in act0, then the same scratch as a
// node of the recurrent model with n = N.
Layout make_llama_layout(const armt_config* c, int64_t N) {
  const size_t d = c->d_model, n = (size_t)N, n_pad = (n + 63) / 64 * 64;
  const size_t es = c->dtype == ARMT_BF16 ? 2 : 4;
  const size_t qkv_dim = (size_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  const size_t hhd = (size_t)c->n_heads * c->head_dim, F = c->ffn_hidden;
  Layout lo{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
  lo.desc = take(sizeof(CallDesc));
  lo.rope = take(n * (c->head_dim / 2) * 2 * sizeof(float));
  lo.A = take(0);
  lo.z = take(0);
  lo.act0 = take(n * d * 4);
  lo.act1 = take(0);
  lo.abuf = take(n * d * es);
  lo.qkv = take(n * qkv_dim * es);
  lo.vt = take(c->dtype == ARMT_BF16 ? c->n_kv_heads * c->head_dim * n_pad * 2 : 0);
  lo.attn = take(n * hhd * es);
  lo.ubuf = take(n * F * es);
  lo.qbuf = take(0);
  lo.kbuf = take(0);
  lo.pden = take(0);
  lo.beta = take(0);
  lo.moff = take(0);
  lo.total = off;
  return lo;
}

enum Sched { SCHED_DIAG = 0, SCHED_SEQ = 1 };

}  // namespace

struct armt_handle {
  armt_config cfg;
  armt_weights w;
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  int device = 0;
  bool bf16 = true;
  int n = 0, n_pad = 0, qkv_dim = 0, mb = 0, cus = 256;   // mb 0: per-launch choice
  int batch = 1;            // sequences per node
  bool llama = false;       // full-attention comparator handle (armt_llama_create)
  int64_t norm_rows = 0;    // rows of the normalised-activation buffer
  size_t es = 2;
  char* ws = nullptr;
  Layout lo{};
  CallDesc* desc = nullptr;
  float* rope = nullptr;
  float* A = nullptr;
  float* z = nullptr;
  armt::bf16* A2 = nullptr;   // bf16 workloads: A split into hi / lo parts for the memory read
  void* act[2] = {nullptr, nullptr};
  void *abuf = nullptr, *qkv = nullptr, *vt = nullptr, *attn = nullptr, *ubuf = nullptr;
  float *qbuf = nullptr, *kbuf = nullptr, *pden = nullptr, *beta = nullptr;
  int* moff = nullptr;
  std::map<std::tuple<int, int, int, int, int>, hipGraphExec_t> graphs;
  bool use_graphs = true;
  bool debug_sync = false;    // sync + error check after every kernel of a forward
  int last_kernel = -1;       // kernel id of the last launch (for error messages)
  int time_kernel = -1;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t events_used = 0;
  int64_t t_launches = 0;
  double t_flops = 0, t_bytes = 0;
};

namespace {

// Algorithmic FLOPs and minimum HBM bytes of kernel k for one node.
void node_cost(const armt_handle* h, int k, double* flops, double* bytes) {
  const armt_config& c = h->cfg;
  const double n = h->n, d = c.d_model, F = c.ffn_hidden, dk = c.d_key, M = c.n_mem;
  const double H = c.n_heads, hd = c.head_dim, q = h->qkv_dim, es = (double)h->es;
  const double tri = n * (n + 1) / 2;
  double f = 0, b = 0;
  switch (k) {
    // the residual stream h (read and written by the memory read, read by the
    // norms, updated by the residual epilogues, read by the memory write) is fp32
    // bf16: the attention norm is fused into the memory read
    case ARMT_K_MEM_READ:
      f = 4 * n * d * dk;
      b = 2 * n * d * 4 + dk * d * es + d * dk * 4 + (h->bf16 ? (n * d + d) * es : 0);
      break;
    case ARMT_K_ATTN_NORM: f = 0; b = h->bf16 ? 0 : n * d * 4 + (n * d + d) * es; break;
    case ARMT_K_QKV: f = 2 * n * d * q; b = (n * d + q * d + n * q) * es; break;
    case ARMT_K_ATTN: f = 4 * tri * hd * H; b = (n * q + n * H * hd) * es; break;
    case ARMT_K_OPROJ: f = 2 * n * H * hd * d; b = (n * H * hd + d * H * hd) * es + 2 * n * d * 4; break;
    case ARMT_K_MLP_NORM: f = 0; b = n * d * 4 + (n * d + d) * es; break;
    case ARMT_K_GATE_UP: f = 4 * n * d * F; b = (n * d + 2 * F * d + n * F) * es; break;
    case ARMT_K_DOWN: f = 2 * n * F * d; b = (n * F + d * F) * es + 2 * n * d * 4; break;
    case ARMT_K_MEM_KEYS: f = 2 * M * d * (dk + 1); b = M * d * 4 + (dk * d + d) * es; break;
    case ARMT_K_MEM_UPDATE: f = 2 * M * d * d + 4 * M * dk * d; b = M * d * 4 + d * d * es + 2 * d * dk * 4; break;
  }
  *flops = f;
  *bytes = b;
}

int pick_row_blocks(int n, int n_cols, int cols_per_tile, int K, int P, int cus);

int gemm_rows(const armt_handle* h, int n_cols, int cols_per_tile, int K, int P) {
  return h->mb ? h->mb : pick_row_blocks(h->n, n_cols, cols_per_tile, K, P * h->batch, h->cus);
}

struct StepCtx {
  armt_handle* h;
  hipStream_t st;
  bool timing;
  bool check = false;   // synchronise and check for errors after every launch
};

hipError_t timed(StepCtx& cx, int kid, int P, hipError_t (*fn)(const void*, hipStream_t), const void* arg) {
  armt_handle* h = cx.h;
  const bool t = cx.timing && h->time_kernel == kid;
  if (t) {
    if (h->events_used == h->events.size()) {
      hipEvent_t a, b;
      hipError_t e = hipEventCreate(&a);
      if (e != hipSuccess) return e;
      e = hipEventCreate(&b);
      if (e != hipSuccess) return e;
      h->events.push_back({a, b});
    }
    hipError_t e = hipEventRecord(h->events[h->events_used].first, cx.st);
    if (e != hipSuccess) return e;
  }
  h->last_kernel = kid;
  hipError_t e = fn(arg, cx.st);
  if (e != hipSuccess) return e;
  if (cx.check) {
    if ((e = hipStreamSynchronize(cx.st)) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (t) {
    e = hipEventRecord(h->events[h->events_used].second, cx.st);
    if (e != hipSuccess) return e;
    h->events_used++;
    double f, b;
    node_cost(h, kid, &f, &b);
    h->t_launches++;
    h->t_flops += f * P;
    h->t_bytes += b * P;
  }
  return hipSuccess;
}

struct GemmCall { const armt_handle* h; GemmArgs g; int epi; int mb; };
struct AttnCall { const armt_handle* h; AttnArgs a; };
struct MemCall { const armt_handle* h; MemArgs m; int which; };

hipError_t run_gemm(const void* p, hipStream_t st) {
  const GemmCall* c = (const GemmCall*)p;
  return c->h->bf16 ? launch_gemm_bf16(c->g, c->epi, c->mb, st) : launch_gemm_f32(c->g, c->epi, st);
}
hipError_t run_attn(const void* p, hipStream_t st) {
  const AttnCall* c = (const AttnCall*)p;
  return launch_attention(c->a, c->h->bf16, st);
}
hipError_t run_mem(const void* p, hipStream_t st) {
  const MemCall* c = (const MemCall*)p;
  switch (c->which) {
    case ARMT_K_MEM_READ: return launch_mem_read(c->m, c->h->bf16, st);
    case ARMT_K_ATTN_NORM:
    case ARMT_K_MLP_NORM: return launch_rmsnorm(c->m, c->h->bf16, st);
    case ARMT_K_MEM_KEYS: return launch_mem_keys(c->m, c->h->bf16, st);
    default: return launch_mem_update(c->m, c->h->bf16, st);
  }
}

// Enqueue the kernels of one step: layers l_lo..l_hi of slot parity par.
hipError_t enqueue_step(StepCtx& cx, int l_lo, int l_hi, int par, int advance) {
  armt_handle* h = cx.h;
  const armt_config& c = h->cfg;
  const int P = l_hi - l_lo + 1, B = h->batch;
  const int d = c.d_model, n = h->n, F = c.ffn_hidden, hhd = c.n_heads * c.head_dim;
  const int64_t nd = (int64_t)n * d;
  const size_t es = h->es;

  // memory kernels and attention: one problem per (layer, sequence); GEMMs:
  // P layers x B sequences
  MemArgs m{};
  m.P = P * B; m.l0 = l_lo * B; m.batch = B;
  m.n = n; m.d = d; m.T = c.seg_len; m.M = c.n_mem; m.dk = c.d_key; m.L = c.n_layers;
  m.act_prev = h->act[par ^ 1]; m.act_cur = h->act[par]; m.abuf = h->abuf; m.act_stride = nd;
  m.mem_emb = h->w.mem_emb; m.w_mq = h->w.w_mq; m.w_mk = h->w.w_mk; m.w_mv = h->w.w_mv; m.w_beta = h->w.w_beta;
  m.A = h->A; m.A2 = h->A2; m.z = h->z; m.qbuf = h->qbuf; m.kbuf = h->kbuf; m.pden = h->pden; m.beta = h->beta; m.desc = h->desc;
  m.moff = h->moff;
  m.mem_eps = c.mem_eps; m.rms_eps = c.rms_eps; m.advance = 0;

  GemmArgs g0{};
  g0.P = P; g0.l0 = l_lo; g0.batch = B; g0.M = n; g0.T = c.seg_len; g0.last_layer = c.n_layers - 1;
  g0.head_dim = c.head_dim;

  hipError_t e;
  // 1. memory read, then the attention norm (one fused kernel for bf16)
  {
    MemCall mc{h, m, ARMT_K_MEM_READ};
    mc.m.gain = h->w.g_attn;
    if ((e = timed(cx, ARMT_K_MEM_READ, P * B, run_mem, &mc)) != hipSuccess) return e;
    if (!h->bf16) {
      MemCall nc{h, m, ARMT_K_ATTN_NORM};
      nc.m.gain = h->w.g_attn;
      if ((e = timed(cx, ARMT_K_ATTN_NORM, P * B, run_mem, &nc)) != hipSuccess) return e;
    }
  }
  // 2. QKV projection with RoPE
  {
    GemmCall gc{h, g0, EPI_QKV, gemm_rows(h, h->qkv_dim, 256, d, P)};
    GemmArgs& g = gc.g;
    g.A = h->abuf; g.a_stride = nd; g.lda = d;
    g.B = h->w.w_qkv; g.b_stride = (int64_t)h->qkv_dim * d; g.N = h->qkv_dim; g.K = d;
    g.C = h->qkv; g.c_stride = (int64_t)n * h->qkv_dim; g.ldc = h->qkv_dim;
    g.rope_cs = h->rope; g.rope_cols = (c.n_heads + c.n_kv_heads) * c.head_dim;
    g.v_col0 = g.rope_cols; g.vt = h->vt; g.vt_ld = h->n_pad;
    g.vt_stride = (int64_t)c.n_kv_heads * c.head_dim * h->n_pad;
    if ((e = timed(cx, ARMT_K_QKV, P * B, run_gemm, &gc)) != hipSuccess) return e;
  }
  // 3. attention
  {
    AttnCall ac{h, {}};
    AttnArgs& a = ac.a;
    a.P = P * B; a.l0 = l_lo * B; a.qkv = h->qkv; a.qkv_stride = (int64_t)n * h->qkv_dim; a.ld_qkv = h->qkv_dim;
    a.vt = h->vt; a.vt_stride = (int64_t)c.n_kv_heads * c.head_dim * h->n_pad; a.vt_ld = h->n_pad;
    a.out = h->attn; a.out_stride = (int64_t)n * hhd; a.ld_out = hhd;
    a.n = n; a.H = c.n_heads; a.G = c.n_kv_heads; a.hd = c.head_dim;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    if ((e = timed(cx, ARMT_K_ATTN, P * B, run_attn, &ac)) != hipSuccess) return e;
  }
  // 4. output projection + residual
  {
    GemmCall gc{h, g0, EPI_RESID, gemm_rows(h, d, 256, hhd, P)};
    GemmArgs& g = gc.g;
    g.A = h->attn; g.a_stride = (int64_t)n * hhd; g.lda = hhd;
    g.B = h->w.w_o; g.b_stride = (int64_t)d * hhd; g.N = d; g.K = hhd;
    g.C = h->act[par]; g.c_stride = nd; g.ldc = d; g.desc = nullptr;
    if ((e = timed(cx, ARMT_K_OPROJ, P * B, run_gemm, &gc)) != hipSuccess) return e;
  }
  // 5. MLP norm
  {
    MemCall mc{h, m, ARMT_K_MLP_NORM};
    mc.m.gain = h->w.g_mlp;
    if ((e = timed(cx, ARMT_K_MLP_NORM, P * B, run_mem, &mc)) != hipSuccess) return e;
  }
  // 6. gate/up + SiLU product
  {
    GemmCall gc{h, g0, EPI_SWIGLU, gemm_rows(h, F, 128, d, P)};
    GemmArgs& g = gc.g;
    g.A = h->abuf; g.a_stride = nd; g.lda = d;
    g.B = h->w.w_gate; g.B2 = h->w.w_up; g.b_stride = (int64_t)F * d; g.N = F; g.K = d;
    g.C = h->ubuf; g.c_stride = (int64_t)n * F; g.ldc = F;
    if ((e = timed(cx, ARMT_K_GATE_UP, P * B, run_gemm, &gc)) != hipSuccess) return e;
  }
  // 7. down projection + residual (+ y rows of the last layer)
  {
    GemmCall gc{h, g0, EPI_RESID, gemm_rows(h, d, 256, F, P)};
    GemmArgs& g = gc.g;
    g.A = h->ubuf; g.a_stride = (int64_t)n * F; g.lda = F;
    g.B = h->w.w_down; g.b_stride = (int64_t)d * F; g.N = d; g.K = F;
    g.C = h->act[par]; g.c_stride = nd; g.ldc = d; g.desc = h->desc;
    if ((e = timed(cx, ARMT_K_DOWN, P * B, run_gemm, &gc)) != hipSuccess) return e;
  }
  // 8-9. memory write
  {
    MemCall mc{h, m, ARMT_K_MEM_KEYS};
    if ((e = timed(cx, ARMT_K_MEM_KEYS, P * B, run_mem, &mc)) != hipSuccess) return e;
    MemCall mu{h, m, ARMT_K_MEM_UPDATE};
    mu.m.advance = advance;
    if ((e = timed(cx, ARMT_K_MEM_UPDATE, P * B, run_mem, &mu)) != hipSuccess) return e;
  }
  (void)es;
  return hipSuccess;
}

// Full-attention comparator: the L Llama-shaped blocks over all N positions
// as one causal window, one layer at a time (no memory read or write).  The
// same kernels as a recurrent node with n = N and one problem per launch;
// activation slabs have stride 0, so every layer reuses the one set of
// buffers, and the fp32 residual stream is updated in place.
hipError_t enqueue_llama(StepCtx& cx, const void* x, int N, void* y) {
  armt_handle* h = cx.h;
  const armt_config& c = h->cfg;
  const int L = c.n_layers, d = c.d_model, F = c.ffn_hidden, hhd = c.n_heads * c.head_dim;
  hipError_t e;
  // the descriptor points the last layer's down projection at y (segment 0)
  if ((e = launch_set_desc(h->desc, x, y, L - 1, 1, N, N, cx.st)) != hipSuccess) return e;
  if ((e = launch_widen(x, (float*)h->act[0], (int64_t)N * d, h->bf16, cx.st)) != hipSuccess) return e;
  auto rows = [&](int n_cols, int cols_per_tile, int K) {
    return h->mb ? h->mb : pick_row_blocks(N, n_cols, cols_per_tile, K, 1, h->cus);
  };
  for (int l = 0; l < L; ++l) {
    MemArgs m{};
    m.P = 1; m.l0 = l; m.batch = 1; m.n = N; m.d = d; m.T = N; m.L = L;
    m.act_cur = h->act[0]; m.act_prev = h->act[0]; m.abuf = h->abuf; m.act_stride = 0;
    m.rms_eps = c.rms_eps;
    GemmArgs g0{};
    g0.P = 1; g0.l0 = l; g0.batch = 1; g0.M = N; g0.T = N; g0.last_layer = L - 1; g0.head_dim = c.head_dim;
    // attention block
    m.gain = h->w.g_attn;
    if ((e = launch_rmsnorm(m, h->bf16, cx.st)) != hipSuccess) return e;
    {
      GemmArgs g = g0;
      g.A = h->abuf; g.a_stride = 0; g.lda = d;
      g.B = h->w.w_qkv; g.b_stride = (int64_t)h->qkv_dim * d; g.N = h->qkv_dim; g.K = d;
      g.C = h->qkv; g.c_stride = 0; g.ldc = h->qkv_dim;
      g.rope_cs = h->rope; g.rope_cols = (c.n_heads + c.n_kv_heads) * c.head_dim;
      g.v_col0 = g.rope_cols; g.vt = h->vt; g.vt_ld = h->n_pad; g.vt_stride = 0;
      e = h->bf16 ? launch_gemm_bf16(g, EPI_QKV, rows(h->qkv_dim, 256, d), cx.st) : launch_gemm_f32(g, EPI_QKV, cx.st);
      if (e != hipSuccess) return e;
    }
    {
      AttnArgs a{};
      a.P = 1; a.l0 = l; a.qkv = h->qkv; a.qkv_stride = 0; a.ld_qkv = h->qkv_dim;
      a.vt = h->vt; a.vt_stride = 0; a.vt_ld = h->n_pad;
      a.out = h->attn; a.out_stride = 0; a.ld_out = hhd;
      a.n = N; a.H = c.n_heads; a.G = c.n_kv_heads; a.hd = c.head_dim;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      if ((e = launch_attention(a, h->bf16, cx.st)) != hipSuccess) return e;
    }
    {
      GemmArgs g = g0;
      g.A = h->attn; g.a_stride = 0; g.lda = hhd;
      g.B = h->w.w_o; g.b_stride = (int64_t)d * hhd; g.N = d; g.K = hhd;
      g.C = h->act[0]; g.c_stride = 0; g.ldc = d; g.desc = nullptr;
      e = h->bf16 ? launch_gemm_bf16(g, EPI_RESID, rows(d, 256, hhd), cx.st) : launch_gemm_f32(g, EPI_RESID, cx.st);
      if (e != hipSuccess) return e;
    }
    // MLP block
    m.gain = h->w.g_mlp;
    if ((e = launch_rmsnorm(m, h->bf16, cx.st)) != hipSuccess) return e;
    {
      GemmArgs g = g0;
      g.A = h->abuf; g.a_stride = 0; g.lda = d;
      g.B = h->w.w_gate; g.B2 = h->w.w_up; g.b_stride = (int64_t)F * d; g.N = F; g.K = d;
      g.C = h->ubuf; g.c_stride = 0; g.ldc = F;
      e = h->bf16 ? launch_gemm_bf16(g, EPI_SWIGLU, rows(F, 128, d), cx.st) : launch_gemm_f32(g, EPI_SWIGLU, cx.st);
      if (e != hipSuccess) return e;
    }
    {
      GemmArgs g = g0;
      g.A = h->ubuf; g.a_stride = 0; g.lda = F;
      g.B = h->w.w_down; g.b_stride = (int64_t)d * F; g.N = d; g.K = F;
      g.C = h->act[0]; g.c_stride = 0; g.ldc = d; g.desc = h->desc;
      e = h->bf16 ? launch_gemm_bf16(g, EPI_RESID, rows(d, 256, F), cx.st) : launch_gemm_f32(g, EPI_RESID, cx.st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

int run_step(armt_handle* h, int sched, int l_lo, int l_hi, int par, int advance) {
  const bool timing = h->time_kernel >= 0;
  if (!h->use_graphs || timing || h->debug_sync) {
    StepCtx cx{h, h->stream, timing, h->debug_sync};
    h->last_kernel = -1;
    hipError_t e = enqueue_step(cx, l_lo, l_hi, par, advance);
    if (e == hipSuccess) return ARMT_OK;
    if (h->debug_sync && h->last_kernel >= 0)
      return fail(ARMT_E_HIP, "HIP error in kernel %d of the wave of layers %d..%d: %s", h->last_kernel, l_lo,
                  l_hi, hipGetErrorString(e));
    return hip_fail(e, "kernel launch");
  }
  auto key = std::make_tuple(sched, l_lo, l_hi, par, advance);
  auto it = h->graphs.find(key);
  if (it == h->graphs.end()) {
    hipError_t e = hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
    StepCtx cx{h, h->cap_stream, false};
    hipError_t le = enqueue_step(cx, l_lo, l_hi, par, advance);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(h->cap_stream, &graph);
    if (le != hipSuccess) {
      if (graph) hipGraphDestroy(graph);
      return hip_fail(le, "kernel launch during capture");
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
    it = h->graphs.emplace(key, exec).first;
  }
  hipError_t e = hipGraphLaunch(it->second, h->stream);
  return e == hipSuccess ? ARMT_OK : hip_fail(e, "hipGraphLaunch");
}

// S segments, the last one t_last (1..T) tokens long.
int forward(armt_handle* h, int sched, const void* x, int32_t S, int32_t t_last, const float* A0,
            const float* z0, void* y, float* A_out, float* z_out) {
  if (!h) return fail(ARMT_E_INVALID, "handle is NULL");
  if (h->llama) return fail(ARMT_E_INVALID, "handle is a full-attention comparator: use armt_llama_forward");
  if (!x || !y || !A_out || !z_out) return fail(ARMT_E_INVALID, "x, y, A_out and z_out must not be NULL");
  if (S < 1) return fail(ARMT_E_INVALID, "n_segments must be >= 1 (got %d)", S);
  const armt_config& c = h->cfg;
  const int L = c.n_layers;
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  const int64_t a_count = (int64_t)L * h->batch * c.d_model * c.d_key, z_count = (int64_t)L * h->batch * c.d_key;
  const int64_t seq_rows = (int64_t)(S - 1) * c.seg_len + t_last;
  if ((e = launch_set_desc(h->desc, x, y, 0, S, t_last, seq_rows, h->stream)) != hipSuccess)
    return hip_fail(e, "set_desc");
  if ((e = launch_fill_f32(h->A, A0, a_count, h->stream)) != hipSuccess) return hip_fail(e, "state init");
  if ((e = launch_fill_f32(h->z, z0, z_count, h->stream)) != hipSuccess) return hip_fail(e, "state init");
  if (h->bf16 && (e = launch_split_state(h->A, h->A2, a_count / c.d_key, h->stream)) != hipSuccess)
    return hip_fail(e, "state init");
  int rc;
  if (sched == SCHED_DIAG) {
    for (int w = 0; w < S + L - 1; ++w) {
      const int l_lo = w - S + 1 > 0 ? w - S + 1 : 0;
      const int l_hi = w < L - 1 ? w : L - 1;
      if ((rc = run_step(h, SCHED_DIAG, l_lo, l_hi, w & 1, 1)) != ARMT_OK) return rc;
    }
  } else {
    for (int s = 0; s < S; ++s)
      for (int l = 0; l < L; ++l) {
        // counter = s + l; after the last layer move to (s + 1) + 0
        const int adv = (l == L - 1) ? 2 - L : 1;
        if ((rc = run_step(h, SCHED_SEQ, l, l, (s + l) & 1, adv)) != ARMT_OK) return rc;
      }
  }
  if ((e = hipMemcpyAsync(A_out, h->A, a_count * 4, hipMemcpyDeviceToDevice, h->stream)) != hipSuccess)
    return hip_fail(e, "copy A_out");
  if ((e = hipMemcpyAsync(z_out, h->z, z_count * 4, hipMemcpyDeviceToDevice, h->stream)) != hipSuccess)
    return hip_fail(e, "copy z_out");
  return ARMT_OK;
}

// 16-row blocks per GEMM tile for one grouped launch of P problems with
// n_cols output columns per problem (cols_per_tile per workgroup).  Every
// tile height gives bitwise identical results, so the choice is free: it
// minimises rounds x (tile rows + a fixed per-tile cost), where a round is
// one workgroup on every compute unit (the tiles hold one workgroup per CU).
// Tiles shorter than 128 rows are not considered: their operand traffic per
// FLOP is too high.
int pick_row_blocks(int n, int n_cols, int cols_per_tile, int K, int P, int cus) {
  constexpr int kLongK = 4096;
  // Tile heights are 16-row blocks.  Cost = rounds of workgroups over the
  // CUs x (tile rows + a fixed per-tile overhead in rows: pipeline fill and
  // epilogue).  Heights of 16 * (4j + 3) rows measured slower on long-K
  // products than the next height up (1B down projection, K = 8192: 176-row
  // tiles 3.4% slower than 192-row tiles over 8.3% fewer rows), so those
  // do not use them.
  constexpr int kTileOverheadRows = 48;
  int best = 12;
  long best_cost = -1;
  for (int i = 0; i < kGemmRowBlocksCount; ++i) {
    const int rb = kGemmRowBlocks[i], bm = 16 * rb;
    if (bm < 128) continue;
    if (K >= kLongK && rb % 4 == 3) continue;
    const long tiles = (long)((n + bm - 1) / bm) * ((n_cols + cols_per_tile - 1) / cols_per_tile) * P;
    const long rounds = (tiles + cus - 1) / cus;
    const long cost = rounds * (bm + kTileOverheadRows);
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && rb > best)) {
      best = rb;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

extern "C" {

int armt_workspace_size_batched(const armt_config* cfg, int32_t batch, size_t* bytes) {
  int rc = validate_config(cfg);
  if (rc != ARMT_OK) return rc;
  if (batch < 1 || batch > 1024) return fail(ARMT_E_INVALID, "batch must be in 1..1024 (got %d)", batch);
  if (!bytes) return fail(ARMT_E_INVALID, "bytes is NULL");
  *bytes = make_layout(cfg, batch).total;
  return ARMT_OK;
}

int armt_workspace_size(const armt_config* cfg, size_t* bytes) { return armt_workspace_size_batched(cfg, 1, bytes); }

}  // extern "C"

namespace {

// Common part of the two create calls: carve the workspace, upload the RoPE
// table for positions 0..n-1 and zero the V^T padding.  Takes ownership of h
// (deleted on failure).
// Handle fields for a workspace at `workspace` laid out as `lo` (no
// allocation, no device work).
void set_fields(armt_handle* h, const armt_config* cfg, const armt_weights* w, const Layout& lo,
                void* workspace, void* hip_stream, int n) {
  h->cfg = *cfg;
  h->w = *w;
  h->stream = (hipStream_t)hip_stream;
  h->bf16 = cfg->dtype == ARMT_BF16;
  h->es = h->bf16 ? 2 : 4;
  h->n = n;
  h->n_pad = (h->n + 63) / 64 * 64;
  h->qkv_dim = (cfg->n_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
  h->mb = 0;
  h->lo = lo;
  char* base = (char*)workspace;
  h->ws = base;
  h->desc = (CallDesc*)(base + lo.desc);
  h->rope = (float*)(base + lo.rope);
  h->A = (float*)(base + lo.A);
  h->z = (float*)(base + lo.z);
  h->A2 = (armt::bf16*)(base + lo.A2);
  h->act[0] = base + lo.act0;
  h->act[1] = base + lo.act1;
  h->abuf = base + lo.abuf;
  h->qkv = base + lo.qkv;
  h->vt = base + lo.vt;
  h->attn = base + lo.attn;
  h->ubuf = base + lo.ubuf;
  h->qbuf = (float*)(base + lo.qbuf);
  h->kbuf = (float*)(base + lo.kbuf);
  h->pden = (float*)(base + lo.pden);
  h->beta = (float*)(base + lo.beta);
  h->moff = (int*)(base + lo.moff);
}

int init_handle(armt_handle* h, const armt_config* cfg, const armt_weights* w, const Layout& lo,
                void* workspace, void* hip_stream, int n, armt_handle** out) {
  set_fields(h, cfg, w, lo, workspace, hip_stream, n);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { delete h; return hip_fail(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess || h->cus <= 0) { delete h; return hip_fail(e, "hipDeviceGetAttribute"); }
  e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) { delete h; return hip_fail(e, "hipStreamCreateWithFlags"); }

  // RoPE table: angle = pos * theta^(-2i/hd), computed in double on the host
  const int half = cfg->head_dim / 2;
  std::vector<float> tab((size_t)h->n * half * 2);
  for (int p = 0; p < h->n; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = p * std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      tab[((size_t)p * half + i) * 2] = (float)std::cos(ang);
      tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  e = hipMemcpy(h->rope, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice);
  // V^T padding columns (keys n .. n_pad-1) must read as zeros; nothing else
  // ever writes them
  if (e == hipSuccess && h->bf16) e = hipMemset(h->vt, 0, lo.attn - lo.vt);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    hipStreamDestroy(h->cap_stream);
    delete h;
    return hip_fail(e, "workspace initialisation");
  }
  *out = h;
  return ARMT_OK;
}

int check_workspace(const Layout& lo, void* workspace, size_t ws_bytes) {
  if (!workspace) return fail(ARMT_E_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(ARMT_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < lo.total)
    return fail(ARMT_E_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, lo.total);
  return ARMT_OK;
}

}  // namespace

extern "C" {

int armt_create(const armt_config* cfg, const armt_weights* w, void* workspace, size_t ws_bytes,
                void* hip_stream, armt_handle** out) {
  return armt_create_batched(cfg, w, 1, workspace, ws_bytes, hip_stream, out);
}

int armt_create_batched(const armt_config* cfg, const armt_weights* w, int32_t batch, void* workspace,
                        size_t ws_bytes, void* hip_stream, armt_handle** out) {
  int rc = validate_config(cfg);
  if (rc != ARMT_OK) return rc;
  if (batch < 1 || batch > 1024) return fail(ARMT_E_INVALID, "batch must be in 1..1024 (got %d)", batch);
  if (!w || !out) return fail(ARMT_E_INVALID, "weights and out must not be NULL");
  const void* ptrs[] = {w->w_qkv, w->w_o, w->w_gate, w->w_up, w->w_down, w->g_attn,
                        w->g_mlp, w->w_mq, w->w_mk, w->w_mv, w->w_beta, w->mem_emb};
  for (const void* p : ptrs)
    if (!p) return fail(ARMT_E_INVALID, "every weight pointer must be non-NULL");
  const Layout lo = make_layout(cfg, batch);
  if ((rc = check_workspace(lo, workspace, ws_bytes)) != ARMT_OK) return rc;
  armt_handle* h = new (std::nothrow) armt_handle();
  if (!h) return fail(ARMT_E_INVALID, "out of host memory");
  h->batch = batch;
  h->norm_rows = (int64_t)cfg->n_layers * batch * (cfg->seg_len + cfg->n_mem);
  return init_handle(h, cfg, w, lo, workspace, hip_stream, cfg->seg_len + cfg->n_mem, out);
}

int armt_llama_workspace_size(const armt_config* cfg, int64_t max_tokens, size_t* bytes) {
  int rc = validate_llama(cfg, max_tokens);
  if (rc != ARMT_OK) return rc;
  if (!bytes) return fail(ARMT_E_INVALID, "bytes is NULL");
  *bytes = make_llama_layout(cfg, max_tokens).total;
  return ARMT_OK;
}

int armt_llama_create(const armt_config* cfg, const armt_weights* w, int64_t max_tokens, void* workspace,
                      size_t ws_bytes, void* hip_stream, armt_handle** out) {
  int rc = validate_llama(cfg, max_tokens);
  if (rc != ARMT_OK) return rc;
  if (!w || !out) return fail(ARMT_E_INVALID, "weights and out must not be NULL");
  const void* ptrs[] = {w->w_qkv, w->w_o, w->w_gate, w->w_up, w->w_down, w->g_attn, w->g_mlp};
  for (const void* p : ptrs)
    if (!p) return fail(ARMT_E_INVALID, "the block weights (w_qkv .. g_mlp) must be non-NULL");
  const Layout lo = make_llama_layout(cfg, max_tokens);
  if ((rc = check_workspace(lo, workspace, ws_bytes)) != ARMT_OK) return rc;
  armt_handle* h = new (std::nothrow) armt_handle();
  if (!h) return fail(ARMT_E_INVALID, "out of host memory");
  h->llama = true;
  h->norm_rows = max_tokens;
  return init_handle(h, cfg, w, lo, workspace, hip_stream, (int)max_tokens, out);
}

int armt_llama_forward(armt_handle* h, const void* x, int64_t n_tokens, void* y) {
  if (!h) return fail(ARMT_E_INVALID, "handle is NULL");
  if (!h->llama) return fail(ARMT_E_INVALID, "handle is not a full-attention comparator (armt_llama_create)");
  if (!x || !y) return fail(ARMT_E_INVALID, "x and y must not be NULL");
  if (n_tokens < 1 || n_tokens > h->n)
    return fail(ARMT_E_INVALID, "n_tokens must be in 1..%d (got %lld)", h->n, (long long)n_tokens);
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  StepCtx cx{h, h->stream, false};
  e = enqueue_llama(cx, x, (int)n_tokens, y);
  return e == hipSuccess ? ARMT_OK : hip_fail(e, "kernel launch");
}

int armt_forward_sequential(armt_handle* h, const void* x, int32_t n_segments, const float* A0,
                            const float* z0, void* y, float* A_out, float* z_out) {
  return forward(h, SCHED_SEQ, x, n_segments, h ? h->cfg.seg_len : 0, A0, z0, y, A_out, z_out);
}

int armt_forward_diagonal(armt_handle* h, const void* x, int32_t n_segments, const float* A0,
                          const float* z0, void* y, float* A_out, float* z_out) {
  return forward(h, SCHED_DIAG, x, n_segments, h ? h->cfg.seg_len : 0, A0, z0, y, A_out, z_out);
}

static int forward_tokens(armt_handle* h, int sched, const void* x, int64_t n_tokens, const float* A0,
                          const float* z0, void* y, float* A_out, float* z_out) {
  if (!h) return fail(ARMT_E_INVALID, "handle is NULL");
  const int64_t T = h->cfg.seg_len;
  if (n_tokens < 1) return fail(ARMT_E_INVALID, "n_tokens must be >= 1 (got %lld)", (long long)n_tokens);
  const int64_t S = (n_tokens + T - 1) / T;
  if (S > (1 << 30)) return fail(ARMT_E_INVALID, "too many segments");
  return forward(h, sched, x, (int32_t)S, (int32_t)(n_tokens - (S - 1) * T), A0, z0, y, A_out, z_out);
}

int armt_forward_sequential_tokens(armt_handle* h, const void* x, int64_t n_tokens, const float* A0,
                                   const float* z0, void* y, float* A_out, float* z_out) {
  return forward_tokens(h, SCHED_SEQ, x, n_tokens, A0, z0, y, A_out, z_out);
}

int armt_forward_diagonal_tokens(armt_handle* h, const void* x, int64_t n_tokens, const float* A0,
                                 const float* z0, void* y, float* A_out, float* z_out) {
  return forward_tokens(h, SCHED_DIAG, x, n_tokens, A0, z0, y, A_out, z_out);
}

int armt_logits(armt_handle* h, const void* y, int64_t rows, const void* g_final, const void* w_lm,
                int32_t vocab, float* logits) {
  if (!h) return fail(ARMT_E_INVALID, "handle is NULL");
  if (!y || !g_final || !w_lm || !logits) return fail(ARMT_E_INVALID, "y, g_final, w_lm and logits must not be NULL");
  if (rows < 1 || vocab < 1) return fail(ARMT_E_INVALID, "rows and vocab must be positive");
  if (h->bf16 && vocab % 8) return fail(ARMT_E_UNSUPPORTED, "bf16: vocab must be a multiple of 8 (got %d)", vocab);
  const armt_config& c = h->cfg;
  const int d = c.d_model;
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  // normalised rows go through the workspace's normalised-activation buffer
  // (L * n rows of a recurrent-model handle, max_tokens of a comparator), a
  // chunk at a time
  const int64_t chunk = h->norm_rows;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int m = (int)(rows - r0 < chunk ? rows - r0 : chunk);
    NormArgs na{};
    na.x = (const char*)y + r0 * d * (int64_t)h->es;
    na.gain = g_final;
    na.out = h->abuf;
    na.rows = m;
    na.d = d;
    na.eps = c.rms_eps;
    if ((e = launch_final_norm(na, h->bf16, h->stream)) != hipSuccess) return hip_fail(e, "final norm launch");
    GemmArgs g{};
    g.P = 1; g.l0 = 0; g.batch = 1;
    g.A = h->abuf; g.a_stride = 0; g.lda = d;
    g.B = w_lm; g.b_stride = 0;
    g.M = m; g.N = vocab; g.K = d;
    g.C = logits + r0 * vocab; g.c_stride = 0; g.ldc = vocab;
    e = h->bf16 ? launch_gemm_bf16(g, EPI_STORE, h->mb ? h->mb : pick_row_blocks(m, vocab, 256, d, 1, h->cus), h->stream)
                : launch_gemm_f32(g, EPI_STORE, h->stream);
    if (e != hipSuccess) return hip_fail(e, "LM-head GEMM launch");
  }
  return ARMT_OK;
}

void armt_destroy(armt_handle* h) {
  if (!h) return;
  hipSetDevice(h->device);
  for (auto& kv : h->graphs) hipGraphExecDestroy(kv.second);
  for (auto& ev : h->events) {
    hipEventDestroy(ev.first);
    hipEventDestroy(ev.second);
  }
  if (h->cap_stream) hipStreamDestroy(h->cap_stream);
  delete h;
}

const char* armt_last_error(void) { return g_last_error; }

int armt_wave_schedule(int32_t n_layers, int32_t n_segments, int32_t* l_lo, int32_t* l_hi, int32_t cap,
                       int32_t* n_waves) {
  if (n_layers <= 0 || n_segments <= 0) return fail(ARMT_E_INVALID, "n_layers and n_segments must be positive");
  if (!l_lo || !l_hi || !n_waves) return fail(ARMT_E_INVALID, "output arrays must not be NULL");
  const int nw = n_layers + n_segments - 1;
  if (cap < nw) return fail(ARMT_E_INVALID, "capacity %d < %d waves", cap, nw);
  for (int w = 0; w < nw; ++w) {
    l_lo[w] = w - n_segments + 1 > 0 ? w - n_segments + 1 : 0;
    l_hi[w] = w < n_layers - 1 ? w : n_layers - 1;
  }
  *n_waves = nw;
  return ARMT_OK;
}

int armt_set_option(armt_handle* h, int32_t option, int32_t value) {
  if (!h) return fail(ARMT_E_INVALID, "handle is NULL");
  switch (option) {
    case ARMT_OPT_GRAPHS: h->use_graphs = value != 0; return ARMT_OK;
    case ARMT_OPT_DEBUG_SYNC:
      if (value != 0 && value != 1) return fail(ARMT_E_INVALID, "debug sync must be 0 or 1 (got %d)", value);
      h->debug_sync = value != 0;
      return ARMT_OK;
    case ARMT_OPT_TIME_KERNEL:
      if (value < -1 || value >= ARMT_K_COUNT) return fail(ARMT_E_INVALID, "kernel id %d out of range", value);
      h->time_kernel = value;
      h->events_used = 0;
      h->t_launches = 0;
      h->t_flops = h->t_bytes = 0;
      return ARMT_OK;
    case ARMT_OPT_GEMM_ROWS: {
      bool ok = value == 0;
      for (int i = 0; i < kGemmRowBlocksCount; ++i) ok = ok || kGemmRowBlocks[i] == value;
      if (!ok || !h->bf16) return fail(ARMT_E_INVALID, "unsupported GEMM row blocks %d", value);
      h->mb = value;
      for (auto& kv : h->graphs) hipGraphExecDestroy(kv.second);
      h->graphs.clear();
      return ARMT_OK;
    }
    default: return fail(ARMT_E_INVALID, "unknown option %d", option);
  }
}

int armt_kernel_stats(armt_handle* h, double* ms, int64_t* launches, double* flops, double* bytes) {
  if (!h || !ms || !launches || !flops || !bytes) return fail(ARMT_E_INVALID, "NULL argument");
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  double total = 0;
  for (size_t i = 0; i < h->events_used; ++i) {
    float t = 0;
    e = hipEventElapsedTime(&t, h->events[i].first, h->events[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    total += t;
  }
  *ms = total;
  *launches = h->t_launches;
  *flops = h->t_flops;
  *bytes = h->t_bytes;
  return ARMT_OK;
}

int armt_debug_view(armt_handle* h, int32_t which, void** ptr, size_t* bytes) {
  if (!h || !ptr || !bytes) return fail(ARMT_E_INVALID, "NULL argument");
  const Layout& lo = h->lo;
  size_t at, end;
  switch (which) {
    case ARMT_VIEW_ACT0: at = lo.act0; end = lo.act1; break;
    case ARMT_VIEW_ACT1: at = lo.act1; end = lo.abuf; break;
    case ARMT_VIEW_NORMED: at = lo.abuf; end = lo.qkv; break;
    case ARMT_VIEW_QKV: at = lo.qkv; end = lo.vt; break;
    case ARMT_VIEW_VT: at = lo.vt; end = lo.attn; break;
    case ARMT_VIEW_ATTN: at = lo.attn; end = lo.ubuf; break;
    case ARMT_VIEW_SWIGLU: at = lo.ubuf; end = lo.qbuf; break;
    case ARMT_VIEW_A: at = lo.A; end = lo.z; break;
    case ARMT_VIEW_Z: at = lo.z; end = lo.act0; break;
    default: return fail(ARMT_E_INVALID, "unknown view %d", which);
  }
  *ptr = h->ws + at;
  *bytes = end - at;
  return ARMT_OK;
}

}  // extern "C"

// ===========================================================================
// Backward pass (fp32 handles): the vector-Jacobian product of the forward
// over the diagonal waves in reverse order (or segment-major in reverse for
// the sequential schedule).  A forward pass first records each node's input
// rows and the state it read into a tape; every node's activations are then
// recomputed from the tape before its backward.
// ===========================================================================
namespace {

struct BwLayout {
  size_t tape_h, tape_A, tape_z;
  size_t u, q, dq, den, r1, r2, dden;
  size_t num, h1, a, h2, b, h3, dh, da, db, dnum;
  size_t qkv, dqkv, O, dO, mx, ls, Dq;
  size_t G, Up, Uo, dG, dUp, dUo;
  size_t uk, k, dk, v, kA, e, de, dv, dkA, bl, beta, denw, ddenw, dbl;
  size_t dH, dA, dz, yscr, g32, a16, O16, b16, U16, ta, tb, wtd, wtgu, wto, wtq, ysp, total;
};

BwLayout make_bw_layout(const armt_config* c, int S) {
  const size_t L = c->n_layers, d = c->d_model, n = c->seg_len + c->n_mem, M = c->n_mem, F = c->ffn_hidden;
  const size_t qd = (size_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim, H = c->n_heads;
  BwLayout lo{};
  size_t off = 0;
  auto take = [&](size_t floats) { size_t at = off; off = align_up(off + floats * 4); return at; };
  lo.tape_h = take(L * S * n * d);
  lo.tape_A = take(L * S * d * 64);
  lo.tape_z = take(L * S * 64);
  lo.u = take(L * n * 64); lo.q = take(L * n * 64); lo.dq = take(L * n * 64);
  lo.den = take(L * n); lo.r1 = take(L * n); lo.r2 = take(L * n); lo.dden = take(L * n);
  lo.num = take(L * n * d); lo.h1 = take(L * n * d); lo.a = take(L * n * d); lo.h2 = take(L * n * d);
  lo.b = take(L * n * d); lo.h3 = take(L * n * d); lo.dh = take(L * n * d); lo.da = take(L * n * d);
  lo.db = take(L * n * d); lo.dnum = take(L * n * d);
  lo.qkv = take(L * n * qd); lo.dqkv = take(L * n * qd);
  lo.O = take(L * n * H * c->head_dim); lo.dO = take(L * n * H * c->head_dim);
  lo.mx = take(L * H * n); lo.ls = take(L * H * n); lo.Dq = take(L * H * n);
  lo.G = take(L * n * F); lo.Up = take(L * n * F); lo.Uo = take(L * n * F);
  lo.dG = take(L * n * F); lo.dUp = take(L * n * F); lo.dUo = take(L * n * F);
  lo.uk = take(L * M * 64); lo.k = take(L * M * 64); lo.dk = take(L * M * 64);
  lo.v = take(L * M * d); lo.kA = take(L * M * d); lo.e = take(L * M * d);
  lo.de = take(L * M * d); lo.dv = take(L * M * d); lo.dkA = take(L * M * d);
  lo.bl = take(L * M); lo.beta = take(L * M); lo.denw = take(L * M); lo.ddenw = take(L * M); lo.dbl = take(L * M);
  lo.dH = take(2 * L * n * d);
  lo.dA = take(L * d * 64);
  lo.dz = take(L * 64);
  lo.yscr = take((size_t)S * c->seg_len * d);   // the recording forward's y (not returned)
  lo.g32 = take(3 * L * d);                      // fp32 g_attn, g_mlp, w_beta of a bf16 model
  // bf16 copies of the recomputed a, O, b, Uo (bf16 models)
  lo.a16 = take(L * n * d / 2 + 1); lo.O16 = take(L * n * H * c->head_dim / 2 + 1);
  lo.b16 = take(L * n * d / 2 + 1); lo.U16 = take(L * n * F / 2 + 1);
  // transposed bf16 operands of the weight gradients (bf16 models): rows of
  // the node padded to a multiple of 64 with zeros
  {
    const size_t n_pad = (n + 63) / 64 * 64;
    size_t cmax = d > F ? d : F;
    cmax = cmax > qd ? cmax : qd;
    cmax = cmax > H * (size_t)c->head_dim ? cmax : H * (size_t)c->head_dim;
    lo.ta = take(L * cmax * n_pad); lo.tb = take(L * cmax * n_pad);   // [cols][2 n_pad] bf16
  }
  // input gradients of the block products (bf16 models): the transposed
  // weights, each twice along k, [W_d^T | W_d^T], [W_g^T | W_g^T | W_u^T |
  // W_u^T], [W_o^T | W_o^T], [W_qkv^T | W_qkv^T]; and the gradients as bf16
  // pairs, [n][hi | lo]
  {
    const size_t hd = H * (size_t)c->head_dim;
    lo.wtd = take(L * F * 2 * d / 2); lo.wtgu = take(L * d * 4 * F / 2);
    lo.wto = take(L * hd * 2 * d / 2); lo.wtq = take(L * d * 2 * qd / 2);
    size_t cmax = 4 * F > 2 * qd ? 4 * F : 2 * qd;
    cmax = cmax > 2 * d ? cmax : 2 * d;
    lo.ysp = take(L * n * cmax / 2);
  }
  lo.total = off;
  return lo;
}

struct BwCtx {
  armt_handle* h;
  hipStream_t st;
  int S;
  char* ws;
  BwLayout lo;
  const armt_weights* gw;   // gradient buffers (fp32, weight shapes)
  const float *g_attn, *g_mlp, *w_beta;   // fp32 views of the gains and the gate vector
  float* f(size_t at) const { return (float*)(ws + at); }
};

// C = (acc ? C : 0) + A B over P problems
// (strides in elements; B is bf16 when b16 is set)
hipError_t gg(const float* A, int64_t a_ps, int64_t a_rs, int64_t a_cs, const void* B, int64_t b_ps, int64_t b_rs,
              int64_t b_cs, float* C, int64_t c_ps, int64_t c_rs, int64_t c_cs, int M, int N, int K, int acc, int P,
              hipStream_t st, int b16 = 0, int matrix_cores = 0) {
  GenGemm g{A, B, C, a_ps, a_rs, a_cs, b_ps, b_rs, b_cs, c_ps, c_rs, c_cs, M, N, K, acc, b16};
  return launch_gemm_gen(g, P, matrix_cores != 0, st);
}

#define BW_TRY(x)                              \
  do {                                         \
    hipError_t _e = (x);                       \
    if (_e != hipSuccess) return _e;           \
  } while (0)

// Backward of the nodes (c - l, l) for l = l0 .. l0 + P - 1 (wave c).
hipError_t backward_wave(BwCtx& cx, int c, int l0, int P, const void* dy, float* dx) {
  armt_handle* h = cx.h;
  const armt_config& cf = h->cfg;
  const int L = cf.n_layers, S = cx.S, d = cf.d_model, n = h->n, M = cf.n_mem, T = cf.seg_len, F = cf.ffn_hidden;
  const int H = cf.n_heads, G = cf.n_kv_heads, hd = cf.head_dim, qd = h->qkv_dim, hhd = H * hd;
  const int64_t nd = (int64_t)n * d, n64 = (int64_t)n * 64, nq = (int64_t)n * qd, nF = (int64_t)n * F;
  const int64_t Md = (int64_t)M * d, M64 = (int64_t)M * 64, D64 = (int64_t)d * 64;
  hipStream_t st = cx.st;
  BwArgs ba{};
  ba.d = d; ba.n = n; ba.M = M; ba.hd = hd; ba.H = H; ba.G = G; ba.qkv_ld = qd; ba.row_ps = n;
  ba.mem_eps = cf.mem_eps; ba.rms_eps = cf.rms_eps; ba.scale = 1.0f / std::sqrt((float)hd); ba.rope = h->rope;
  // per-layer slab pointers, offset to layer l0
  auto S1 = [&](size_t at, int64_t per) { return cx.f(at) + (int64_t)l0 * per; };
  const int64_t tap = (int64_t)l0 * S + (c - l0);       // tape index of problem 0; problem p adds p (S - 1)
  const float* hin = cx.f(cx.lo.tape_h) + tap * nd;
  const float* Ast = cx.f(cx.lo.tape_A) + tap * D64;
  const float* zst = cx.f(cx.lo.tape_z) + tap * 64;
  const int64_t hin_ps = (int64_t)(S - 1) * nd, A_ps = (int64_t)(S - 1) * D64, z_ps = (int64_t)(S - 1) * 64;
  // weight matrices in the model's dtype (bf16 ones are widened exactly as
  // the products load them); gains and the gate vector as fp32 views
  const int wb = h->bf16 ? 1 : 0;
  auto wp = [&](const void* base, int64_t elems) { return (const void*)((const char*)base + elems * (wb ? 2 : 4)); };
  const void* W_mq = wp(h->w.w_mq, (int64_t)l0 * 64 * d);
  const void* W_qkv = wp(h->w.w_qkv, (int64_t)l0 * qd * d);
  const void* W_o = wp(h->w.w_o, (int64_t)l0 * d * hhd);
  const void* W_g = wp(h->w.w_gate, (int64_t)l0 * F * d);
  const void* W_u = wp(h->w.w_up, (int64_t)l0 * F * d);
  const void* W_d = wp(h->w.w_down, (int64_t)l0 * d * F);
  const void* W_mk = wp(h->w.w_mk, (int64_t)l0 * 64 * d);
  const void* W_mv = wp(h->w.w_mv, (int64_t)l0 * d * d);
  const float* w_b = cx.w_beta + (int64_t)l0 * d;
  const float* g_at = cx.g_attn + (int64_t)l0 * d;
  const float* g_ml = cx.g_mlp + (int64_t)l0 * d;
  float* dW_mq = (float*)cx.gw->w_mq + (int64_t)l0 * 64 * d;
  float* dW_qkv = (float*)cx.gw->w_qkv + (int64_t)l0 * qd * d;
  float* dW_o = (float*)cx.gw->w_o + (int64_t)l0 * d * hhd;
  float* dW_g = (float*)cx.gw->w_gate + (int64_t)l0 * F * d;
  float* dW_u = (float*)cx.gw->w_up + (int64_t)l0 * F * d;
  float* dW_d = (float*)cx.gw->w_down + (int64_t)l0 * d * F;
  float* dW_mk = (float*)cx.gw->w_mk + (int64_t)l0 * 64 * d;
  float* dW_mv = (float*)cx.gw->w_mv + (int64_t)l0 * d * d;
  float* dw_b = (float*)cx.gw->w_beta + (int64_t)l0 * d;
  float* dg_at = (float*)cx.gw->g_attn + (int64_t)l0 * d;
  float* dg_ml = (float*)cx.gw->g_mlp + (int64_t)l0 * d;
  float *u = S1(cx.lo.u, n64), *q = S1(cx.lo.q, n64), *dq = S1(cx.lo.dq, n64);
  float *den = S1(cx.lo.den, n), *r1 = S1(cx.lo.r1, n), *r2 = S1(cx.lo.r2, n), *dden = S1(cx.lo.dden, n);
  float *num = S1(cx.lo.num, nd), *h1 = S1(cx.lo.h1, nd), *a = S1(cx.lo.a, nd), *h2 = S1(cx.lo.h2, nd);
  float *b = S1(cx.lo.b, nd), *h3 = S1(cx.lo.h3, nd), *dh = S1(cx.lo.dh, nd), *da = S1(cx.lo.da, nd);
  float *db = S1(cx.lo.db, nd), *dnum = S1(cx.lo.dnum, nd);
  float *qkv = S1(cx.lo.qkv, nq), *dqkv = S1(cx.lo.dqkv, nq), *O = S1(cx.lo.O, nd), *dO = S1(cx.lo.dO, nd);
  const int64_t Hn = (int64_t)H * n;
  float *mx = S1(cx.lo.mx, Hn), *ls = S1(cx.lo.ls, Hn), *Dq = S1(cx.lo.Dq, Hn);
  float *Gt = S1(cx.lo.G, nF), *Up = S1(cx.lo.Up, nF), *Uo = S1(cx.lo.Uo, nF);
  float *dG = S1(cx.lo.dG, nF), *dUp = S1(cx.lo.dUp, nF), *dUo = S1(cx.lo.dUo, nF);
  float *uk = S1(cx.lo.uk, M64), *kk = S1(cx.lo.k, M64), *dk = S1(cx.lo.dk, M64);
  float *v = S1(cx.lo.v, Md), *kA = S1(cx.lo.kA, Md), *e = S1(cx.lo.e, Md), *de = S1(cx.lo.de, Md);
  float *dv = S1(cx.lo.dv, Md), *dkA = S1(cx.lo.dkA, Md);
  float *bl = S1(cx.lo.bl, M), *beta = S1(cx.lo.beta, M), *denw = S1(cx.lo.denw, M), *ddenw = S1(cx.lo.ddenw, M);
  float* dbl = S1(cx.lo.dbl, M);
  float* dA = S1(cx.lo.dA, D64);
  float* dz = S1(cx.lo.dz, 64);

  // ---- upstream gradient of each node's output into dh
  const int l_hi = l0 + P - 1;
  const int Pn = (l_hi == L - 1) ? P - 1 : P;   // problems fed by the layer above
  float* dH_in = cx.f(cx.lo.dH) + (int64_t)((c + 1) & 1) * L * nd;
  if (Pn > 0) BW_TRY(bw_copy(dH_in + (int64_t)(l0 + 1) * nd, dh, nd, nd, nd, 0, Pn, st));
  if (l_hi == L - 1) {
    float* top = dh + (int64_t)(P - 1) * nd;
    const int s = c - (L - 1);
    if (wb) BW_TRY(launch_widen((const bf16*)dy + (int64_t)s * T * d, top, (int64_t)T * d, true, st));
    else BW_TRY(bw_copy((const float*)dy + (int64_t)s * T * d, top, (int64_t)T * d, 0, 0, 0, 1, st));
    BW_TRY(hipMemsetAsync(top + (int64_t)T * d, 0, (size_t)M * d * 4, st));
  }

  // bf16 models: the activations that the bf16 forward rounds before a
  // product (the attention and MLP inputs a and b, the attention output O,
  // the SwiGLU output Uo) are kept rounded in bf16 slabs; the recomputed
  // products that take them as inputs run on the forward's own grouped GEMM
  // (fp32 store, or += on the residual), and the weight gradients take them
  // as bf16 operands.  Every other fp32 operand of a matrix-core product
  // enters as a hi/lo pair.
  bf16* const a16 = (bf16*)(cx.ws + cx.lo.a16);
  bf16* const O16 = (bf16*)(cx.ws + cx.lo.O16);
  bf16* const b16 = (bf16*)(cx.ws + cx.lo.b16);
  bf16* const U16 = (bf16*)(cx.ws + cx.lo.U16);
  const int64_t nh = (int64_t)n * hhd;
  // C (fp32 slab, layer-indexed) = or += A16 W^T over the wave's layers
  auto fwd_gemm = [&](const bf16* A16, int64_t a_ps, int K, const void* W, float* C, int64_t c_ps, int N,
                      int epi) -> hipError_t {
    GemmArgs g{};
    g.P = P; g.l0 = l0; g.batch = 1;
    g.A = A16; g.a_stride = a_ps; g.lda = K;
    g.B = W; g.b_stride = (int64_t)N * K;
    g.M = n; g.N = N; g.K = K;
    g.C = C; g.c_stride = c_ps; g.ldc = N;
    g.desc = nullptr; g.last_layer = L - 1; g.T = T;
    return launch_gemm_bf16(g, epi, gemm_rows(h, N, 256, K, P), st);
  };
  const int64_t Lo = (int64_t)l0;   // slab offsets of layer l0
  // dX (fp32, layer-indexed slab) = dY W on the forward's grouped GEMM: the
  // bf16 value of dY (the hi half of the per-layer scratch ysp, [n][hi | lo])
  // against the transposed weights (the first half of wt, [in][W^T | W^T]);
  // the gradient enters the product rounded once to bf16
  bf16* const ysp = (bf16*)(cx.ws + cx.lo.ysp);
  auto dx_gemm = [&](int Kx, const bf16* wt, float* C, int64_t c_ps, int N) -> hipError_t {
    GemmArgs g{};
    g.P = P; g.l0 = l0; g.batch = 1;
    g.A = ysp; g.a_stride = (int64_t)n * Kx; g.lda = Kx;
    g.B = wt; g.b_stride = (int64_t)N * Kx; g.ldb = Kx;
    g.M = n; g.N = N; g.K = Kx / 2;
    g.C = C; g.c_stride = c_ps; g.ldc = N;
    g.desc = nullptr; g.last_layer = L - 1; g.T = T;
    return launch_gemm_bf16(g, EPI_STORE, gemm_rows(h, N, 256, Kx, P), st);
  };
  // dW (fp32, [L][out][in], layer-indexed) += dY^T X on the forward's grouped
  // GEMM, in one pass over dW: K runs over the node's rows with the bf16 value
  // of dY against X (dY^T -> the first half of [out][2 n_pad], X^T -> the
  // first half of [in][2 n_pad], n_pad rows with zeros past the node)
  const int n_pad = (n + 63) / 64 * 64;
  bf16* const ta = (bf16*)(cx.ws + cx.lo.ta);
  bf16* const tb = (bf16*)(cx.ws + cx.lo.tb);
  auto dw_gemm = [&](const float* dY, int64_t y_ps, int out, const bf16* X16, int64_t x_ps, int in,
                     const void* dW) -> hipError_t {
    const int k2 = 2 * n_pad;
    const int64_t sa = (int64_t)out * k2, sb = (int64_t)in * k2;
    bf16* a0 = ta + Lo * sa;
    bf16* b0 = tb + Lo * sb;
    hipError_t e = bw_transpose_bf16(dY, false, out, y_ps, n, n_pad, out, a0, nullptr, k2, sa, P, st);
    if (e != hipSuccess) return e;
    if ((e = bw_transpose_bf16(X16, true, in, x_ps, n, n_pad, in, b0, nullptr, k2, sb, P, st)) != hipSuccess)
      return e;
    GemmArgs g{};
    g.P = P; g.l0 = l0; g.batch = 1;
    g.A = ta; g.a_stride = sa; g.lda = k2;
    g.B = tb; g.b_stride = sb; g.ldb = k2;
    g.M = out; g.N = in; g.K = n_pad;
    g.C = const_cast<void*>(dW); g.c_stride = (int64_t)out * in; g.ldc = in;   // caller's gradient buffer
    g.desc = nullptr; g.last_layer = L - 1; g.T = T;
    return launch_gemm_bf16(g, EPI_RESID, h->mb ? h->mb : pick_row_blocks(out, in, 256, n_pad, P, h->cus), st);
  };

  // ---- recompute the forward of each node
  BW_TRY(gg(hin, hin_ps, d, 1, W_mq, 64 * (int64_t)d, 1, d, u, n64, 64, 1, n, 64, d, 0, P, st, wb, wb));
  BW_TRY(bw_phi_den(ba, u, q, den, zst, n64, z_ps, n, P, st));
  BW_TRY(gg(q, n64, 64, 1, Ast, A_ps, 1, 64, num, nd, d, 1, n, d, 64, 0, P, st, 0, wb));
  BW_TRY(bw_copy(hin, h1, nd, hin_ps, nd, 0, P, st));
  BW_TRY(bw_add_div(ba, h1, num, den, h1, nd, n, P, st));
  BW_TRY(bw_rms_fwd(ba, h1, g_at, a, r1, nd, d, n, P, st));
  if (wb) {
    BW_TRY(bw_to_bf16(a, a16 + Lo * nd, nd, nd, P, st));
    BW_TRY(fwd_gemm(a16, nd, d, h->w.w_qkv, cx.f(cx.lo.qkv), nq, qd, EPI_STORE));
  } else {
    BW_TRY(gg(a, nd, d, 1, W_qkv, (int64_t)qd * d, 1, d, qkv, nq, qd, 1, n, qd, d, 0, P, st));
  }
  BW_TRY(bw_rope(ba, qkv, nq, qd, 0, H, 1.f, n, P, st));
  BW_TRY(bw_rope(ba, qkv, nq, qd, H * hd, G, 1.f, n, P, st));
  // bf16 models: attention on the matrix cores (bf16 operands), as their
  // forward computes it; fp32 models: the fp32 kernels
  const bool attn_mm = wb && bw_attn_mfma_ok(ba);
  if (attn_mm) BW_TRY(bw_attn_mfma_fwd(ba, qkv, O, mx, ls, nq, nd, Hn, P, st));
  else BW_TRY(bw_attn_fwd(ba, qkv, O, mx, ls, nq, nd, Hn, P, st));
  BW_TRY(bw_copy(h1, h2, nd, nd, nd, 0, P, st));
  if (wb) {
    BW_TRY(bw_to_bf16(O, O16 + Lo * nh, nh, nh, P, st));
    BW_TRY(fwd_gemm(O16, nh, hhd, h->w.w_o, cx.f(cx.lo.h2), nd, d, EPI_RESID));
  } else {
    BW_TRY(gg(O, nd, hhd, 1, W_o, (int64_t)d * hhd, 1, hhd, h2, nd, d, 1, n, d, hhd, 1, P, st));
  }
  BW_TRY(bw_rms_fwd(ba, h2, g_ml, b, r2, nd, d, n, P, st));
  if (wb) {
    BW_TRY(bw_to_bf16(b, b16 + Lo * nd, nd, nd, P, st));
    BW_TRY(fwd_gemm(b16, nd, d, h->w.w_gate, cx.f(cx.lo.G), nF, F, EPI_STORE));
    BW_TRY(fwd_gemm(b16, nd, d, h->w.w_up, cx.f(cx.lo.Up), nF, F, EPI_STORE));
  } else {
    BW_TRY(gg(b, nd, d, 1, W_g, (int64_t)F * d, 1, d, Gt, nF, F, 1, n, F, d, 0, P, st));
    BW_TRY(gg(b, nd, d, 1, W_u, (int64_t)F * d, 1, d, Up, nF, F, 1, n, F, d, 0, P, st));
  }
  BW_TRY(bw_swiglu(Gt, Up, Uo, nF, nF, P, st));
  BW_TRY(bw_copy(h2, h3, nd, nd, nd, 0, P, st));
  if (wb) {
    BW_TRY(bw_to_bf16(Uo, U16 + Lo * nF, nF, nF, P, st));
    BW_TRY(fwd_gemm(U16, nF, F, h->w.w_down, cx.f(cx.lo.h3), nd, d, EPI_RESID));
  } else {
    BW_TRY(gg(Uo, nF, F, 1, W_d, (int64_t)d * F, 1, F, h3, nd, d, 1, n, d, F, 1, P, st));
  }
  const float* Y = h3 + (int64_t)T * d;
  BW_TRY(gg(Y, nd, d, 1, W_mk, 64 * (int64_t)d, 1, d, uk, M64, 64, 1, M, 64, d, 0, P, st, wb, wb));
  BW_TRY(gg(Y, nd, d, 1, W_mv, (int64_t)d * d, 1, d, v, Md, d, 1, M, d, d, 0, P, st, wb, wb));
  BW_TRY(gg(Y, nd, d, 1, w_b, d, 1, 0, bl, M, 1, 0, M, 1, d, 0, P, st, 0, wb));
  BwArgs bm = ba;
  bm.row_ps = M;
  BW_TRY(bw_phi_den(bm, uk, kk, denw, zst, M64, z_ps, M, P, st));
  BW_TRY(gg(kk, M64, 64, 1, Ast, A_ps, 1, 64, kA, Md, d, 1, M, d, 64, 0, P, st, 0, wb));
  BW_TRY(bw_memw_fwd(ba, uk, kk, bl, beta, zst, denw, kA, v, e, z_ps, P, st));

  // ---- memory write backward (dA, dz hold the gradient of the state it wrote)
  BW_TRY(gg(kk, M64, 64, 1, dA, D64, 1, 64, de, Md, d, 1, M, d, 64, 0, P, st, 0, wb));
  BW_TRY(gg(e, Md, d, 1, dA, D64, 64, 1, dk, M64, 64, 1, M, 64, d, 0, P, st, 0, wb));
  BW_TRY(bw_memw_bwd(ba, de, v, kA, beta, denw, dv, dkA, ddenw, dbl, P, st));
  BW_TRY(gg(dkA, Md, 1, d, kk, M64, 64, 1, dA, D64, 64, 1, d, 64, M, 1, P, st, 0, wb));
  BW_TRY(gg(dkA, Md, d, 1, Ast, A_ps, 64, 1, dk, M64, 64, 1, M, 64, d, 1, P, st, 0, wb));
  BW_TRY(bw_memw_dk(ba, dk, uk, kk, ddenw, zst, dz, z_ps, 64, P, st));
  float* dY = dh + (int64_t)T * d;
  BW_TRY(gg(dk, M64, 64, 1, W_mk, 64 * (int64_t)d, d, 1, dY, nd, d, 1, M, d, 64, 1, P, st, wb, wb));
  BW_TRY(gg(dv, Md, d, 1, W_mv, (int64_t)d * d, d, 1, dY, nd, d, 1, M, d, d, 1, P, st, wb, wb));
  BW_TRY(bw_memw_beta(ba, dbl, w_b, Y, dY, dw_b, nd, d, P, st));
  BW_TRY(gg(dk, M64, 1, 64, Y, nd, d, 1, dW_mk, 64 * (int64_t)d, d, 1, 64, d, M, 1, P, st, 0, wb));
  BW_TRY(gg(dv, Md, 1, d, Y, nd, d, 1, dW_mv, (int64_t)d * d, d, 1, d, d, M, 1, P, st, 0, wb));
  // ---- MLP block backward
  if (wb) {
    BW_TRY(bw_split_bf16(dh, d, nd, n, d, ysp + Lo * n * 2 * d, 2 * d, (int64_t)n * 2 * d, d, P, st));
    BW_TRY(dx_gemm(2 * d, (const bf16*)(cx.ws + cx.lo.wtd), cx.f(cx.lo.dUo), nF, F));
  } else {
    BW_TRY(gg(dh, nd, d, 1, W_d, (int64_t)d * F, F, 1, dUo, nF, F, 1, n, F, d, 0, P, st));
  }
  if (wb) BW_TRY(dw_gemm(dh, nd, d, U16 + Lo * nF, nF, F, cx.gw->w_down));
  else BW_TRY(gg(dh, nd, 1, d, Uo, nF, F, 1, dW_d, (int64_t)d * F, F, 1, d, F, n, 1, P, st));
  BW_TRY(bw_swiglu_bwd(Gt, Up, dUo, dG, dUp, nF, nF, P, st));
  if (wb) {
    // db = dG W_g + dUp W_u as one product: [dG | dUp] (bf16 values, the hi
    // halves of [dG_hi | dUp_hi | dG_lo | dUp_lo]) against [W_g^T | W_u^T]
    bf16* y0 = ysp + Lo * n * 4 * F;
    BW_TRY(bw_split_bf16(dG, F, nF, n, F, y0, 4 * F, (int64_t)n * 4 * F, 2 * F, P, st));
    BW_TRY(bw_split_bf16(dUp, F, nF, n, F, y0 + F, 4 * F, (int64_t)n * 4 * F, 2 * F, P, st));
    BW_TRY(dx_gemm(4 * F, (const bf16*)(cx.ws + cx.lo.wtgu), cx.f(cx.lo.db), nd, d));
  } else {
    BW_TRY(gg(dG, nF, F, 1, W_g, (int64_t)F * d, d, 1, db, nd, d, 1, n, d, F, 0, P, st));
    BW_TRY(gg(dUp, nF, F, 1, W_u, (int64_t)F * d, d, 1, db, nd, d, 1, n, d, F, 1, P, st));
  }
  if (wb) {
    BW_TRY(dw_gemm(dG, nF, F, b16 + Lo * nd, nd, d, cx.gw->w_gate));
    BW_TRY(dw_gemm(dUp, nF, F, b16 + Lo * nd, nd, d, cx.gw->w_up));
  } else {
    BW_TRY(gg(dG, nF, 1, F, b, nd, d, 1, dW_g, (int64_t)F * d, d, 1, F, d, n, 1, P, st));
    BW_TRY(gg(dUp, nF, 1, F, b, nd, d, 1, dW_u, (int64_t)F * d, d, 1, F, d, n, 1, P, st));
  }
  BW_TRY(bw_rms_bwd(ba, h2, g_ml, r2, db, dh, dg_ml, nd, d, n, 1, P, st));
  // ---- attention block backward
  if (wb) {
    BW_TRY(bw_split_bf16(dh, d, nd, n, d, ysp + Lo * n * 2 * d, 2 * d, (int64_t)n * 2 * d, d, P, st));
    BW_TRY(dx_gemm(2 * d, (const bf16*)(cx.ws + cx.lo.wto), cx.f(cx.lo.dO), nd, hhd));
  } else {
    BW_TRY(gg(dh, nd, d, 1, W_o, (int64_t)d * hhd, hhd, 1, dO, nd, hhd, 1, n, hhd, d, 0, P, st));
  }
  if (wb) BW_TRY(dw_gemm(dh, nd, d, O16 + Lo * nh, nh, hhd, cx.gw->w_o));
  else BW_TRY(gg(dh, nd, 1, d, O, nd, hhd, 1, dW_o, (int64_t)d * hhd, hhd, 1, d, hhd, n, 1, P, st));
  if (attn_mm) BW_TRY(bw_attn_mfma_bwd(ba, qkv, O, dO, mx, ls, Dq, dqkv, nq, nd, Hn, P, st));
  else BW_TRY(bw_attn_bwd(ba, qkv, O, dO, mx, ls, Dq, dqkv, nq, nd, Hn, P, st));
  BW_TRY(bw_rope(ba, dqkv, nq, qd, 0, H, -1.f, n, P, st));
  BW_TRY(bw_rope(ba, dqkv, nq, qd, H * hd, G, -1.f, n, P, st));
  if (wb) {
    BW_TRY(bw_split_bf16(dqkv, qd, nq, n, qd, ysp + Lo * n * 2 * qd, 2 * qd, (int64_t)n * 2 * qd, qd, P, st));
    BW_TRY(dx_gemm(2 * qd, (const bf16*)(cx.ws + cx.lo.wtq), cx.f(cx.lo.da), nd, d));
  } else {
    BW_TRY(gg(dqkv, nq, qd, 1, W_qkv, (int64_t)qd * d, d, 1, da, nd, d, 1, n, d, qd, 0, P, st));
  }
  if (wb) BW_TRY(dw_gemm(dqkv, nq, qd, a16 + Lo * nd, nd, d, cx.gw->w_qkv));
  else BW_TRY(gg(dqkv, nq, 1, qd, a, nd, d, 1, dW_qkv, (int64_t)qd * d, d, 1, qd, d, n, 1, P, st));
  BW_TRY(bw_rms_bwd(ba, h1, g_at, r1, da, dh, dg_at, nd, d, n, 1, P, st));
  // ---- memory read backward
  BW_TRY(bw_memr_bwd(ba, dh, num, den, dnum, dden, nd, n, P, st));
  BW_TRY(gg(dnum, nd, d, 1, Ast, A_ps, 64, 1, dq, n64, 64, 1, n, 64, d, 0, P, st, 0, wb));
  BW_TRY(gg(dnum, nd, 1, d, q, n64, 64, 1, dA, D64, 64, 1, d, 64, n, 1, P, st, 0, wb));
  BW_TRY(bw_memr_dq(ba, dq, u, q, dden, zst, dz, n64, z_ps, 64, n, P, st));
  BW_TRY(gg(dq, n64, 64, 1, W_mq, 64 * (int64_t)d, d, 1, dh, nd, d, 1, n, d, 64, 1, P, st, wb, wb));
  BW_TRY(gg(dq, n64, 1, 64, hin, hin_ps, d, 1, dW_mq, 64 * (int64_t)d, d, 1, 64, d, n, 1, P, st, 0, wb));

  // ---- the gradient of each node's input rows: to the layer below, or to x
  // and the memory embeddings at layer 0
  float* dH_out = cx.f(cx.lo.dH) + (int64_t)(c & 1) * L * nd;
  const int p0 = (l0 == 0) ? 1 : 0;
  if (P - p0 > 0) BW_TRY(bw_copy(dh + p0 * nd, dH_out + (int64_t)(l0 + p0) * nd, nd, nd, nd, 0, P - p0, st));
  if (l0 == 0) {
    const int s = c;
    BW_TRY(bw_copy(dh, dx + (int64_t)s * T * d, (int64_t)T * d, 0, 0, 0, 1, st));
    BW_TRY(bw_copy(dh + (int64_t)T * d, (float*)cx.gw->mem_emb, (int64_t)M * d, 0, 0, 1, 1, st));
  }
  return hipSuccess;
}

// Record node (c - l, l)'s input rows and the state it reads, l = l0 ..
// l0 + P - 1, before wave c runs.
hipError_t save_wave(BwCtx& cx, int c, int l0, int P, const void* x) {
  armt_handle* h = cx.h;
  const armt_config& cf = h->cfg;
  const int S = cx.S, d = cf.d_model, n = h->n, T = cf.seg_len, M = cf.n_mem;
  const int64_t nd = (int64_t)n * d, D64 = (int64_t)d * 64;
  const int64_t tap = (int64_t)l0 * S + (c - l0);
  float* th = cx.f(cx.lo.tape_h) + tap * nd;
  const int64_t hps = (int64_t)(S - 1) * nd;
  hipStream_t st = cx.st;
  const int p0 = (l0 == 0) ? 1 : 0;
  if (l0 == 0) {
    const int s = c;
    if (h->bf16) {
      BW_TRY(launch_widen((const bf16*)x + (int64_t)s * T * d, th, (int64_t)T * d, true, st));
      BW_TRY(launch_widen(h->w.mem_emb, th + (int64_t)T * d, (int64_t)M * d, true, st));
    } else {
      BW_TRY(bw_copy((const float*)x + (int64_t)s * T * d, th, (int64_t)T * d, 0, 0, 0, 1, st));
      BW_TRY(bw_copy((const float*)h->w.mem_emb, th + (int64_t)T * d, (int64_t)M * d, 0, 0, 0, 1, st));
    }
  }
  if (P - p0 > 0) {
    const float* prev = (const float*)h->act[(c - 1) & 1] + (int64_t)(l0 + p0 - 1) * nd;
    BW_TRY(bw_copy(prev, th + p0 * hps, nd, nd, hps, 0, P - p0, st));
  }
  BW_TRY(bw_copy(h->A + (int64_t)l0 * D64, cx.f(cx.lo.tape_A) + tap * D64, D64, D64, (int64_t)(S - 1) * D64, 0, P, st));
  BW_TRY(bw_copy(h->z + (int64_t)l0 * 64, cx.f(cx.lo.tape_z) + tap * 64, 64, 64, (int64_t)(S - 1) * 64, 0, P, st));
  return hipSuccess;
}

}  // namespace

extern "C" {

int armt_backward_workspace_size(armt_handle* h, int32_t n_segments, size_t* bytes) {
  if (!h || !bytes) return fail(ARMT_E_INVALID, "NULL argument");
  if (h->llama) return fail(ARMT_E_INVALID, "handle is a full-attention comparator");
  if (h->batch != 1) return fail(ARMT_E_UNSUPPORTED, "the backward runs on batch-1 handles");
  if (n_segments < 1) return fail(ARMT_E_INVALID, "n_segments must be >= 1");
  if (h->bf16) {
    // the input-gradient products run on the grouped bf16 GEMM with the
    // weights transposed: every weight dimension a multiple of 64
    const armt_config& c = h->cfg;
    const int hd = c.n_heads * c.head_dim;
    if (c.d_model % 64 || c.ffn_hidden % 64 || h->qkv_dim % 64 || hd % 64)
      return fail(ARMT_E_UNSUPPORTED, "bf16 backward needs d, F, (H + 2G) hd and H hd multiples of 64");
  }
  *bytes = make_bw_layout(&h->cfg, n_segments).total;
  return ARMT_OK;
}

int armt_backward(armt_handle* h, int32_t schedule, const void* x, int32_t n_segments, const float* A0,
                  const float* z0, const void* dy, const float* dA_out, const float* dz_out, void* dx, float* dA0,
                  float* dz0, const armt_weights* grads, void* workspace, size_t ws_bytes) {
  size_t need = 0;
  int rc = armt_backward_workspace_size(h, n_segments, &need);
  if (rc != ARMT_OK) return rc;
  if (schedule != 0 && schedule != 1) return fail(ARMT_E_INVALID, "schedule must be 0 (diagonal) or 1 (sequential)");
  if (!x || !dy || !dx || !dA0 || !dz0 || !grads) return fail(ARMT_E_INVALID, "x, dy, dx, dA0, dz0 and grads must not be NULL");
  const void* gp[] = {grads->w_qkv, grads->w_o, grads->w_gate, grads->w_up, grads->w_down, grads->g_attn,
                      grads->g_mlp, grads->w_mq, grads->w_mk, grads->w_mv, grads->w_beta, grads->mem_emb};
  for (const void* p : gp)
    if (!p) return fail(ARMT_E_INVALID, "every gradient pointer must be non-NULL");
  if (!workspace || (uintptr_t)workspace % kAlign) return fail(ARMT_E_WORKSPACE, "workspace missing or misaligned");
  if (ws_bytes < need) return fail(ARMT_E_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  const armt_config& c = h->cfg;
  const int L = c.n_layers, S = n_segments, d = c.d_model, F = c.ffn_hidden;
  const int qd = h->qkv_dim, hhd = c.n_heads * c.head_dim;
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  BwCtx cx{h, h->stream, S, (char*)workspace, make_bw_layout(&c, S), grads, nullptr, nullptr, nullptr};
  hipStream_t st = h->stream;
  if (h->bf16) {
    float* g32 = cx.f(cx.lo.g32);
    const int64_t Ld = (int64_t)L * d;
    if ((e = launch_widen(h->w.g_attn, g32, Ld, true, st)) != hipSuccess) return hip_fail(e, "widen gains");
    if ((e = launch_widen(h->w.g_mlp, g32 + Ld, Ld, true, st)) != hipSuccess) return hip_fail(e, "widen gains");
    if ((e = launch_widen(h->w.w_beta, g32 + 2 * Ld, Ld, true, st)) != hipSuccess) return hip_fail(e, "widen gains");
    cx.g_attn = g32;
    cx.g_mlp = g32 + Ld;
    cx.w_beta = g32 + 2 * Ld;
    // transposed weights for the input-gradient products ([in][out] rows of
    // ld elements; W_g^T and W_u^T side by side for the one gate/up product)
    const int hd = c.n_heads * c.head_dim;
    struct { const void* w; int out, in; size_t at; int ld, off; } tw[] = {
        {h->w.w_down, d, F, cx.lo.wtd, 2 * d, 0},
        {h->w.w_gate, F, d, cx.lo.wtgu, 4 * F, 0},
        {h->w.w_up, F, d, cx.lo.wtgu, 4 * F, F},
        {h->w.w_o, d, hd, cx.lo.wto, 2 * d, 0},
        {h->w.w_qkv, qd, d, cx.lo.wtq, 2 * qd, 0}};
    for (const auto& t : tw) {
      bf16* dst = (bf16*)((char*)workspace + t.at);
      const int64_t dps = (int64_t)t.in * t.ld;
      if ((e = bw_transpose_bf16(t.w, true, t.in, (int64_t)t.out * t.in, t.out, t.out, t.in, dst + t.off, nullptr,
                                 t.ld, dps, L, st)) != hipSuccess)
        return hip_fail(e, "transposed weights");
    }
  } else {
    cx.g_attn = (const float*)h->w.g_attn;
    cx.g_mlp = (const float*)h->w.g_mlp;
    cx.w_beta = (const float*)h->w.w_beta;
  }
  // 1. forward, recording the tape (direct launches, the chosen order)
  const int64_t a_count = (int64_t)L * d * 64, z_count = (int64_t)L * 64;
  if ((e = launch_set_desc(h->desc, x, cx.f(cx.lo.yscr), 0, S, c.seg_len, (int64_t)S * c.seg_len, st)) != hipSuccess)
    return hip_fail(e, "set_desc");
  if ((e = launch_fill_f32(h->A, A0, a_count, st)) != hipSuccess) return hip_fail(e, "state init");
  if ((e = launch_fill_f32(h->z, z0, z_count, st)) != hipSuccess) return hip_fail(e, "state init");
  if (h->bf16 && (e = launch_split_state(h->A, h->A2, a_count / 64, st)) != hipSuccess) return hip_fail(e, "state init");
  StepCtx sc{h, st, false};
  if (schedule == 0) {
    for (int w = 0; w < S + L - 1; ++w) {
      const int l_lo = w - S + 1 > 0 ? w - S + 1 : 0, l_hi = w < L - 1 ? w : L - 1;
      if ((e = save_wave(cx, w, l_lo, l_hi - l_lo + 1, x)) != hipSuccess) return hip_fail(e, "tape");
      if ((e = enqueue_step(sc, l_lo, l_hi, w & 1, 1)) != hipSuccess) return hip_fail(e, "forward");
    }
  } else {
    for (int s = 0; s < S; ++s)
      for (int l = 0; l < L; ++l) {
        if ((e = save_wave(cx, s + l, l, 1, x)) != hipSuccess) return hip_fail(e, "tape");
        if ((e = enqueue_step(sc, l, l, (s + l) & 1, l == L - 1 ? 2 - L : 1)) != hipSuccess) return hip_fail(e, "forward");
      }
  }
  // 2. zero the gradients; the state gradient starts from dA_out, dz_out
  const size_t wsz[] = {(size_t)L * qd * d, (size_t)L * d * hhd, (size_t)L * F * d, (size_t)L * F * d,
                        (size_t)L * d * F, (size_t)L * d, (size_t)L * d, (size_t)L * 64 * d, (size_t)L * 64 * d,
                        (size_t)L * d * d, (size_t)L * d, (size_t)c.n_mem * d};
  for (int i = 0; i < 12; ++i)
    if ((e = hipMemsetAsync((void*)gp[i], 0, wsz[i] * 4, st)) != hipSuccess) return hip_fail(e, "zero gradients");
  if ((e = launch_fill_f32(cx.f(cx.lo.dA), dA_out, a_count, st)) != hipSuccess) return hip_fail(e, "dA init");
  if ((e = launch_fill_f32(cx.f(cx.lo.dz), dz_out, z_count, st)) != hipSuccess) return hip_fail(e, "dz init");
  // 3. the reversed schedule
  if (schedule == 0) {
    for (int w = S + L - 2; w >= 0; --w) {
      const int l_lo = w - S + 1 > 0 ? w - S + 1 : 0, l_hi = w < L - 1 ? w : L - 1;
      if ((e = backward_wave(cx, w, l_lo, l_hi - l_lo + 1, dy, (float*)dx)) != hipSuccess)
        return hip_fail(e, "backward");
    }
  } else {
    for (int s = S - 1; s >= 0; --s)
      for (int l = L - 1; l >= 0; --l)
        if ((e = backward_wave(cx, s + l, l, 1, dy, (float*)dx)) != hipSuccess)
          return hip_fail(e, "backward");
  }
  if ((e = hipMemcpyAsync(dA0, cx.f(cx.lo.dA), a_count * 4, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return hip_fail(e, "copy dA0");
  if ((e = hipMemcpyAsync(dz0, cx.f(cx.lo.dz), z_count * 4, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return hip_fail(e, "copy dz0");
  return ARMT_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Diagonal forward for callers that cannot allocate (graph capture, tight
// serving loops): the workspace is a file-scope device array instead of a
// caller buffer.
// ---------------------------------------------------------------------------

namespace {

// Largest workspace the static scratch holds (the tiny and small workloads
// and mid-sized models; the 1B / 3B shapes need a caller workspace).
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

// Each GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (the array's name is only a host-side stand-in).
void* g_scratch[kMaxDevices];
std::atomic<int> g_scratch_lock{0};

int scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return fail(ARMT_E_UNSUPPORTED, "device %d: too many devices", device);
  while (g_scratch_lock.exchange(1, std::memory_order_acquire)) {
  }
  hipError_t e = hipSuccess;
  if (!g_scratch[device]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) g_scratch[device] = p;
  }
  *ptr = g_scratch[device];
  g_scratch_lock.store(0, std::memory_order_release);
  return e == hipSuccess ? ARMT_OK : hip_fail(e, "hipGetSymbolAddress(scratch)");
}

// RoPE table [n][hd/2](cos, sin) of the angles pos * theta^(-2i/hd), in
// double precision as the host table of the workspace path.
__global__ void rope_table_kernel(float* tab, int n, int hd, double theta) {
  const int half = hd / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * half) return;
  const int p = idx / half, i = idx % half;
  const double ang = p * pow(theta, -2.0 * i / hd);
  tab[2 * idx] = (float)cos(ang);
  tab[2 * idx + 1] = (float)sin(ang);
}

__global__ void zero_words_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

extern "C" {

int armt_forward_diagonal_noalloc(const armt_config* cfg, const armt_weights* w, const void* x, int32_t n_segments,
                                  const float* A0, const float* z0, void* y, float* A_out, float* z_out,
                                  void* hip_stream) {
  int rc = validate_config(cfg);
  if (rc != ARMT_OK) return rc;
  if (!w) return fail(ARMT_E_INVALID, "weights must not be NULL");
  const void* ptrs[] = {w->w_qkv, w->w_o, w->w_gate, w->w_up, w->w_down, w->g_attn,
                        w->g_mlp, w->w_mq, w->w_mk, w->w_mv, w->w_beta, w->mem_emb};
  for (const void* p : ptrs)
    if (!p) return fail(ARMT_E_INVALID, "every weight pointer must be non-NULL");
  const Layout lo = make_layout(cfg, 1);
  if (lo.total > kScratchBytes)
    return fail(ARMT_E_WORKSPACE,
                "this model needs %zu bytes of workspace; the static scratch of "
                "armt_forward_diagonal_noalloc holds %zu: create a handle with a workspace instead",
                lo.total, kScratchBytes);
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  if ((rc = scratch_address(device, &ws)) != ARMT_OK) return rc;
  // a handle on the stack over the scratch: direct launches (no graphs)
  armt_handle h;
  h.batch = 1;
  h.norm_rows = (int64_t)cfg->n_layers * (cfg->seg_len + cfg->n_mem);
  set_fields(&h, cfg, w, lo, ws, hip_stream, cfg->seg_len + cfg->n_mem);
  h.device = device;
  h.use_graphs = false;
  e = hipDeviceGetAttribute(&h.cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess || h.cus <= 0) return hip_fail(e, "hipDeviceGetAttribute");
  // what the forward reads before writing: the RoPE table and the zero V^T
  // padding (another call may have left other values in the scratch)
  const int half = cfg->head_dim / 2, items = h.n * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((items + 255) / 256), dim3(256), 0, h.stream, h.rope, h.n,
                     cfg->head_dim, (double)cfg->rope_theta);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "RoPE table");
  if (h.bf16) {
    const int64_t words = (int64_t)(lo.attn - lo.vt) / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, h.stream, (uint32_t*)h.vt, words);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "V^T padding");
  }
  return forward(&h, SCHED_DIAG, x, n_segments, cfg->seg_len, A0, z0, y, A_out, z_out);
}

}  // extern "C"
