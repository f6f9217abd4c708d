/*
 * armt.h -- C ABI of libarmt.so: the forward pass of a layer-level recurrent
 * memory transformer (ARMT) on one AMD Instinct MI355X (gfx950), run either
 * segment-major ("sequential") or by diagonal waves ("diagonal batching").
 *
 * What is computed.  A sequence of S segments of T tokens passes through L
 * layers.  Node (s, l) -- segment s at layer l -- reads layer l's associative
 * memory (A_l, z_l), runs a Llama-shaped block over its n = T + M rows (the T
 * segment tokens followed by M memory tokens) and then updates (A_l, z_l) from
 * its M memory-token rows.  Node (s, l) needs only node (s, l-1)'s hidden
 * states and node (s-1, l)'s memory state, so all nodes with s + l = i are
 * independent and the grid runs as S + L - 1 waves, each launched as one
 * grouped layer over stacked per-layer weights (Pith review of arXiv
 * 2506.05229, "What carries the argument", Lemma 3.1 and Section 3.3 on
 * uniform layer geometry; skill page "Diagonal Batching for Recurrent Memory
 * Transformers", Implementation and Practical Guidance).  Per node:
 *
 *   read : h  = h_in + (q A^T) / (q . z + mem_eps),  q = phi(h_in W_mq^T)
 *   attn : a  = R(rms(h) * g_attn);  Q|K|V = a W_qkv^T;  Q, K = RoPE;  R(Q,K,V)
 *          O  = R(causal softmax(Q K^T / sqrt(hd)) V), q-head j reads kv-head
 *               j / (H/G);  h = h + O W_o^T
 *   mlp  : b  = R(rms(h) * g_mlp);  U = R(silu(b W_gate^T) * (b W_up^T))
 *          h  = h + U W_down^T               -> node output; rows 0..T-1 of the
 *                                               last layer give y[sT:(s+1)T] = R(h)
 *   write: Y = h[T:n]; k_m = phi(Y_m W_mk^T); v_m = Y_m W_mv^T;
 *          beta_m = sigmoid(Y_m . w_beta); vbar_m = (k_m A^T) / (k_m . z + mem_eps)
 *          A += sum_m beta_m (v_m - vbar_m) k_m^T;  z += sum_m k_m
 *
 * phi(u) = elu(u) + 1; rms(u) = u / sqrt(mean(u^2) + rms_eps); RoPE pairs
 * coordinate i with i + hd/2 at angle pos * rope_theta^(-2i/hd), positions
 * 0..n-1 in every segment.  R() stores a branch activation in the config
 * dtype (identity for ARMT_F32, round-to-nearest-even bfloat16 for ARMT_BF16);
 * the residual stream h -- the running sum of the memory read and the branch
 * outputs across layers -- is fp32 in both dtypes, and so is the memory state
 * (A, z); products accumulate in fp32.  The pages name the model family but
 * print none of these equations: this is the reading the library implements.
 *
 * Conventions.  Every pointer argument that is not documented as host memory
 * is a device pointer on the HIP device that was current at armt_create.
 * Matrices are row-major [out_features, in_features], stacked over a leading
 * layer axis.  All calls return an armt_status; a non-OK return enqueues no
 * GPU work and armt_last_error() gives a message.  No C++ exception crosses
 * this boundary.
 */
#ifndef ARMT_H
#define ARMT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ARMT_OK = 0,
  ARMT_E_INVALID = -1,      /* NULL pointer, non-positive or inconsistent size */
  ARMT_E_UNSUPPORTED = -2,  /* valid but outside what the kernels implement   */
  ARMT_E_WORKSPACE = -3,    /* workspace missing, too small or misaligned      */
  ARMT_E_HIP = -4           /* a HIP runtime call failed                       */
} armt_status;

typedef enum { ARMT_F32 = 0, ARMT_BF16 = 1 } armt_dtype;

/* Model geometry.  All layers share it (uniform layer geometry, Pith review
 * assumptions / Section 3.3).  Constraints checked by armt_create:
 * every size > 0; d_model == n_heads * head_dim; n_heads % n_kv_heads == 0;
 * head_dim in {32, 64, 128}; d_key == 64; d_model % 64 == 0;
 * ffn_hidden % 64 == 0; n_mem <= 64; dtype ARMT_BF16 or ARMT_F32;
 * ARMT_BF16: seg_len + n_mem <= 4096, d_model % 128 == 0 and d_model <= 3072;
 * ARMT_F32: seg_len + n_mem <= 2048 and d_model <= 1024.  Defaults used by the workloads:
 * rms_eps 1e-5, rope_theta 10000, mem_eps 1e-6. */
typedef struct {
  int32_t n_layers;    /* L */
  int32_t d_model;     /* d */
  int32_t n_heads;     /* H query heads */
  int32_t n_kv_heads;  /* G key/value heads */
  int32_t head_dim;    /* hd */
  int32_t ffn_hidden;  /* F (SwiGLU hidden size) */
  int32_t seg_len;     /* T tokens per segment */
  int32_t n_mem;       /* M memory tokens per segment */
  int32_t d_key;       /* d_k, phi-key width of the associative memory */
  int32_t dtype;       /* armt_dtype of activations and weights */
  float rms_eps;
  float rope_theta;
  float mem_eps;
} armt_config;

/* Stacked weights, all in the config's dtype, device memory.  Borrowed: they
 * must stay alive and unchanged until armt_destroy. */
typedef struct {
  const void *w_qkv;   /* [L, (H + 2G) * hd, d]  rows: Q heads, K heads, V heads */
  const void *w_o;     /* [L, d, H * hd] */
  const void *w_gate;  /* [L, F, d] */
  const void *w_up;    /* [L, F, d] */
  const void *w_down;  /* [L, d, F] */
  const void *g_attn;  /* [L, d]  RMSNorm gain before attention */
  const void *g_mlp;   /* [L, d]  RMSNorm gain before the MLP */
  const void *w_mq;    /* [L, d_k, d]  memory-read query projection */
  const void *w_mk;    /* [L, d_k, d]  memory-write key projection */
  const void *w_mv;    /* [L, d, d]    memory-write value projection */
  const void *w_beta;  /* [L, d]       memory-write gate */
  const void *mem_emb; /* [M, d]       memory-token embeddings */
} armt_weights;

typedef struct armt_handle armt_handle;

/* Bytes of device workspace armt_create needs for this config (host call,
 * no GPU work).  Returns ARMT_E_INVALID / ARMT_E_UNSUPPORTED for a config
 * armt_create would reject. */
int armt_workspace_size(const armt_config *cfg, size_t *bytes);

/* Validate the config, borrow the weights and carve the caller's workspace
 * (device memory of at least armt_workspace_size bytes, 256-byte aligned,
 * owned by the caller and not touched by anyone else until armt_destroy).
 * hip_stream is the hipStream_t every forward is enqueued on (NULL = the
 * device's null stream).  Uploads the RoPE table (synchronous, once).
 * On success *out receives a handle to release with armt_destroy. */
int armt_create(const armt_config *cfg, const armt_weights *w, void *workspace,
                size_t ws_bytes, void *hip_stream, armt_handle **out);

/* Several independent sequences per node (batch B): each node (s, l) runs
 * segment s of all B sequences through layer l, each sequence with its own
 * memory state, in the same grouped launches (the kernels see P layers x B
 * sequences).  The pages contrast diagonal batching with batching several
 * requests (paper page, abstract; skill page, Practical Guidance); both
 * compose.  armt_workspace_size_batched / armt_create_batched are
 * armt_workspace_size / armt_create for a batch of 1 <= batch <= 1024; the
 * forward calls of such a handle take
 *   x, y         [B][rows][d]   (rows = n_segments * T, or n_tokens)
 *   A0, A_out    [L][B][d][d_k] fp32;  z0, z_out [L][B][d_k] fp32
 * and all B sequences have the same length.  With B = 1 everything is as
 * documented for the unbatched calls. */
int armt_workspace_size_batched(const armt_config *cfg, int32_t batch, size_t *bytes);
int armt_create_batched(const armt_config *cfg, const armt_weights *w, int32_t batch,
                        void *workspace, size_t ws_bytes, void *hip_stream,
                        armt_handle **out);

/* Forward over n_segments segments in segment-major order: for s, for l,
 * node(s, l) -- the S*L-step baseline schedule (Pith review, Figure 3).
 *   x     [n_segments * T, d]  input token embeddings (config dtype)
 *   A0    [L, d, d_k] fp32 initial memory, or NULL for zeros
 *   z0    [L, d_k]    fp32 initial normaliser, or NULL for zeros
 *   y     [n_segments * T, d]  last layer's segment-token rows (config dtype)
 *   A_out [L, d, d_k], z_out [L, d_k]  fp32 memory after the last segment;
 *         may alias A0 / z0 (streaming a long input chunk by chunk).
 * Asynchronous on the handle's stream, no host synchronisation; results are
 * valid once the stream is synchronised.  Calls on one handle must not
 * overlap (they share the workspace). */
int armt_forward_sequential(armt_handle *h, const void *x, int32_t n_segments,
                            const float *A0, const float *z0, void *y,
                            float *A_out, float *z_out);

/* Same arguments and results; runs the S + L - 1 diagonal waves, each wave's
 * nodes as one grouped launch per step (Pith review, "What carries the
 * argument"; abstract on the paper page).  Bitwise identical to
 * armt_forward_sequential: the kernels never depend on the wave width. */
int armt_forward_diagonal(armt_handle *h, const void *x, int32_t n_segments,
                          const float *A0, const float *z0, void *y,
                          float *A_out, float *z_out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * diagonal forward of one sequence with no handle and no caller workspace.
 * Its workspace is a static device array of the library (64 MiB per GPU,
 * held until the process ends); models whose armt_workspace_size exceeds it
 * return ARMT_E_WORKSPACE.  Arguments as armt_forward_diagonal (batch 1) plus
 * the config and the stacked device weights (borrowed for the call) and the
 * HIP stream (NULL = default stream) the kernels are launched on; results
 * equal those of a handle's armt_forward_diagonal up to the rounding of the
 * RoPE table (computed on the device here).  Launches kernels only: no
 * allocation, no host synchronisation, no graphs.  Every call on one GPU
 * uses the same array: calls that overlap on one GPU (other streams, other
 * threads) race; calls queued on one stream are ordered. */
int armt_forward_diagonal_noalloc(const armt_config *cfg, const armt_weights *w,
                                  const void *x, int32_t n_segments,
                                  const float *A0, const float *z0, void *y,
                                  float *A_out, float *z_out, void *hip_stream);

/* Any sequence length ("dynamic" segmenting): n_tokens >= 1 tokens run as
 * S = ceil(n_tokens / T) segments, the last one t = n_tokens - (S - 1) T
 * tokens long (1..T); x and y span n_tokens rows, everything else as above.
 * A short last segment is its t tokens followed by the M memory tokens
 * (positions 0..t+M-1), so its memory write reads the node's rows t..t+M-1;
 * nothing else changes (the pages' skill page, Implementation: the segment
 * count is left dynamic).  With n_tokens = S * T these are bitwise identical
 * to the calls above. */
int armt_forward_sequential_tokens(armt_handle *h, const void *x, int64_t n_tokens,
                                   const float *A0, const float *z0, void *y,
                                   float *A_out, float *z_out);
int armt_forward_diagonal_tokens(armt_handle *h, const void *x, int64_t n_tokens,
                                 const float *A0, const float *z0, void *y,
                                 float *A_out, float *z_out);

/* Final RMSNorm and LM head over rows of a forward's output: the logits the
 * pages compare between the sequential and the diagonal schedule (Pith review
 * of arXiv 2506.05229: falsifier, and the referee report on the relative
 * logit drift of Table 2; skill page "Diagonal Batching for Recurrent Memory
 * Transformers", the results listed after Practical Guidance: error
 * accumulation under 2% at 32K tokens).
 *   logits[r, v] = sum_k R(rms(y_r) * g_final)[k] * w_lm[v, k]
 * accumulated and stored in fp32 (rms and R as above, eps = rms_eps).
 *   y       [rows, d]     config dtype, e.g. the y of a forward
 *   g_final [d]           config dtype, final RMSNorm gain
 *   w_lm    [vocab, d]    config dtype, row-major [out, in]
 *   logits  [rows, vocab] fp32, row-major; must not overlap y
 * rows >= 1 and vocab >= 1 (ARMT_E_INVALID otherwise); ARMT_BF16 needs
 * vocab % 8 == 0 (ARMT_E_UNSUPPORTED).  The normalised rows pass through the
 * handle's workspace, L * (T + M) rows at a time (max_tokens for a
 * full-attention handle), so the call is ordered with
 * the forwards on the handle's stream and must not overlap them from another
 * thread.  Asynchronous; logits are valid once the stream is synchronised.
 * The weights are read only during the call (not borrowed). */
int armt_logits(armt_handle *h, const void *y, int64_t rows, const void *g_final,
                const void *w_lm, int32_t vocab, float *logits);

/* Full-attention comparator: the same Llama-shaped block stack with no memory,
 * run over a whole sequence as one causal window -- the standard transformer
 * the paper page's abstract and the Pith review's Figure 1 compare against
 * (3.3x slower than the diagonal ARMT at 131,072 tokens there, on another
 * GPU).  Per layer l, over positions 0..N-1 of x:
 *   h = h + R(causal softmax(Q K^T / sqrt(hd)) V) W_o^T  (Q, K, V as above,
 *       from R(rms(h) * g_attn[l]), RoPE positions 0..N-1)
 *   h = h + R(silu(b W_gate^T) * (b W_up^T)) W_down^T,  b = R(rms(h) * g_mlp[l])
 * with h_0 = x (fp32 stream) and y = R(h_L).  Uses the config's layer
 * geometry, dtype, rms_eps and rope_theta; seg_len, n_mem, d_key and mem_eps
 * are ignored.  Constraints: head_dim in {32, 64, 128}; d_model and
 * ffn_hidden multiples of 64, d_model <= 4096; 1 <= max_tokens <= 262144
 * (ARMT_BF16, with max_tokens * (n_heads + 2 n_kv_heads) * head_dim * 2
 * bytes of Q, K, V below 2^31) or 4096 (ARMT_F32); ARMT_E_UNSUPPORTED
 * otherwise.
 * armt_llama_workspace_size: bytes of workspace for up to max_tokens
 * positions (host call).  armt_llama_create: as armt_create, but only
 * w_qkv, w_o, w_gate, w_up, w_down, g_attn and g_mlp are used (borrowed);
 * the memory fields may be NULL.  armt_llama_forward: x [n_tokens, d] ->
 * y [n_tokens, d] (config dtype), 1 <= n_tokens <= max_tokens; asynchronous
 * on the handle's stream.  armt_logits works on such a handle too
 * (max_tokens rows per chunk); armt_forward_* reject it. */
int armt_llama_workspace_size(const armt_config *cfg, int64_t max_tokens, size_t *bytes);
int armt_llama_create(const armt_config *cfg, const armt_weights *w, int64_t max_tokens,
                      void *workspace, size_t ws_bytes, void *hip_stream, armt_handle **out);
int armt_llama_forward(armt_handle *h, const void *x, int64_t n_tokens, void *y);

/* Backward pass (training; handles with batch 1): the gradients of
 *   <y, dy> + <A_out, dA_out> + <z_out, dz_out>
 * with respect to x, A0, z0 and every weight, for the forward of
 * armt_forward_diagonal / _sequential over n_segments full segments.  Node
 * (s, l)'s backward needs the gradients from (s, l+1) and (s+1, l), so it runs
 * as the S + L - 1 waves in reverse order, one grouped launch per step
 * (schedule 0), or node by node in reverse segment-major order (schedule 1);
 * the two give bitwise equal results (the pages' appendix on the grouped
 * backward; Pith review, "What carries the argument").  A forward pass first
 * records each node's input rows and the state it read in the workspace; each
 * node's activations are recomputed from that record.
 *   x, dy  [S*T, d] in the handle's dtype;  A0, dA_out [L, d, d_k],
 *          z0, dz_out [L, d_k] fp32 (A0, z0, dA_out, dz_out may be NULL for
 *          zeros)
 *   dx [S*T, d], dA0 [L, d, d_k], dz0 [L, d_k] fp32 (outputs)
 *   grads  gradient buffers with the layout of armt_weights, fp32, device
 *          memory; overwritten
 *   workspace  device memory of armt_backward_workspace_size bytes,
 *          256-byte aligned
 * For an ARMT_BF16 handle the recording forward is the bf16 forward, and each
 * node is differentiated at the input rows that forward gave it, the
 * forward's bf16 roundings of branch activations counting as identity in the
 * gradient; its products run on the matrix cores, the bf16-rounded
 * activations as single bf16 values and every other fp32 operand (the
 * gradients among them) as a bf16 pair (about 16 bits kept), attention with
 * bf16 operands, fp32 accumulation.  ARMT_E_UNSUPPORTED unless d, F,
 * (H + 2G) hd and H hd are multiples of 64.  ARMT_F32 handles use fp32
 * vector-ALU kernels throughout.
 * Asynchronous on the handle's stream; uses the handle's workspace too (must
 * not overlap a forward on the handle).  ARMT_E_UNSUPPORTED for batched
 * handles. */
int armt_backward_workspace_size(armt_handle *h, int32_t n_segments, size_t *bytes);
int armt_backward(armt_handle *h, int32_t schedule, const void *x, int32_t n_segments,
                  const float *A0, const float *z0, const void *dy, const float *dA_out,
                  const float *dz_out, void *dx, float *dA0, float *dz0,
                  const armt_weights *grads, void *workspace, size_t ws_bytes);

void armt_destroy(armt_handle *h);

/* Message of the last non-OK status on this thread ("" if none).  Host
 * memory owned by the library, valid until the next call on this thread. */
const char *armt_last_error(void);

/* Host-only: the diagonal schedule.  Wave i runs layers l_lo[i]..l_hi[i]
 * with segment s = i - l (Lemma 3.1: S + L - 1 waves).  l_lo, l_hi are host
 * arrays of capacity `cap`; *n_waves receives S + L - 1.  ARMT_E_INVALID if
 * a size is non-positive or cap is too small. */
int armt_wave_schedule(int32_t n_layers, int32_t n_segments, int32_t *l_lo,
                       int32_t *l_hi, int32_t cap, int32_t *n_waves);

/* Execution options (host call).  ARMT_OPT_GRAPHS: 1 = replay one captured
 * hipGraph per wave shape (default), 0 = launch kernels directly.
 * ARMT_OPT_TIME_KERNEL: k >= 0 brackets every launch of kernel k (an
 * armt_kernel_id) with HIP events on the handle's stream (forces direct
 * launches); -1 turns it off.  ARMT_OPT_GEMM_ROWS: rows per grouped-GEMM
 * tile as a multiple of 16 (4, 6, 8 .. 14; 0 = pick for the workload);
 * results do not depend on it.  Changing it drops the captured graphs.
 * ARMT_OPT_DEBUG_SYNC: 1 = forwards launch their kernels directly and, after
 * every kernel, synchronise the stream and check for a HIP error, so a
 * failure returns ARMT_E_HIP naming the kernel and the wave's layers (slow;
 * for debugging); 0 = off (default).  Results are unchanged. */
enum { ARMT_OPT_GRAPHS = 0, ARMT_OPT_TIME_KERNEL = 1, ARMT_OPT_GEMM_ROWS = 2, ARMT_OPT_DEBUG_SYNC = 3 };
int armt_set_option(armt_handle *h, int32_t option, int32_t value);

/* Kernels of one wave, in launch order. */
typedef enum {
  ARMT_K_MEM_READ = 0,   /* memory read: q projection and h += (q A^T)/(q.z+eps) */
  ARMT_K_ATTN_NORM = 1,  /* RMSNorm (attention input) */
  ARMT_K_QKV = 2,        /* grouped GEMM, RoPE epilogue */
  ARMT_K_ATTN = 3,       /* batched causal segment attention */
  ARMT_K_OPROJ = 4,      /* grouped GEMM, residual epilogue */
  ARMT_K_MLP_NORM = 5,   /* RMSNorm (MLP input) */
  ARMT_K_GATE_UP = 6,    /* grouped dual GEMM, SiLU * up epilogue */
  ARMT_K_DOWN = 7,       /* grouped GEMM, residual (+ y rows) epilogue */
  ARMT_K_MEM_KEYS = 8,   /* memory-write keys, gate, normaliser update */
  ARMT_K_MEM_UPDATE = 9, /* memory-write delta-rule update of A */
  ARMT_K_COUNT = 10
} armt_kernel_id;

/* Accumulated timing of the kernel selected with ARMT_OPT_TIME_KERNEL since it
 * was selected: total milliseconds, number of launches and the algorithmic
 * FLOPs and minimum HBM bytes those launches process.  Synchronises the
 * handle's stream.  All outputs are host pointers. */
int armt_kernel_stats(armt_handle *h, double *ms, int64_t *launches,
                      double *flops, double *bytes);

/* Read-only view of an internal workspace buffer, for white-box tests of the
 * individual steps (host call, no GPU work).  After a forward the buffers hold
 * the last wave's values, slabbed by layer:
 *   ARMT_VIEW_ACT0 / ACT1  [L][n][d] fp32 node outputs of even / odd waves
 *   ARMT_VIEW_NORMED       [L][n][d] last RMSNorm output (MLP input)
 *   ARMT_VIEW_QKV          [L][n][(H+2G)hd] (bf16: V columns unused)
 *   ARMT_VIEW_VT           [L][G*hd][roundup(n, 64)] (bf16 only); within every
 *                          aligned group of 16 keys the stored order is
 *                          0-3, 8-11, 4-7, 12-15
 *   ARMT_VIEW_ATTN         [L][n][H*hd]
 *   ARMT_VIEW_SWIGLU       [L][n][F]
 *   ARMT_VIEW_A / Z        fp32 state [L][d][d_k] / [L][d_k]
 * *ptr receives a device pointer into the workspace, *bytes its size. */
enum { ARMT_VIEW_ACT0 = 0, ARMT_VIEW_ACT1 = 1, ARMT_VIEW_NORMED = 2, ARMT_VIEW_QKV = 3,
       ARMT_VIEW_VT = 4, ARMT_VIEW_ATTN = 5, ARMT_VIEW_SWIGLU = 6, ARMT_VIEW_A = 7,
       ARMT_VIEW_Z = 8 };
int armt_debug_view(armt_handle *h, int32_t which, void **ptr, size_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* ARMT_H */
