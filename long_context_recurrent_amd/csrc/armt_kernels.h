// Launch-argument structs and host launchers of the ARMT kernels (internal to
// libarmt.so; the public boundary is include/armt.h).
//
// Every kernel works on the P consecutive layers l0 .. l0+P-1 of one wave, and
// on every sequence of the batch: problem p = layer * batch + sequence.
// Buffers indexed "by problem" hold one [n, ...] slab per problem at a fixed
// stride, weights are indexed by layer, so a node's kernels read and write the
// same addresses whatever the wave width -- the grouped launch and the
// one-node launch compute bitwise identical results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "armt_common.h"

namespace armt {

// EPI_STORE: plain fp32 store of the product (LM-head logits)
enum { EPI_STORE = 0, EPI_QKV = 1, EPI_RESID = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  int P, l0;                 // layers l0 .. l0+P-1, each with `batch` problems
  int batch;                 // sequences per node: problem = layer * batch + sequence
  const void* A;             // activations, layer l at A + l * a_stride
  int64_t a_stride;
  int lda;
  const void* B;             // weights [L][N][K]
  const void* B2;            // EPI_SWIGLU: up weights [L][N][K] (B = gate)
  int64_t b_stride;
  int M, N, K;               // per problem (N = output columns)
  void* C;                   // output, layer l at C + l * c_stride
  int64_t c_stride;
  int ldc;
  // EPI_QKV
  const float* rope_cs;      // [n][hd/2] (cos, sin) pairs
  int rope_cols;             // columns below get RoPE ((H + G) * hd)
  int head_dim;
  int v_col0;                // first V column ((H + G) * hd)
  void* vt;                  // bf16 path: V transposed [L][G*hd][vt_ld]
  int64_t vt_stride;
  int vt_ld;
  // EPI_RESID
  const CallDesc* desc;      // y pointer and wave counter (nullptr: no y)
  int last_layer;            // layer whose segment rows also go to y
  int T;                     // segment rows
  int ldb;                   // row stride of B in elements (0: K)
};

struct AttnArgs {
  int P, l0;
  const void* qkv;           // [L][n][(H + 2G) * hd]
  int64_t qkv_stride;
  int ld_qkv;
  const void* vt;            // bf16 path: [L][G*hd][vt_ld]
  int64_t vt_stride;
  int vt_ld;
  void* out;                 // [L][n][H * hd]
  int64_t out_stride;
  int ld_out;
  int n, H, G, hd;
  float scale;               // 1 / sqrt(hd)
};

struct MemArgs {
  int P, l0;                 // problems l0 .. l0+P-1, problem = layer * batch + sequence
  int batch;                 // sequences per node (weights are indexed by problem / batch)
  int n, d, T, M, dk, L;
  const void* act_prev;      // previous-wave slot [L][n][d] (layer l reads l-1)
  void* act_cur;             // this wave's slot [L][n][d]
  void* abuf;                // normalised activations [L][n][d]
  int64_t act_stride;        // n * d
  const void* mem_emb;       // [M][d]
  const void* w_mq;          // [L][dk][d]
  const void* w_mk;          // [L][dk][d]
  const void* w_mv;          // [L][d][d]
  const void* w_beta;        // [L][d]
  const void* gain;          // [L][d] (g_attn or g_mlp)
  float* A;                  // [L][d][dk] fp32 state
  bf16* A2;                  // [L][d][2][dk] the state as bf16 hi / lo parts (bf16 path)
  float* z;                  // [L][dk]
  float* qbuf;               // [L][n][dk] read keys phi(h W_mq^T) (bf16 path)
  float* kbuf;               // [L][M][dk] write keys phi(Y W_mk^T)
  float* pden;               // [L][M][4] partial k . z (pre-update z), 16 keys each
  float* beta;               // [L][M]
  int* moff;                 // [L] first memory row of the node (mem_keys -> mem_update)
  CallDesc* desc;
  int advance;               // mem_update: wave-counter increment (0: none)
  float mem_eps, rms_eps;
};

// Final RMSNorm: out[r] = R(x[r] / sqrt(mean(x[r]^2) + eps) * gain), rows of d.
struct NormArgs {
  const void* x;             // [rows][d] config dtype
  const void* gain;          // [d]
  void* out;                 // [rows][d]
  int rows, d;
  float eps;
};

// ---- backward (fp32) ----------------------------------------------------
// Generic strided GEMM over P problems (the backward's products):
// C = (accumulate ? C : 0) + A B with A(m, k) = A + p*a_ps + m*a_rs + k*a_cs,
// B(k, n) and C(m, n) likewise; A and C fp32, B fp32 or bf16.
struct GenGemm {
  const float* A;
  const void* B;             // fp32, or bf16 when b_bf16 (strides in elements)
  float* C;
  int64_t a_ps, a_rs, a_cs, b_ps, b_rs, b_cs, c_ps, c_rs, c_cs;
  int M, N, K, accumulate;
  int b_bf16;
};

// Shapes shared by the backward kernels.
struct BwArgs {
  int d, n, M, hd, H, G, qkv_ld;
  int row_ps;                // per-problem stride of row-scalar arrays (n)
  float mem_eps, rms_eps, scale;
  const float* rope;         // [n][hd/2] (cos, sin)
};

// Causal attention of the backward on the matrix cores (bf16 operands, fp32
// accumulation; head dimension 64 or 128): the recomputed forward (O, base-2
// row statistics) and dQ, dK, dV.  bw_attn_mfma_ok tells whether a shape is
// supported.
bool bw_attn_mfma_ok(const BwArgs& a);
hipError_t bw_attn_mfma_fwd(const BwArgs& a, const float* qkv, float* O, float* mx, float* ls, int64_t qkv_ps,
                            int64_t o_ps, int64_t st_ps, int P, hipStream_t st);
hipError_t bw_attn_mfma_bwd(const BwArgs& a, const float* qkv, const float* O, const float* dO, const float* mx,
                            const float* ls, float* Dq, float* dqkv, int64_t qkv_ps, int64_t o_ps, int64_t st_ps,
                            int P, hipStream_t st);
// matrix_cores: bf16 MFMA with fp32 operands split into bf16 pairs (about
// 16 bits each survive), else fp32 fused multiply-adds in k order
hipError_t launch_gemm_gen(const GenGemm& g, int P, bool matrix_cores, hipStream_t st);
hipError_t bw_phi_den(const BwArgs& a, const float* u, float* q, float* den, const float* z, int64_t u_ps,
                      int64_t z_ps, int rows, int P, hipStream_t st);
hipError_t bw_add_div(const BwArgs& a, const float* base, const float* num, const float* den, float* out, int64_t ps,
                      int rows, int P, hipStream_t st);
hipError_t bw_rms_fwd(const BwArgs& a, const float* x, const float* g, float* out, float* rs, int64_t ps,
                      int64_t g_ps, int rows, int P, hipStream_t st);
hipError_t bw_rms_bwd(const BwArgs& a, const float* x, const float* g, const float* rs, const float* dy, float* dx,
                      float* dg, int64_t ps, int64_t g_ps, int rows, int accumulate, int P, hipStream_t st);
hipError_t bw_rope(const BwArgs& a, float* x, int64_t ps, int ld, int col0, int heads, float sign, int rows, int P,
                   hipStream_t st);
hipError_t bw_attn_fwd(const BwArgs& a, const float* qkv, float* O, float* mx, float* ls, int64_t qkv_ps,
                       int64_t o_ps, int64_t st_ps, int P, hipStream_t st);
hipError_t bw_attn_bwd(const BwArgs& a, const float* qkv, const float* O, const float* dO, const float* mx,
                       const float* ls, float* Dq, float* dqkv, int64_t qkv_ps, int64_t o_ps, int64_t st_ps, int P,
                       hipStream_t st);
hipError_t bw_swiglu(const float* G, const float* Up, float* Uo, int64_t count, int64_t ps, int P, hipStream_t st);
hipError_t bw_swiglu_bwd(const float* G, const float* Up, const float* dUo, float* dG, float* dUp, int64_t count,
                         int64_t ps, int P, hipStream_t st);
hipError_t bw_memw_fwd(const BwArgs& a, const float* uk, float* k, const float* bl, float* beta, const float* z,
                       float* denw, const float* kA, const float* v, float* e, int64_t z_ps, int P, hipStream_t st);
hipError_t bw_memw_bwd(const BwArgs& a, const float* de, const float* v, const float* kA, const float* beta,
                       const float* denw, float* dv, float* dkA, float* ddenw, float* dbl, int P, hipStream_t st);
hipError_t bw_memw_dk(const BwArgs& a, float* dk, const float* uk, const float* k, const float* ddenw, const float* z,
                      float* dz, int64_t z_ps, int64_t dz_ps, int P, hipStream_t st);
hipError_t bw_memw_beta(const BwArgs& a, const float* dbl, const float* wb, const float* Y, float* dY, float* dwb,
                        int64_t y_ps, int64_t wb_ps, int P, hipStream_t st);
hipError_t bw_memr_bwd(const BwArgs& a, const float* dh1, const float* num, const float* den, float* dnum, float* dden,
                       int64_t ps, int rows, int P, hipStream_t st);
hipError_t bw_memr_dq(const BwArgs& a, float* dq, const float* u, const float* q, const float* dden, const float* z,
                      float* dz, int64_t u_ps, int64_t z_ps, int64_t dz_ps, int rows, int P, hipStream_t st);
hipError_t bw_copy(const float* src, float* dst, int64_t count, int64_t src_ps, int64_t dst_ps, int accumulate, int P,
                   hipStream_t st);
hipError_t bw_to_bf16(const float* src, bf16* dst, int64_t count, int64_t ps, int P, hipStream_t st);
// dst[r][c] = hi(src[r][c]), dst[r][lo_off + c] = lo(src[r][c]): fp32 rows as
// bf16 pairs, per problem
hipError_t bw_split_bf16(const float* src, int64_t ld_src, int64_t src_ps, int rows, int cols, bf16* dst,
                         int64_t ld_dst, int64_t dst_ps, int lo_off, int P, hipStream_t st);
// dst[c][r] = src[r][c] (r < rows; zero up to rows_pad, a multiple of 64) as
// bf16 hi (and lo when dst_lo) parts, per problem; destination rows ld_dst apart
hipError_t bw_transpose_bf16(const void* src, bool src_bf16, int64_t ld_src, int64_t src_ps, int rows, int rows_pad,
                             int cols, bf16* dst_hi, bf16* dst_lo, int64_t ld_dst, int64_t dst_ps, int P,
                             hipStream_t st);

// tile heights of the bf16 GEMM, in 32-row MFMA blocks, that have instantiations
extern const int kGemmRowBlocks[];
extern const int kGemmRowBlocksCount;

hipError_t launch_gemm_bf16(const GemmArgs& g, int epi, int mb, hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs& g, int epi, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, bool use_bf16, hipStream_t st);
hipError_t launch_mem_read(const MemArgs& m, bool use_bf16, hipStream_t st);
hipError_t launch_rmsnorm(const MemArgs& m, bool use_bf16, hipStream_t st);
hipError_t launch_mem_keys(const MemArgs& m, bool use_bf16, hipStream_t st);
hipError_t launch_mem_update(const MemArgs& m, bool use_bf16, hipStream_t st);
hipError_t launch_mem_read_bf16(const MemArgs& m, hipStream_t st);
hipError_t launch_mem_keys_bf16(const MemArgs& m, hipStream_t st);
hipError_t launch_mem_update_bf16(const MemArgs& m, hipStream_t st);
hipError_t launch_final_norm(const NormArgs& a, bool use_bf16, hipStream_t st);
// dst[i] = (float)src[i], count a multiple of 8
hipError_t launch_widen(const void* src, float* dst, int64_t count, bool use_bf16, hipStream_t st);
hipError_t launch_set_desc(CallDesc* desc, const void* x, void* y, int c0, int S, int t_last, int64_t seq_rows,
                           hipStream_t st);
hipError_t launch_fill_f32(float* dst, const float* src, int64_t count, hipStream_t st);
// A2[r] = (hi, lo) of A[r] for rows of 64 (hi = R(v), lo = R(v - hi)): the
// bf16 path's copy of the memory state, refreshed by every memory update
hipError_t launch_split_state(const float* A, bf16* A2, int64_t rows, hipStream_t st);

}  // namespace armt
