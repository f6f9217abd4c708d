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

// number of 16-row MFMA blocks per GEMM tile that have instantiations
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

}  // namespace armt
