// Grouped fp32 GEMM (vector ALU) for fp32 workloads: same problem layout and
// epilogues as the bf16 MFMA kernel (one problem per active layer of the wave;
// Pith review of arXiv 2506.05229, "What carries the argument"), used where
// activations and weights are fp32.  A workgroup of 256 lanes owns a 32 x 128
// tile (each lane 4 x 4 outputs), K advances 16 at a time through LDS.  The
// epilogue stages the tile in LDS so RoPE can pair columns i and i + hd/2
// (hd <= 128 divides the tile width).  In this path V stays row-major inside
// the QKV buffer.  EPI_STORE writes the plain product (LM-head logits).
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {
constexpr int TM = 32, TN = 128, TK = 16;
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int NOUT = (EPI == EPI_SWIGLU) ? TN / 2 : TN;
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  __shared__ float Cs[TM][TN + 1];

  const int tid = threadIdx.x;
  const int tx = tid & 31, ty = tid >> 5;
  const int prob = g.l0 * g.batch + blockIdx.z;   // (layer, sequence) problem
  const int layer = prob / g.batch, seq = prob - layer * g.batch;
  const int m0 = blockIdx.x * TM;
  const int n0 = blockIdx.y * NOUT;
  const float* A = (const float*)g.A + (int64_t)prob * g.a_stride;
  const float* B = (const float*)g.B + (int64_t)layer * g.b_stride;
  const float* B2 = (EPI == EPI_SWIGLU) ? (const float*)g.B2 + (int64_t)layer * g.b_stride : B;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
    for (int c = tid; c < TM * TK; c += 256) {
      const int r = c / TK, k = c % TK;
      const int m = m0 + r;
      As[k][r] = (m < g.M && k0 + k < g.K) ? A[(int64_t)m * g.lda + k0 + k] : 0.f;
    }
    for (int c = tid; c < TN * TK; c += 256) {
      const int r = c / TK, k = c % TK;
      float v = 0.f;
      if (EPI == EPI_SWIGLU) {
        const int nn = n0 + (r % NOUT);
        const float* src = (r < NOUT) ? B : B2;
        if (nn < g.N && k0 + k < g.K) v = src[(int64_t)nn * g.K + k0 + k];
      } else {
        const int nn = n0 + r;
        if (nn < g.N && k0 + k < g.K) v = B[(int64_t)nn * g.K + k0 + k];
      }
      Bs[k][r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
  __syncthreads();

  float* C = (float*)g.C + (int64_t)prob * g.c_stride;
  float* Y = nullptr;
  int y_rows = 0;
  if (EPI == EPI_RESID && g.desc != nullptr && layer == g.last_layer) {
    const int s = g.desc->c - layer;
    Y = (float*)g.desc->y + ((int64_t)seq * g.desc->seq_rows + (int64_t)s * g.T) * g.ldc;
    y_rows = seg_tokens(g.desc, s, g.T);
  }
  for (int c = tid; c < TM * NOUT; c += 256) {
    const int r = c / NOUT, cc = c % NOUT;
    const int m = m0 + r, n = n0 + cc;
    if (m >= g.M || n >= g.N) continue;
    float v = Cs[r][cc];
    if (EPI == EPI_QKV) {
      if (n < g.rope_cols) {
        const int hd = g.head_dim, half = hd >> 1;
        const int e = n % hd;
        if (e < half) {
          const float2 cs = *(const float2*)(g.rope_cs + ((int64_t)m * half + e) * 2);
          v = v * cs.x - Cs[r][cc + half] * cs.y;
        } else {
          const float2 cs = *(const float2*)(g.rope_cs + ((int64_t)m * half + e - half) * 2);
          v = v * cs.x + Cs[r][cc - half] * cs.y;
        }
      }
    } else if (EPI == EPI_SWIGLU) {
      const float up = Cs[r][cc + NOUT];
      v = v * sigmoid_f(v) * up;
    } else if (EPI == EPI_RESID) {
      v += C[(int64_t)m * g.ldc + n];
    }
    C[(int64_t)m * g.ldc + n] = v;
    if (m < y_rows) Y[(int64_t)m * g.ldc + n] = v;
  }
}

hipError_t launch_gemm_f32(const GemmArgs& g, int epi, hipStream_t st) {
  if (g.P <= 0 || g.batch <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0) return hipErrorInvalidValue;
  const int nout = (epi == EPI_SWIGLU) ? TN / 2 : TN;
  dim3 grid((g.M + TM - 1) / TM, (g.N + nout - 1) / nout, g.P * g.batch);
  switch (epi) {
    case EPI_QKV:
      if (g.head_dim > TN || TN % g.head_dim) return hipErrorInvalidValue;
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, grid, dim3(256), 0, st, g);
      break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, dim3(256), 0, st, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, st, g); break;
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, dim3(256), 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace armt
