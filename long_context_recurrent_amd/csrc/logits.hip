// Kernels outside the recurrent node.
//
// Final RMSNorm ahead of the LM head.  The logits that follow it are what the
// pages compare between the sequential and the diagonal schedule (Pith review
// of arXiv 2506.05229: falsifier, and the referee report on the relative
// logit drift of Table 2).  The LM-head product itself is the plain-store
// epilogue of the GEMM kernels (fp32 logits).  One wave per row: the lane
// holds 8-element pieces c * 512 + 8 * lane of the row in registers from load
// to store; the sum of squares goes lane-local in piece order, then across
// the wave.
//
// Stream initialisation of the full-attention comparator: the input rows,
// widened to the fp32 residual stream.
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

__device__ __forceinline__ void ld8(const bf16* p, float* v) {
  const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void ld8(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}
__device__ __forceinline__ void st8(bf16* p, const float* v) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
  *(bf16x8*)p = x;
}
__device__ __forceinline__ void st8(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

constexpr int kMaxPieces = 8;   // d <= 8 * 64 * 8 = 4096

template <typename T>
__global__ __launch_bounds__(256) void final_norm_kernel(NormArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= a.rows) return;
  const int d = a.d;
  const T* x = (const T*)a.x + (int64_t)row * d;
  float v[kMaxPieces][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxPieces; ++c) {
    const int k = (c * 64 + lane) * 8;
    if (k < d) {
      ld8(x + k, v[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[c][e], v[c][e], ss);
    }
  }
  ss = wave_sum(ss);
  const float rs = rsqrtf(ss / (float)d + a.eps);
  const T* gain = (const T*)a.gain;
  T* o = (T*)a.out + (int64_t)row * d;
#pragma unroll
  for (int c = 0; c < kMaxPieces; ++c) {
    const int k = (c * 64 + lane) * 8;
    if (k < d) {
      float gv[8], r[8];
      ld8(gain + k, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = v[c][e] * rs * gv[e];
      st8(o + k, r);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void widen_kernel(const T* __restrict__ src, float* __restrict__ dst,
                                                    int64_t count8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count8) return;
  float v[8];
  ld8(src + 8 * i, v);
  st8(dst + 8 * i, v);
}

}  // namespace

hipError_t launch_widen(const void* src, float* dst, int64_t count, bool use_bf16, hipStream_t st) {
  if (count <= 0 || count % 8) return hipErrorInvalidValue;
  const int64_t c8 = count / 8;
  const dim3 grid((unsigned)((c8 + 255) / 256));
  if (use_bf16) hipLaunchKernelGGL(widen_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)src, dst, c8);
  else hipLaunchKernelGGL(widen_kernel<float>, grid, dim3(256), 0, st, (const float*)src, dst, c8);
  return hipGetLastError();
}

hipError_t launch_final_norm(const NormArgs& a, bool use_bf16, hipStream_t st) {
  if (a.rows <= 0 || a.d <= 0 || a.d % 8 || a.d > kMaxPieces * 64 * 8) return hipErrorInvalidValue;
  const dim3 grid((a.rows + 3) / 4);
  if (use_bf16) hipLaunchKernelGGL(final_norm_kernel<bf16>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(final_norm_kernel<float>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace armt
