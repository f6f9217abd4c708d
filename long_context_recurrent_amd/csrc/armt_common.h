// Shared device helpers and the launch-parameter structs of the ARMT kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace armt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- element conversions (round to nearest even on the way to bf16) ----
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// phi(u) = elu(u) + 1
__device__ __forceinline__ float phi_f(float u) { return u > 0.f ? u + 1.f : __expf(u); }
// sigmoid with the hardware reciprocal (about 1 ulp; an IEEE division costs
// ten instructions per element in the SwiGLU epilogue).  exp(-u) = inf gives 0.
__device__ __forceinline__ float sigmoid_f(float u) { return __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

// Per-call descriptor shared by the kernels of one forward: the caller's
// input/output pointers and the running wave counter c.  In wave c the node
// of layer l works on segment s = c - l.  Kept in device memory so captured
// graphs can be replayed for any call and any wave of the same shape.
struct CallDesc {
  const void* x;     // [B][(S-1)*T + t_last][d]
  void* y;           // same layout as x
  int64_t seq_rows;  // rows of one sequence in x and y ((S-1)*T + t_last)
  int32_t c;         // current wave (diagonal) or s + l (sequential)
  int32_t n_segments;
  int32_t t_last;    // tokens of the last segment (1..T)
};

// Tokens of segment s: T, except a shorter last segment.  The node keeps its
// n = T + M rows; a short segment's memory tokens follow its t tokens and the
// rows after them are padding no real row attends to.
__device__ __forceinline__ int seg_tokens(const CallDesc* d, int s, int T) {
  return s == d->n_segments - 1 ? d->t_last : T;
}

// ---- wave reductions -------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace armt
