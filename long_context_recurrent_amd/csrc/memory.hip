// Associative-memory kernels of one wave, plus the RMSNorm that feeds the MLP.
//
// The pages name the memory (ARMT: per-layer associative memory updated once
// per segment, a fast-weight / delta-rule family; Pith review of arXiv
// 2506.05229, "What carries the argument" and its reference list) but print no
// equations.  The reading implemented here, per layer l with state
// A_l [d, d_k], z_l [d_k] (fp32) and phi(u) = elu(u) + 1:
//   read : q = phi(h W_mq^T);  h <- h + (q A^T) / (q . z + eps)
//   write: from the node's M memory-token output rows Y,
//          k = phi(Y W_mk^T), v = Y W_mv^T, beta = sigmoid(Y w_beta),
//          vbar = (k A^T) / (k . z + eps) against the pre-update state,
//          A += sum_m beta_m (v_m - vbar_m) k_m^T,  z += sum_m k_m.
// The state never leaves the GPU between waves (skill page "Diagonal Batching
// for Recurrent Memory Transformers", Practical Guidance: keep per-layer
// memory on the GPU, synchronise only at the end).
//
// These kernels are bound by HBM traffic and fp32 vector arithmetic, not by a
// dense contraction, so they use coalesced 16-byte loads and wave reductions
// rather than MFMA tiles.  Every sum runs in a fixed order (no atomics), so a
// node's result does not depend on how many nodes share the launch.
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

// 8 consecutive elements <-> fp32
__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
  *(bf16x8*)p = x;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void copy8(bf16* d, const bf16* s) { *(u32x4*)d = *(const u32x4*)s; }
__device__ __forceinline__ void copy8(float* d, const float* s) {
  *(f32x4*)d = *(const f32x4*)s;
  *(f32x4*)(d + 4) = *(const f32x4*)(s + 4);
}

constexpr int RB = 8;    // rows per memory-read workgroup

}  // namespace

// ---------------------------------------------------------------------------
// Memory read (fp32 workloads).  Workgroup = (8 rows, node).  Builds the
// node's input (layer 0: the segment's token rows from x, then the memory
// embeddings; deeper layers: the previous layer's output slot), reads the
// memory and writes h to this wave's slot.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mem_read_kernel(MemArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int d = a.d, dk = a.dk;
  T* hs = (T*)smem_raw;                                   // [RB][d]
  float* qs = (float*)(smem_raw + (size_t)RB * d * sizeof(T));   // [RB][64]
  float* dens = qs + RB * 64;                             // [RB]

  const int layer = a.l0 + blockIdx.y;          // (layer, sequence) problem
  const int wl = layer / a.batch;                // model layer
  const int r0 = blockIdx.x * RB;
  const int nr = min(RB, a.n - r0);
  const int tid = threadIdx.x;
  const int64_t slab = (int64_t)layer * a.act_stride;

  // (a) stage the input rows
  const int chunks = d / 8;
  for (int idx = tid; idx < RB * chunks; idx += 256) {
    const int r = idx / chunks, c8 = (idx % chunks) * 8;
    T* dst = hs + r * d + c8;
    if (r < nr) {
      const int row = r0 + r;
      const T* src;
      if (wl == 0) {
        const int s = a.desc->c;   // layer 0 works on segment c - 0
        const int ts = seg_tokens(a.desc, s, a.T);
        if (row < ts) {
          // at layer 0 the problem index is the sequence index
          src = (const T*)a.desc->x + ((int64_t)layer * a.desc->seq_rows + (int64_t)s * a.T + row) * d;
        } else if (row < ts + a.M) {
          src = (const T*)a.mem_emb + (int64_t)(row - ts) * d;
        } else {
          src = nullptr;             // padding row of a short last segment
        }
      } else {
        src = (const T*)a.act_prev + (int64_t)(layer - a.batch) * a.act_stride + (int64_t)row * d;
      }
      if (src) {
        copy8(dst, src + c8);
      } else {
        float zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        store8(dst, zero);
      }
    } else {
      float zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      store8(dst, zero);
    }
  }
  __syncthreads();

  // (b) q = phi(h W_mq^T): lane group of 4 per key column j, interleaved k
  {
    const int j = tid >> 2, kq = tid & 3;
    const T* wrow = (const T*)a.w_mq + ((int64_t)wl * dk + j) * d;
    float u[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) u[r] = 0.f;
    for (int k = kq * 8; k < d; k += 32) {
      float wv[8];
      load8(wrow + k, wv);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float hv[8];
        load8(hs + r * d + k, hv);
#pragma unroll
        for (int e = 0; e < 8; ++e) u[r] = fmaf(hv[e], wv[e], u[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      u[r] += __shfl_xor(u[r], 1, kWave);
      u[r] += __shfl_xor(u[r], 2, kWave);
    }
    if (kq == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) qs[r * 64 + j] = phi_f(u[r]);
    }
  }
  __syncthreads();

  // (c) denominators q . z + eps
  const float* z = a.z + (int64_t)layer * dk;
  if (tid < RB) {
    float s = 0.f;
    for (int j = 0; j < dk; ++j) s = fmaf(qs[tid * 64 + j], z[j], s);
    dens[tid] = s + a.mem_eps;
  }
  __syncthreads();

  // (d) h <- R(h + (q A^T) / den); one model coordinate i per lane
  const float* A = a.A + (int64_t)layer * d * dk;
  T* out = (T*)a.act_cur + slab;
  for (int i = tid; i < d; i += 256) {
    float num[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) num[r] = 0.f;
    const f32x4* arow = (const f32x4*)(A + (int64_t)i * dk);
    for (int j4 = 0; j4 < 16; ++j4) {
      const f32x4 av = arow[j4];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const f32x4 qv = *(const f32x4*)(qs + r * 64 + j4 * 4);
        num[r] = fmaf(qv[0], av[0], num[r]);
        num[r] = fmaf(qv[1], av[1], num[r]);
        num[r] = fmaf(qv[2], av[2], num[r]);
        num[r] = fmaf(qv[3], av[3], num[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < nr) {
        out[(int64_t)(r0 + r) * d + i] = from_f32<T>(to_f32(hs[r * d + i]) + num[r] / dens[r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm of this wave's slot (the fp32 residual stream) into abuf:
// a = R(rms(h) g), R the storage rounding of the workload dtype T.  One wave
// per row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(MemArgs a) {
  constexpr int MAXC = 8;   // d <= 8 * 8 * 64 = 4096
  const int layer = a.l0 + blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= a.n) return;
  const int d = a.d;
  const int64_t off = (int64_t)layer * a.act_stride + (int64_t)row * d;
  const float* h = (const float*)a.act_cur + off;     // residual stream: fp32
  float v[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int k = (c * 64 + lane) * 8;
    if (k < d) {
      load8(h + k, v[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[c][e], v[c][e], ss);
    }
  }
  ss = wave_sum(ss);
  const float rs = rsqrtf(ss / (float)d + a.rms_eps);
  const T* gain = (const T*)a.gain + (int64_t)(layer / a.batch) * d;
  T* o = (T*)a.abuf + off;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int k = (c * 64 + lane) * 8;
    if (k < d) {
      float gv[8], r[8];
      load8(gain + k, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = v[c][e] * rs * gv[e];
      store8(o + k, r);
    }
  }
}

// ---------------------------------------------------------------------------
// Memory write, part 1 (fp32 workloads).  Workgroup (jg < 4, node): keys
// k[:, 16jg .. 16jg+15] (wave w computes columns 16jg + 4w .. +3, lanes over
// d), the partial denominators sum_{j in group} k_mj z_j with the pre-update
// z, then z_j += sum_m k_mj for the group's own columns.  Workgroup jg = 4:
// the gates beta_m.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mem_keys_kernel(MemArgs a) {
  __shared__ float ks[64][16];
  const int layer = a.l0 + blockIdx.y;
  const int jg = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int d = a.d, M = a.M, dk = a.dk;
  const int wl = layer / a.batch;
  const int ts = seg_tokens(a.desc, a.desc->c - wl, a.T);      // memory rows start here
  if (jg == 0 && tid == 0) a.moff[layer] = ts;                 // for mem_update (next launch)
  const T* Y = (const T*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)ts * d;
  if (jg < 4) {
    for (int jj = 0; jj < 4; ++jj) {
      const int jl = 4 * w + jj, j = 16 * jg + jl;
      const T* wk = (const T*)a.w_mk + ((int64_t)wl * dk + j) * d;
      for (int m = 0; m < M; ++m) {
        float s = 0.f;
        for (int k = lane * 8; k < d; k += 512) {
          float yv[8], wv[8];
          load8(Y + (int64_t)m * d + k, yv);
          load8(wk + k, wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) s = fmaf(yv[e], wv[e], s);
        }
        s = wave_sum(s);
        if (lane == 0) ks[m][jl] = phi_f(s);
      }
    }
    __syncthreads();
    float* z = a.z + (int64_t)layer * dk + jg * 16;
    if (tid < M) {
      float pd = 0.f;
      for (int jj = 0; jj < 16; ++jj) {
        pd = fmaf(ks[tid][jj], z[jj], pd);
        a.kbuf[((int64_t)layer * M + tid) * dk + jg * 16 + jj] = ks[tid][jj];
      }
      a.pden[((int64_t)layer * M + tid) * 4 + jg] = pd;
    }
    __syncthreads();   // every read of the old z of this group is done
    if (tid < 16) {
      float s = 0.f;
      for (int m = 0; m < M; ++m) s += ks[m][tid];
      z[tid] = z[tid] + s;
    }
  } else {
    const T* wb = (const T*)a.w_beta + (int64_t)wl * d;
    for (int m = w; m < M; m += 4) {
      float s = 0.f;
      for (int k = lane * 8; k < d; k += 512) {
        float yv[8], wv[8];
        load8(Y + (int64_t)m * d + k, yv);
        load8(wb + k, wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(yv[e], wv[e], s);
      }
      s = wave_sum(s);
      if (lane == 0) a.beta[(int64_t)layer * M + m] = sigmoid_f(s);
    }
  }
}

// ---------------------------------------------------------------------------
// Memory write, part 2 (fp32 workloads).  Workgroup = (16 rows i of A, node): values
// v_m[i] = Y_m . W_mv[i] (one wave per 4 rows, lanes over d), retrieved values
// vbar_m[i] = (k_m . A[i]) / (sum of the partial denominators + eps), then
// A[i][j] += sum_m beta_m (v_m[i] - vbar_m[i]) k_mj.  Each A row is owned by
// one workgroup.  Optionally advances the wave counter (no kernel of this
// launch reads it).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mem_update_kernel(MemArgs a) {
  __shared__ float ks[64][64];
  __shared__ float betas[64], dens[64];
  __shared__ float vv[64][16];
  __shared__ float delta[64][16];
  const int layer = a.l0 + blockIdx.y;
  const int i0 = blockIdx.x * 16;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int d = a.d, M = a.M, dk = a.dk;
  // memory rows' offset from mem_keys (this kernel advances the wave counter,
  // so it must not derive the segment from it)
  const T* Y = (const T*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)a.moff[layer] * d;

  for (int idx = tid; idx < M * dk; idx += 256)
    ks[idx / dk][idx % dk] = a.kbuf[(int64_t)layer * M * dk + idx];
  if (tid < M) {
    betas[tid] = a.beta[(int64_t)layer * M + tid];
    const float* pd = a.pden + ((int64_t)layer * M + tid) * 4;
    dens[tid] = ((pd[0] + pd[1]) + (pd[2] + pd[3])) + a.mem_eps;
  }

  // v_m[i] for the wave's 4 rows, memory tokens in chunks of 16
  const T* wv_base = (const T*)a.w_mv + (int64_t)(layer / a.batch) * d * d;
  for (int mc = 0; mc < M; mc += 16) {
    float acc[16][4];
#pragma unroll
    for (int mm = 0; mm < 16; ++mm)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) acc[mm][ii] = 0.f;
    for (int k = lane * 8; k < d; k += 512) {
      float wv[4][8];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) load8(wv_base + (int64_t)(i0 + 4 * w + ii) * d + k, wv[ii]);
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) {
        if (mc + mm < M) {
          float yv[8];
          load8(Y + (int64_t)(mc + mm) * d + k, yv);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[mm][ii] = fmaf(yv[e], wv[ii][e], acc[mm][ii]);
        }
      }
    }
#pragma unroll
    for (int mm = 0; mm < 16; ++mm)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float s = wave_sum(acc[mm][ii]);
        if (lane == 0 && mc + mm < M) vv[mc + mm][4 * w + ii] = s;
      }
  }
  __syncthreads();

  const float* A = a.A + (int64_t)layer * d * dk;
  for (int idx = tid; idx < M * 16; idx += 256) {
    const int m = idx >> 4, ii = idx & 15;
    const float* arow = A + (int64_t)(i0 + ii) * dk;
    float s = 0.f;
    for (int j = 0; j < dk; ++j) s = fmaf(ks[m][j], arow[j], s);
    delta[m][ii] = betas[m] * (vv[m][ii] - s / dens[m]);
  }
  __syncthreads();   // all reads of the old A rows are done
  float* Aw = a.A + (int64_t)layer * d * dk;
  for (int idx = tid; idx < 16 * dk; idx += 256) {
    const int ii = idx / dk, j = idx % dk;
    float s = 0.f;
    for (int m = 0; m < M; ++m) s = fmaf(delta[m][ii], ks[m][j], s);
    float* dst = Aw + (int64_t)(i0 + ii) * dk + j;
    *dst = *dst + s;
  }
  if (a.advance != 0 && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.desc->c += a.advance;
}

// ---------------------------------------------------------------------------
__global__ void set_desc_kernel(CallDesc* desc, const void* x, void* y, int c0, int S, int t_last,
                                int64_t seq_rows) {
  desc->x = x;
  desc->y = y;
  desc->seq_rows = seq_rows;
  desc->c = c0;
  desc->n_segments = S;
  desc->t_last = t_last;
}

__global__ void fill_f32_kernel(float* dst, const float* src, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
hipError_t launch_mem_read(const MemArgs& m, bool use_bf16, hipStream_t st) {
  if (m.P <= 0 || m.batch <= 0 || m.l0 < 0) return hipErrorInvalidValue;
  if (use_bf16) return launch_mem_read_bf16(m, st);
  const size_t lds = (size_t)RB * m.d * sizeof(float) + (RB * 64 + RB) * sizeof(float);
  if (lds > 64 * 1024 || m.dk != 64 || m.d % 8) return hipErrorInvalidValue;
  dim3 grid((m.n + RB - 1) / RB, m.P);
  hipLaunchKernelGGL(mem_read_kernel<float>, grid, dim3(256), lds, st, m);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const MemArgs& m, bool use_bf16, hipStream_t st) {
  if (m.P <= 0 || m.batch <= 0 || m.l0 < 0) return hipErrorInvalidValue;
  if (m.d > 4096 || m.d % 8) return hipErrorInvalidValue;
  dim3 grid((m.n + 3) / 4, m.P);
  if (use_bf16) hipLaunchKernelGGL(rmsnorm_kernel<bf16>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_keys(const MemArgs& m, bool use_bf16, hipStream_t st) {
  if (m.P <= 0 || m.batch <= 0 || m.l0 < 0) return hipErrorInvalidValue;
  if (use_bf16) return launch_mem_keys_bf16(m, st);
  if (m.dk != 64 || m.M > 64 || m.d % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mem_keys_kernel<float>, dim3(5, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_update(const MemArgs& m, bool use_bf16, hipStream_t st) {
  if (m.P <= 0 || m.batch <= 0 || m.l0 < 0) return hipErrorInvalidValue;
  if (use_bf16) return launch_mem_update_bf16(m, st);
  if (m.dk != 64 || m.M > 64 || m.d % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mem_update_kernel<float>, dim3(m.d / 16, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_set_desc(CallDesc* desc, const void* x, void* y, int c0, int S, int t_last, int64_t seq_rows,
                           hipStream_t st) {
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, st, desc, x, y, c0, S, t_last, seq_rows);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* dst, const float* src, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, dst, src, count);
  return hipGetLastError();
}

}  // namespace armt
