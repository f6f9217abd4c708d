// Associative-memory kernels for bf16 workloads, on CDNA4 matrix cores.
//
// Same reading of the ARMT memory as the fp32 kernels (see memory.hip):
//   read : q = phi(h W_mq^T);  h <- h + (q A^T) / (q . z + eps)
//   write: k = phi(Y W_mk^T), v = Y W_mv^T, beta = sigmoid(Y w_beta),
//          vbar = (k A^T) / (k . z + eps) against the pre-update state,
//          A += sum_m beta_m (v_m - vbar_m) k_m^T,  z += sum_m k_m
// (the pages name the memory -- ARMT, a delta-rule fast-weight memory, Pith
// review of arXiv 2506.05229 and its reference list -- but print no
// equations).
//
// h and Y belong to the residual stream, which is fp32 (bf16 only for the
// layer-0 inputs x and the memory embeddings).  Their products with the bf16
// weights (h W_mq^T, Y W_mk^T, Y W_mv^T) run on v_mfma_f32_16x16x32_bf16 with
// each fp32 operand split into a bf16 pair, v = hi + lo (hi = R(v),
// lo = R(v - hi), |v - hi - lo| <= 2^-17 |v|), so the stream enters the
// products without being rounded to bf16; accumulation is fp32.  The product with the fp32 state (q A^T) uses the fp32 matrix
// instruction v_mfma_f32_16x16x4_f32, so the state is never rounded.  The
// small state updates stay on the vector ALU.  All sums have a fixed order.
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

__device__ __forceinline__ void load8f(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}

// Elements col..col+7 of row `row` of the node input h_in as fp32.  Layer 0:
// the segment's token rows of the caller's x, then the memory embeddings
// (bf16); deeper layers: the previous layer's fp32 output in the other slot.
__device__ __forceinline__ void input8(const MemArgs& a, int layer, int row, int col, float* v) {
  if (layer == 0) {
    const bf16* p = row < a.T ? (const bf16*)a.desc->x + ((int64_t)a.desc->c * a.T + row) * a.d
                              : (const bf16*)a.mem_emb + (int64_t)(row - a.T) * a.d;
    const bf16x8 x = *(const bf16x8*)(p + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  } else {
    load8f((const float*)a.act_prev + (int64_t)(layer - 1) * a.act_stride + (int64_t)row * a.d + col, v);
  }
}

// v = hi + lo with both parts bf16 (hi = R(v), lo = R(v - hi)).
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)v[e];
    lo[e] = (bf16)(v[e] - (float)hi[e]);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// q = phi(h_in W_mq^T) -> qbuf [L][n][64] fp32.  Workgroup = (64 rows, node);
// wave w owns rows 16w..16w+15 and all 64 key columns (4 MFMA blocks).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void memq_bf16_kernel(MemArgs a) {
  const int layer = a.l0 + blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int row = blockIdx.x * 64 + 16 * w + c16;
  const int rowc = row < a.n ? row : a.n - 1;
  const bf16* wq = (const bf16*)a.w_mq + ((int64_t)layer * 64 + c16) * a.d + 8 * g;
  const int64_t jstride = (int64_t)16 * a.d;
  f32x4 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < a.d; k0 += 32) {
    float v[8];
    input8(a, layer, rowc, k0 + 8 * g, v);
    bf16x8 hi, lo;
    split8(v, hi, lo);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const bf16x8 bv = *(const bf16x8*)(wq + jb * jstride + k0);
      acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv, acc[jb], 0, 0, 0);
      acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv, acc[jb], 0, 0, 0);
    }
  }
  // lane holds rows 4g + r of the wave's 16, column c16 of each block
  float* q = a.qbuf + (int64_t)layer * a.n * 64;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = blockIdx.x * 64 + 16 * w + 4 * g + r;
    if (rr < a.n) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) q[(int64_t)rr * 64 + jb * 16 + c16] = phi_f(acc[jb][r]);
    }
  }
}

// ---------------------------------------------------------------------------
// h = h_in + (q A^T) / (q . z + eps) (fp32) for a 64-row x 256-column tile.
// q and the A rows of the tile are staged in LDS; wave w computes rows
// 16w..16w+15 x 256 columns with v_mfma_f32_16x16x4_f32.  Lane (c16, g) feeds
// key indices 16g + ks at step ks, so its 16 values per row are one
// contiguous 64-byte run (four 16-byte LDS reads; a 68-float pitch makes them
// conflict-free).  The result is staged in LDS and written with coalesced
// 16-byte stores.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void memapply_bf16_kernel(MemArgs a) {
  constexpr int QP = 68;            // q / A tile pitch (floats)
  constexpr int SP = 256 + 4;       // staging pitch
  __shared__ __attribute__((aligned(16))) float qs[64 * QP];
  __shared__ __attribute__((aligned(16))) float big[256 * QP];   // A tile, then staging
  __shared__ float dens[64];
  static_assert(64 * SP <= 256 * QP, "staging fits");

  const int layer = a.l0 + blockIdx.z;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 256;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int d = a.d;

  const float* qsrc = a.qbuf + (int64_t)layer * a.n * 64;
  for (int idx = tid; idx < 64 * 16; idx += 256) {
    const int r = idx >> 4, c4 = (idx & 15) * 4;
    const int rr = r0 + r < a.n ? r0 + r : a.n - 1;
    *(f32x4*)(qs + r * QP + c4) = *(const f32x4*)(qsrc + (int64_t)rr * 64 + c4);
  }
  const float* A = a.A + (int64_t)layer * d * 64;
  for (int idx = tid; idx < 256 * 16; idx += 256) {
    const int i = idx >> 4, c4 = (idx & 15) * 4;
    const int ii = c0 + i < d ? c0 + i : d - 1;
    *(f32x4*)(big + i * QP + c4) = *(const f32x4*)(A + (int64_t)ii * 64 + c4);
  }
  __syncthreads();
  if (tid < 64) {
    const float* z = a.z + (int64_t)layer * 64;
    float s = 0.f;
    for (int j = 0; j < 64; ++j) s = fmaf(qs[tid * QP + j], z[j], s);
    dens[tid] = s + a.mem_eps;
  }

  float qa[16];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const f32x4 t = *(const f32x4*)(qs + (16 * w + c16) * QP + 16 * g + 4 * v);
#pragma unroll
    for (int e = 0; e < 4; ++e) qa[4 * v + e] = t[e];
  }
  f32x4 acc[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
    float bb[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 t = *(const f32x4*)(big + (16 * cb + c16) * QP + 16 * g + 4 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) bb[4 * v + e] = t[e];
    }
    f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[ks], bb[ks], c, 0, 0, 0);
    acc[cb] = c;
  }
  __syncthreads();   // A tile no longer needed; dens visible
  float* st = big;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = 16 * w + 4 * g + r;
      st[rl * SP + 16 * cb + c16] = acc[cb][r] / dens[rl];
    }
  __syncthreads();
  float* out = (float*)a.act_cur + (int64_t)layer * a.act_stride;
  for (int idx = tid; idx < 64 * 32; idx += 256) {
    const int r = idx >> 5, c8 = (idx & 31) * 8;
    const int row = r0 + r, col = c0 + c8;
    if (row >= a.n || col >= d) continue;
    float o[8];
    input8(a, layer, row, col, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += st[r * SP + c8 + e];
    float* dst = out + (int64_t)row * d + col;
    *(f32x4*)dst = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4*)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// ---------------------------------------------------------------------------
// Memory write, part 1.  Workgroup (jb < 4, node): keys k[:, 16jb .. 16jb+15]
// = phi(Y W_mk^T) with the 4 waves splitting d (interleaved 32-wide steps) and
// a fixed-order reduction in LDS; then the partial denominators
// sum_{j in block} k_mj z_j with the pre-update z, and z_j += sum_m k_mj for
// the block's own columns.  Workgroup jb = 4: the gates beta_m.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void memkeys_bf16_kernel(MemArgs a) {
  __shared__ float red[4][4][64][4];   // [wave][m-block][lane][r]
  __shared__ float ks[64][17];
  const int layer = a.l0 + blockIdx.y;
  const int jb = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int d = a.d, M = a.M;
  const float* Y = (const float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)a.T * d;
  if (jb < 4) {
    const int mblocks = (M + 15) / 16;
    const bf16* wk = (const bf16*)a.w_mk + ((int64_t)layer * 64 + 16 * jb + c16) * d + 8 * g;
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 32 * w; k0 < d; k0 += 128) {
      const bf16x8 bv = *(const bf16x8*)(wk + k0);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < mblocks) {
          int m = 16 * mb + c16;
          m = m < M ? m : M - 1;
          float v[8];
          load8f(Y + (int64_t)m * d + k0 + 8 * g, v);
          bf16x8 hi, lo;
          split8(v, hi, lo);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv, acc[mb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][mb][lane][r] = acc[mb][r];
    __syncthreads();
    // lane (c16, g) of block mb holds rows m = 16mb + 4g + r, column c16
    for (int idx = tid; idx < mblocks * 64 * 4; idx += 256) {
      const int mb = idx / 256, ln = (idx / 4) % 64, r = idx % 4;
      const int m = 16 * mb + 4 * (ln >> 4) + r;
      const float s = red[0][mb][ln][r] + red[1][mb][ln][r] + red[2][mb][ln][r] + red[3][mb][ln][r];
      if (m < M) ks[m][ln & 15] = phi_f(s);
    }
    __syncthreads();
    float* z = a.z + (int64_t)layer * 64 + 16 * jb;
    if (tid < M) {
      float pd = 0.f;
      for (int jj = 0; jj < 16; ++jj) {
        pd = fmaf(ks[tid][jj], z[jj], pd);
        a.kbuf[((int64_t)layer * M + tid) * 64 + 16 * jb + jj] = ks[tid][jj];
      }
      a.pden[((int64_t)layer * M + tid) * 4 + jb] = pd;
    }
    __syncthreads();   // every read of this block's old z is done
    if (tid < 16) {
      float s = 0.f;
      for (int m = 0; m < M; ++m) s += ks[m][tid];
      z[tid] = z[tid] + s;
    }
  } else {
    const bf16* wb = (const bf16*)a.w_beta + (int64_t)layer * d;
    for (int m = w; m < M; m += 4) {
      float s = 0.f;
      for (int k = lane * 8; k < d; k += 512) {
        float yv[8];
        load8f(Y + (int64_t)m * d + k, yv);
        const bf16x8 wv = *(const bf16x8*)(wb + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(yv[e], (float)wv[e], s);
      }
      s = wave_sum(s);
      if (lane == 0) a.beta[(int64_t)layer * M + m] = sigmoid_f(s);
    }
  }
}

// ---------------------------------------------------------------------------
// Memory write, part 2.  Workgroup = (64 rows i of A, node).  v_m[i] =
// Y_m . W_mv[i] on MFMA (wave w: rows i0 + 16w .. +15), then with the A tile
// staged in LDS: vbar_m[i] = (k_m . A[i]) / (sum of partial denominators +
// eps), delta_m[i] = beta_m (v_m[i] - vbar_m[i]), A[i][j] += sum_m delta_m[i]
// k_mj.  W_mv is read exactly once per node.  Optionally advances the wave
// counter (no kernel of this launch reads it).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void memupdate_bf16_kernel(MemArgs a) {
  constexpr int P65 = 65;
  __shared__ float ks[64][64];
  __shared__ float betas[64], dens[64];
  __shared__ float vvs[64][P65];
  __shared__ float At[64][P65];
  __shared__ float delta[64][P65];
  const int layer = a.l0 + blockIdx.y;
  const int i0 = blockIdx.x * 64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int d = a.d, M = a.M;
  const float* Y = (const float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)a.T * d;
  float* A = a.A + (int64_t)layer * d * 64;

  for (int idx = tid; idx < M * 64; idx += 256) ks[idx >> 6][idx & 63] = a.kbuf[(int64_t)layer * M * 64 + idx];
  if (tid < M) {
    betas[tid] = a.beta[(int64_t)layer * M + tid];
    const float* pd = a.pden + ((int64_t)layer * M + tid) * 4;
    dens[tid] = ((pd[0] + pd[1]) + (pd[2] + pd[3])) + a.mem_eps;
  }
  for (int idx = tid; idx < 64 * 16; idx += 256) {
    const int i = idx >> 4, c4 = (idx & 15) * 4;
    const f32x4 t = *(const f32x4*)(A + (int64_t)(i0 + i) * 64 + c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) At[i][c4 + e] = t[e];
  }

  const int mblocks = (M + 15) / 16;
  const bf16* wv = (const bf16*)a.w_mv + ((int64_t)layer * d + i0 + 16 * w + c16) * d + 8 * g;
  f32x4 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = 0; k0 < d; k0 += 32) {
    const bf16x8 bv = *(const bf16x8*)(wv + k0);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < mblocks) {
        int m = 16 * mb + c16;
        m = m < M ? m : M - 1;
        float v[8];
        load8f(Y + (int64_t)m * d + k0 + 8 * g, v);
        bf16x8 hi, lo;
        split8(v, hi, lo);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv, acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv, acc[mb], 0, 0, 0);
      }
    }
  }
  // lane holds v[m = 16mb + 4g + r][i = i0 + 16w + c16]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mb + 4 * g + r;
      if (mb < mblocks && m < M) vvs[m][16 * w + c16] = acc[mb][r];
    }
  __syncthreads();
  for (int idx = tid; idx < M * 64; idx += 256) {
    const int m = idx >> 6, ii = idx & 63;
    float s = 0.f;
#pragma unroll 8
    for (int j = 0; j < 64; ++j) s = fmaf(ks[m][j], At[ii][j], s);
    delta[m][ii] = betas[m] * (vvs[m][ii] - s / dens[m]);
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int ii = idx >> 6, j = idx & 63;
    float s = 0.f;
    for (int m = 0; m < M; ++m) s = fmaf(delta[m][ii], ks[m][j], s);
    A[(int64_t)(i0 + ii) * 64 + j] = At[ii][j] + s;
  }
  if (a.advance != 0 && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.desc->c += a.advance;
}

// ---------------------------------------------------------------------------
hipError_t launch_mem_read_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(memq_bf16_kernel, dim3((m.n + 63) / 64, m.P), dim3(256), 0, st, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(memapply_bf16_kernel, dim3((m.n + 63) / 64, (m.d + 255) / 256, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_keys_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(memkeys_bf16_kernel, dim3(5, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_update_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(memupdate_bf16_kernel, dim3(m.d / 64, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace armt
