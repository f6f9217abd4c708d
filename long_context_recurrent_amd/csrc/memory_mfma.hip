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
// Memory read fused with the attention RMSNorm, for 16 rows of one node:
//   q  = phi(h_in W_mq^T),  h = h_in + (q A^T) / (q . z + eps)   (fp32 stream)
//   a  = R(rms(h) * g_attn)                                       (bf16)
// Workgroup = (16 rows, node); wave w owns the column quarter
// [w d/4, (w+1) d/4) as 32-column blocks, and keeps its h values in registers
// from the first load to the last store.  Lane (c16, g) holds row c16 and, in
// block b, the columns 32b + 4g + {0..3} and 32b + 16 + 4g + {0..3} (slots
// 0..3 and 4..7): the MFMA output layout of a 16x16 block of r^T = A q^T, so
// r lands in the lane that holds h.  The same slot order is the k order of
// the first product (its weight operand is loaded in the same order).
//   * q A^T: both fp32 operands as bf16 pairs, three products
//     (A_hi q_hi + A_hi q_lo + A_lo q_hi), relative error ~2^-16.
//   * The four waves' partial h W_mq^T, and their partial sums of squares,
//     are added in LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int NBM>   // 32-column blocks per wave this instantiation can hold
__global__ __launch_bounds__(256) void memread_norm_bf16_kernel(MemArgs a) {
  __shared__ float ured[4][16][65];
  __shared__ float qs[16][68];
  __shared__ float dens[16];
  __shared__ float ssq[4][16];
  const int layer = a.l0 + blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int d = a.d, nb = d >> 7;
  const int row = blockIdx.x * 16 + c16;
  const int rowc = row < a.n ? row : a.n - 1;
  const int colw = w * (d >> 2) + 4 * g;     // + 32 b (+ 16 for slots 4..7)

  // h_in rows (fp32 stream, or bf16 x / memory embeddings at layer 0)
  float hv[NBM][8];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < nb) {
      const int c = colw + 32 * b;
      if (layer == 0) {
        const bf16* p = rowc < a.T ? (const bf16*)a.desc->x + ((int64_t)a.desc->c * a.T + rowc) * d
                                   : (const bf16*)a.mem_emb + (int64_t)(rowc - a.T) * d;
        const bf16x4 x0 = *(const bf16x4*)(p + c), x1 = *(const bf16x4*)(p + c + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) { hv[b][e] = (float)x0[e]; hv[b][4 + e] = (float)x1[e]; }
      } else {
        const float* p = (const float*)a.act_prev + (int64_t)(layer - 1) * a.act_stride + (int64_t)rowc * d;
        const f32x4 x0 = *(const f32x4*)(p + c), x1 = *(const f32x4*)(p + c + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) { hv[b][e] = x0[e]; hv[b][4 + e] = x1[e]; }
      }
    }
  }

  // u = h W_mq^T over this wave's columns: key block jb, lane key c16
  f32x4 u[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) u[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16* wq = (const bf16*)a.w_mq + (int64_t)layer * 64 * d;
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < nb) {
      bf16x8 hi, lo;
      split8(hv[b], hi, lo);
      const int c = colw + 32 * b;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const bf16* wr = wq + (int64_t)(16 * jb + c16) * d;
        const bf16x4 w0 = *(const bf16x4*)(wr + c), w1 = *(const bf16x4*)(wr + c + 16);
        const bf16x8 bv = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        u[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv, u[jb], 0, 0, 0);
        u[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv, u[jb], 0, 0, 0);
      }
    }
  }
  // lane (c16, g) of block jb holds u[row 4g + i][key 16 jb + c16]
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int i = 0; i < 4; ++i) ured[w][4 * g + i][16 * jb + c16] = u[jb][i];
  __syncthreads();
  for (int idx = tid; idx < 16 * 64; idx += 256) {
    const int r = idx >> 6, k = idx & 63;
    qs[r][k] = phi_f(((ured[0][r][k] + ured[1][r][k]) + ured[2][r][k]) + ured[3][r][k]);
  }
  __syncthreads();
  if (tid < 16) {
    const float* z = a.z + (int64_t)layer * 64;
    float sd = 0.f;
    for (int k = 0; k < 64; ++k) sd = fmaf(qs[tid][k], z[k], sd);
    dens[tid] = sd + a.mem_eps;
  }
  // q^T as the second operand of r^T = A q^T: lane (c16, g) brings
  // q[row c16][32 ks + 8 g .. + 7] as a bf16 pair
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = qs[c16][32 * ks + 8 * g + e];
    split8(v, qh[ks], ql[ks]);
  }
  __syncthreads();   // dens visible
  const float den = dens[c16];

  // h += r^T / den, block by block; partial sum of squares of the new h
  const float* Ast = a.A + (int64_t)layer * d * 64;
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < nb) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const float* ar = Ast + (int64_t)(w * (d >> 2) + 32 * b + 16 * sb + c16) * 64 + 8 * g;
        f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float av[8];
          load8f(ar + 32 * ks, av);
          bf16x8 ah, al;
          split8(av, ah, al);
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, qh[ks], r, 0, 0, 0);
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ql[ks], r, 0, 0, 0);
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, qh[ks], r, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float hn = hv[b][4 * sb + i] + r[i] / den;
          hv[b][4 * sb + i] = hn;
          ss = fmaf(hn, hn, ss);
        }
      }
    }
  }
  ss += __shfl_xor(ss, 16, kWave);
  ss += __shfl_xor(ss, 32, kWave);
  if (g == 0) ssq[w][c16] = ss;
  __syncthreads();
  const float rs = rsqrtf((((ssq[0][c16] + ssq[1][c16]) + ssq[2][c16]) + ssq[3][c16]) / (float)d + a.rms_eps);
  if (row < a.n) {
    float* ho = (float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)row * d;
    bf16* ao = (bf16*)a.abuf + (int64_t)layer * a.act_stride + (int64_t)row * d;
    const bf16* gn = (const bf16*)a.gain + (int64_t)layer * d;
#pragma unroll
    for (int b = 0; b < NBM; ++b) {
      if (b < nb) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int c = colw + 32 * b + 16 * sb;
          const float* v = &hv[b][4 * sb];
          *(f32x4*)(ho + c) = f32x4{v[0], v[1], v[2], v[3]};
          const bf16x4 gv = *(const bf16x4*)(gn + c);
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)(v[e] * rs * (float)gv[e]);
          *(bf16x4*)(ao + c) = o;
        }
      }
    }
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
    // waves take interleaved 64-wide k chunks; lane group g brings
    // k0 + 16g .. +15 (same slot order for both operands, as in memupdate)
    const bf16* wk = (const bf16*)a.w_mk + ((int64_t)layer * 64 + 16 * jb + c16) * d + 16 * g;
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 64 * w; k0 < d; k0 += 256) {
      const bf16x8 bv0 = *(const bf16x8*)(wk + k0), bv1 = *(const bf16x8*)(wk + k0 + 8);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < mblocks) {
          int m = 16 * mb + c16;
          m = m < M ? m : M - 1;
          float v[16];
          load8f(Y + (int64_t)m * d + k0 + 16 * g, v);
          load8f(Y + (int64_t)m * d + k0 + 16 * g + 8, v + 8);
          bf16x8 hi0, lo0, hi1, lo1;
          split8(v, hi0, lo0);
          split8(v + 8, hi1, lo1);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi0, bv0, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo0, bv0, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi1, bv1, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo1, bv1, acc[mb], 0, 0, 0);
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

  // k moves 64 per step: lane group g brings k0 + 16g .. +15 of its row (32
  // bytes of W_mv, a whole 128-byte line per row across the four groups) and
  // feeds them to two MFMAs (slots k0 + 16g + j, then k0 + 16g + 8 + j); the
  // Y operand uses the same slot order.
  const int mblocks = (M + 15) / 16;
  const bf16* wv = (const bf16*)a.w_mv + ((int64_t)layer * d + i0 + 16 * w + c16) * d + 16 * g;
  f32x4 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += 64) {
    const bf16x8 bv0 = *(const bf16x8*)(wv + k0), bv1 = *(const bf16x8*)(wv + k0 + 8);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < mblocks) {
        int m = 16 * mb + c16;
        m = m < M ? m : M - 1;
        float v[16];
        load8f(Y + (int64_t)m * d + k0 + 16 * g, v);
        load8f(Y + (int64_t)m * d + k0 + 16 * g + 8, v + 8);
        bf16x8 hi0, lo0, hi1, lo1;
        split8(v, hi0, lo0);
        split8(v + 8, hi1, lo1);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi0, bv0, acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo0, bv0, acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi1, bv1, acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo1, bv1, acc[mb], 0, 0, 0);
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
  // d / 4 columns per wave in 32-column blocks; up to 24 blocks held per wave
  if (m.dk != 64 || m.d % 128 || m.d > 3072) return hipErrorInvalidValue;
  const dim3 grid((m.n + 15) / 16, m.P);
  const int nb = m.d / 128;
  if (nb <= 4) hipLaunchKernelGGL(memread_norm_bf16_kernel<4>, grid, dim3(256), 0, st, m);
  else if (nb <= 8) hipLaunchKernelGGL(memread_norm_bf16_kernel<8>, grid, dim3(256), 0, st, m);
  else if (nb <= 16) hipLaunchKernelGGL(memread_norm_bf16_kernel<16>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(memread_norm_bf16_kernel<24>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_keys_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(memkeys_bf16_kernel, dim3(5, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_update_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(memupdate_bf16_kernel, dim3(m.d / 64, m.P), dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace armt
