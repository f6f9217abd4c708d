// Batched causal segment attention over the nodes of one wave: every node is
// one batch element and attends only over its own n = T + M rows (segment
// tokens, then memory tokens); query head j reads key/value head
// j / (H/G) (Pith review of arXiv 2506.05229, "What carries the argument":
// batched attention inside the grouped layer; Figure 5 caption: groups are
// treated as batches).
//
// bf16 path (flash-style, CDNA4 MFMA).  Workgroup = (64-query block, query
// head, node); each of its 4 waves owns 16 queries.  Key tiles of 64 rows and
// the matching V^T tile (V is stored transposed by the QKV GEMM) are staged in
// LDS and shared by the 4 waves.  Scores are computed transposed,
// S^T = K Q^T, with v_mfma_f32_16x16x32_bf16, so each lane holds 4 keys of one
// query: the probabilities then sit in registers exactly as the B operand of
// O^T = V^T P^T needs them (the two MFMA operands agree on which key each of a
// lane's 8 k-slots means), and the online-softmax rescale is one scalar per
// lane.  Row max and row sum over a tile need only two cross-lane exchanges
// (lanes 16 and 32 apart).  Softmax statistics are fp32; P enters the second
// product as a bf16 pair (hi + lo), so only the output O is rounded to bf16,
// as in the layer definition.  Query blocks are launched heaviest first.
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KP = HD + 8;    // K tile pitch (elements)
  constexpr int VP = 64 + 8;    // V^T tile pitch
  constexpr int ES = HD / 32;   // MFMA k-steps over the head dim
  constexpr int EB = HD / 16;   // 16-row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[HD * VP];

  const int n = a.n;
  const int nqb = (n + 63) / 64;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int h = blockIdx.y;
  const int layer = a.l0 + blockIdx.z;
  const int kvh = h / (a.H / a.G);
  const bf16* qkv = (const bf16*)a.qkv + (int64_t)layer * a.qkv_stride;
  const bf16* vt = (const bf16*)a.vt + (int64_t)layer * a.vt_stride + (int64_t)kvh * HD * a.vt_ld;
  const int kcol = (a.H + kvh) * HD;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int q = qb * 64 + 16 * w + c16;
  const int qrow = q < n ? q : n - 1;

  bf16x8 qf[ES];
#pragma unroll
  for (int es = 0; es < ES; ++es)
    qf[es] = *(const bf16x8*)(qkv + (int64_t)qrow * a.ld_qkv + h * HD + 32 * es + g * 8);

  f32x4 o[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) o[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;   // scores in log2 units

  for (int t = 0; t <= qb; ++t) {
    __syncthreads();
    for (int c = tid; c < 64 * (HD / 8); c += 256) {
      const int key = c / (HD / 8), ch = c % (HD / 8);
      int krow = t * 64 + key;
      krow = krow < n ? krow : n - 1;
      *(u32x4*)(Ks + key * KP + ch * 8) = *(const u32x4*)(qkv + (int64_t)krow * a.ld_qkv + kcol + ch * 8);
    }
    for (int c = tid; c < HD * 8; c += 256) {
      const int e = c >> 3, ch = c & 7;
      *(u32x4*)(Vs + e * VP + ch * 8) = *(const u32x4*)(vt + (int64_t)e * a.vt_ld + t * 64 + ch * 8);
    }
    __syncthreads();

    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int es = 0; es < ES; ++es) {
        const bf16x8 kf = *(const bf16x8*)(Ks + (kb * 16 + c16) * KP + 32 * es + g * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[es], s[kb], 0, 0, 0);
      }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t * 64 + kb * 16 + 4 * g + r;
        const float v = (key <= q) ? s[kb][r] * sl2 : -INFINITY;
        s[kb][r] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float mnew = fmaxf(mrun, mloc);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) o[eb] *= alpha;
    // P = P_hi + P_lo with both parts bf16: the two products together carry
    // P to about 16 significant bits, so P itself is never rounded to bf16.
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p0 = exp2f(s[2 * c][r] - mnew);
        const float p1 = exp2f(s[2 * c + 1][r] - mnew);
        lsum += p0 + p1;
        ph[c][r] = (bf16)p0;
        ph[c][4 + r] = (bf16)p1;
        pl[c][r] = (bf16)(p0 - (float)ph[c][r]);
        pl[c][4 + r] = (bf16)(p1 - (float)ph[c][4 + r]);
      }
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16* vrow = Vs + (eb * 16 + c16) * VP + c * 32 + 4 * g;
        const bf16x4 lo = *(const bf16x4*)vrow;
        const bf16x4 hi = *(const bf16x4*)(vrow + 16);
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph[c], o[eb], 0, 0, 0);
        o[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[c], o[eb], 0, 0, 0);
      }
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (q < n) {
    const float inv = 1.f / lsum;
    bf16* out = (bf16*)a.out + (int64_t)layer * a.out_stride + (int64_t)q * a.ld_out + h * HD;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16)(o[eb][r] * inv);
      *(bf16x4*)(out + eb * 16 + 4 * g) = v;
    }
  }
}

// fp32 path: one wave per query, lanes over keys for the scores and over the
// head dimension for the weighted sum.  Used for the small fp32 workloads.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float pbuf[];   // [4][n + 1]
  const int h = blockIdx.x, layer = a.l0 + blockIdx.y;
  const int kvh = h / (a.H / a.G), hd = a.hd, n = a.n;
  const float* qkv = (const float*)a.qkv + (int64_t)layer * a.qkv_stride;
  const int kcol = (a.H + kvh) * hd, vcol = (a.H + a.G + kvh) * hd;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* p = pbuf + w * (n + 1);
  float* out = (float*)a.out + (int64_t)layer * a.out_stride;
  // uniform trip count over query groups so every barrier is reached by all waves
  for (int q0 = 0; q0 < n; q0 += 4) {
    const int q = q0 + w;
    if (q < n) {
      const float* qv = qkv + (int64_t)q * a.ld_qkv + h * hd;
      float mx = -INFINITY;
      for (int k = lane; k <= q; k += 64) {
        const float* kv = qkv + (int64_t)k * a.ld_qkv + kcol;
        float sc = 0.f;
        for (int e = 0; e < hd; ++e) sc = fmaf(qv[e], kv[e], sc);
        sc *= a.scale;
        p[k] = sc;
        mx = fmaxf(mx, sc);
      }
      mx = wave_max(mx);
      float sum = 0.f;
      for (int k = lane; k <= q; k += 64) {
        const float e = __expf(p[k] - mx);
        p[k] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      p[n] = sum;  // slot past the keys (buffer holds n + 1 per wave)
    }
    __syncthreads();  // p[] written by one lane is read by all lanes of the wave
    if (q < n) {
      const float inv = 1.f / p[n];
      for (int e = lane; e < hd; e += 64) {
        float acc = 0.f;
        for (int k = 0; k <= q; ++k) acc = fmaf(p[k], qkv[(int64_t)k * a.ld_qkv + vcol + e], acc);
        out[(int64_t)q * a.ld_out + h * hd + e] = acc * inv;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_attention(const AttnArgs& a, bool use_bf16, hipStream_t st) {
  if (a.P <= 0 || a.n <= 0) return hipErrorInvalidValue;
  if (use_bf16) {
    dim3 grid((a.n + 63) / 64, a.H, a.P);
    switch (a.hd) {
      case 32: hipLaunchKernelGGL(attn_bf16_kernel<32>, grid, dim3(256), 0, st, a); break;
      case 64: hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st, a); break;
      case 128: hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (a.n > 4096) return hipErrorInvalidValue;
    dim3 grid(a.H, a.P);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 4 * (a.n + 1) * sizeof(float), st, a);
  }
  return hipGetLastError();
}

}  // namespace armt
