// Batched causal segment attention over the nodes of one wave: every node is
// one batch element and attends only over its own n = T + M rows (segment
// tokens, then memory tokens); query head j reads key/value head
// j / (H/G) (Pith review of arXiv 2506.05229, "What carries the argument":
// batched attention inside the grouped layer; Figure 5 caption: groups are
// treated as batches).
//
// bf16 path (flash-style, CDNA4 MFMA).  Workgroup = (128-query block, query
// head, node); each of its 4 waves owns 32 queries.  Key tiles of 64 rows
// and the matching V^T tiles (V is stored transposed by the QKV GEMM) stream
// into LDS through global->LDS DMA loads, several tiles ahead, and are shared
// by the 4 waves.  Both products run on v_mfma_f32_32x32x16_bf16:
//  * S^T = K Q^T, so lane (r32, h) holds 16 keys of query r32 per 32-key
//    block and the online-softmax statistics are per lane (one exchange with
//    the lane 32 apart);
//  * O^T = V^T P^T, with P taken straight from the S^T registers as the
//    second operand.  A lane's 8 k-slots then name keys 4h..4h+3 and
//    8+4h..8+4h+3 of a 16-key group, so V^T keeps the keys of every aligned
//    group of 16 in the order 0-3, 8-11, 4-7, 12-15: each lane's V^T operand
//    is one 16-byte read.
// Softmax statistics and the row sums are fp32; P enters the second product
// rounded to bf16 (the usual flash-attention practice; a bf16 hi + lo pair
// would keep P exact at the cost of 8 more MFMAs and 64 more VALU operations
// per 64-key tile, which made this kernel 30% slower for a 5% smaller error
// at depth), and O is rounded to bf16 once at the end.  Tile rows keep their 16-byte chunks XOR-swizzled so the
// fragment reads are free of bank conflicts.  Query blocks are launched
// heaviest first.
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Physical 16-byte chunk of logical chunk c in row r of a tile whose rows
// hold CH chunks: the same logical chunk of 8 (and of 16) consecutive rows
// falls in distinct bank groups.
template <int CH>
__device__ __forceinline__ int swzc(int r, int c) {
  if (CH == 4) return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
  if (CH == 8) return c ^ ((r ^ (r >> 3)) & 7);
  return c ^ (r & 15);
}

// s_waitcnt immediate: vmcnt <= n, lgkmcnt = 0, expcnt free
__host__ __device__ constexpr int att_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

__device__ __forceinline__ void att_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = HD / 8;                  // 16-byte chunks per K row
  constexpr int K_BYTES = 64 * HD * 2;        // K tile: 64 keys x HD
  constexpr int V_BYTES = HD * 64 * 2;        // V^T tile: HD rows x 64 keys
  constexpr int TILE = K_BYTES + V_BYTES;
  constexpr int NBUF = HD >= 128 ? 2 : 3;
  constexpr int K_BLOCKS = K_BYTES / 1024;    // 1 KB wave loads per tile
  constexpr int LOADS = (TILE / 1024) / 4;    // per wave per tile
  constexpr int KROWS = 1024 / (HD * 2);      // K rows per 1 KB load
  constexpr int ES = HD / 16, DB = HD / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * TILE];

  const int n = a.n;
  const int nqb = (n + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int head = blockIdx.y;
  const int layer = a.l0 + blockIdx.z;
  const int kvh = head / (a.H / a.G);
  const bf16* qkv = (const bf16*)a.qkv + (int64_t)layer * a.qkv_stride;
  const bf16* vt = (const bf16*)a.vt + (int64_t)layer * a.vt_stride + (int64_t)kvh * HD * a.vt_ld;
  const int kcol = (a.H + kvh) * HD;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r32 = lane & 31, hh = lane >> 5;
  const int q0w = qb * 128 + 32 * w;
  const int q = q0w + r32;
  const int qc = q < n ? q : n - 1;
  const int q_end = (qb + 1) * 128 < n ? (qb + 1) * 128 : n;
  const int ntile = (q_end + 63) / 64;
  const int wq_end = q0w + 32 < n ? q0w + 32 : n;
  const int wtiles = wq_end > q0w ? (wq_end + 63) / 64 : 0;

  // DMA slots: 1 KB block b = w + 4t of a tile; K blocks first, then V^T
  int roff[LOADS], coff[LOADS], dst[LOADS];
#pragma unroll
  for (int t = 0; t < LOADS; ++t) {
    const int b = w + 4 * t;
    dst[t] = b * 1024;
    if (b < K_BLOCKS) {
      const int r = b * KROWS + lane / CH;           // key row in the tile
      roff[t] = r;
      coff[t] = kcol + swzc<CH>(r, lane % CH) * 8;
    } else {
      const int dim = (b - K_BLOCKS) * 8 + lane / 8;   // V^T row
      roff[t] = dim;
      coff[t] = swzc<8>(dim, lane % 8) * 8;
    }
  }
  auto issue = [&](int t) {
    const int tt = t < ntile ? t : ntile - 1;
    unsigned char* st = smem + (t % NBUF) * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int b = w + 4 * i;
      const bf16* src;
      if (b < K_BLOCKS) {
        int row = tt * 64 + roff[i];
        row = row < n ? row : n - 1;
        src = qkv + (int64_t)row * a.ld_qkv + coff[i];
      } else {
        src = vt + (int64_t)roff[i] * a.vt_ld + tt * 64 + coff[i];
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(st + dst[i]),
                                       16, 0, 0);
    }
  };

#pragma unroll
  for (int s = 0; s < NBUF - 1; ++s) issue(s);

  bf16x8 qf[ES];
#pragma unroll
  for (int ks = 0; ks < ES; ++ks)
    qf[ks] = *(const bf16x8*)(qkv + (int64_t)qc * a.ld_qkv + head * HD + 16 * ks + 8 * hh);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float mrun = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;   // scores in log2 units

  for (int t = 0; t < ntile; ++t) {
    // tile t landed (this wave's loads; the barrier covers the others'),
    // and every wave is done with tile t - 1, whose buffer is refilled next
    __builtin_amdgcn_s_waitcnt(att_wait((NBUF - 2) * LOADS));
    att_barrier();
    issue(t + NBUF - 1);
    if (t >= wtiles) continue;
    const unsigned char* kt = smem + (t % NBUF) * TILE;
    const unsigned char* vtile = kt + K_BYTES;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < ES; ++ks) {
        const int r = kb * 32 + r32;
        const bf16x8 kf = *(const bf16x8*)(kt + r * (HD * 2) + swzc<CH>(r, 2 * ks + hh) * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // element e of block kb: key t*64 + 32kb + 8(e/4) + 4hh + e%4, query q.
    // Only tiles that reach past the wave's first query need the causal mask.
    float mloc = -INFINITY;
    if (t * 64 + 63 > q0w) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * 64 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key > q) s[kb][e] = -INFINITY;
          mloc = fmaxf(mloc, s[kb][e]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, s[kb][e]);
    }
    // running max in raw score units; p = 2^(s * sl2 - m * sl2) (sl2 > 0)
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float mnew = fmaxf(mrun, mloc);
    // rescale the running sums only when some lane's maximum grew
    if (__any(mnew > mrun)) {
      const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float mb = mnew * sl2;
    mrun = mnew;
    // P as the second operand of O^T = V^T P^T: 16-key group G = 2kb + ks,
    // slot j = element 8ks + j of block kb
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x8 pv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * ks + j], sl2, -mb));
          lsum += pv[j];
        }
        const bf16x8 ph = __builtin_convertvector(pv, bf16x8);
        const int c = 2 * (2 * kb + ks) + hh;    // logical chunk of the V^T row
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int r = db * 32 + r32;
          const bf16x8 vf = *(const bf16x8*)(vtile + r * 128 + swzc<8>(r, c) * 16);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph, o[db], 0, 0, 0);
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(att_wait(0));
  lsum += __shfl_xor(lsum, 32, kWave);
  if (q < n) {
    const float inv = 1.f / lsum;
    bf16* out = (bf16*)a.out + (int64_t)layer * a.out_stride + (int64_t)q * a.ld_out + head * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[db][4 * g4 + e] * inv);
        *(bf16x4*)(out + db * 32 + 8 * g4 + 4 * hh) = v;
      }
  }
}

// fp32 path: one wave per query (4 queries per workgroup), lanes over keys
// for the scores and over the head dimension for the weighted sum.  Used for
// the small fp32 workloads.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float pbuf[];   // [4][n + 1]
  const int h = blockIdx.x, layer = a.l0 + blockIdx.y;
  const int kvh = h / (a.H / a.G), hd = a.hd, n = a.n;
  const float* qkv = (const float*)a.qkv + (int64_t)layer * a.qkv_stride;
  const int kcol = (a.H + kvh) * hd, vcol = (a.H + a.G + kvh) * hd;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* p = pbuf + w * (n + 1);
  float* out = (float*)a.out + (int64_t)layer * a.out_stride;
  const int q = blockIdx.z * 4 + w;
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
}

hipError_t launch_attention(const AttnArgs& a, bool use_bf16, hipStream_t st) {
  if (a.P <= 0 || a.n <= 0) return hipErrorInvalidValue;
  if (use_bf16) {
    dim3 grid((a.n + 127) / 128, a.H, a.P);
    switch (a.hd) {
      case 32: hipLaunchKernelGGL(attn_bf16_kernel<32>, grid, dim3(256), 0, st, a); break;
      case 64: hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st, a); break;
      case 128: hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (a.n > 4096) return hipErrorInvalidValue;
    dim3 grid(a.H, a.P, (a.n + 3) / 4);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 4 * (a.n + 1) * sizeof(float), st, a);
  }
  return hipGetLastError();
}

}  // namespace armt
