// Causal attention for the backward of bf16 models, on the matrix cores
// (v_mfma_f32_32x32x16_bf16): the recomputed forward (O and the row
// statistics), then dQ, then dK and dV -- the gradient of softmax attention
// (Pith review of arXiv 2506.05229, "What carries the argument": batched
// attention inside the grouped layer; the appendix's grouped backward runs the
// same waves in reverse).  One launch covers every node of a wave (problem p).
//
// Operands arrive in fp32 (the backward's recomputed activations) and enter
// the products rounded to bf16 -- Q, K and V as the bf16 forward rounds them,
// dO, P and dS as the usual flash-attention backward does; accumulation,
// softmax statistics and the outputs are fp32.  Per query q of head j:
//   S = scale Q K^T,  P = softmax(S) (causal),  O = P V,
//   D = rowsum(dO * O),  dS = P * (dO V^T - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// (dK and dV summed over the query heads of a key/value head).
//
// Layout: each wave owns 32 queries (or 32 keys) and multiplies with the
// transposed score tile so that a lane holds 16 scores of ONE query (key):
// S^T = K Q^T for the query-side kernels, S = Q K^T for the key side.  The
// probabilities then feed the second product straight from registers as its
// second operand; the first operand's rows (V^T, K^T, dO^T, Q^T staged in
// LDS) keep, within every aligned group of 16 keys / queries, the order
// 0-3, 8-11, 4-7, 12-15, which is the order of a lane's 8 operand slots.
// Tiles of 64 keys (queries) are staged from fp32 global memory into LDS as
// bf16 by all 256 threads, the next tile's loads in flight while the current
// one multiplies; 16-byte chunks are XOR-swizzled for conflict-free fragment
// reads.  Row statistics use base-2 exponentials: m2 = max(S) log2(e) and
// l = sum 2^(S log2 e - m2).
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// physical 16-byte chunk of chunk c in row r of a tile with CH chunks per row
template <int CH>
__device__ __forceinline__ int swzc(int r, int c) {
  if (CH == 8) return c ^ ((r ^ (r >> 3)) & 7);
  return c ^ (r & 15);   // CH == 16
}
// stored position of index i within its aligned group of 16
__device__ __forceinline__ int perm16(int i) {
  const int a = (i >> 2) & 3;
  return (i & ~15) + 4 * (((a & 1) << 1) | (a >> 1)) + (i & 3);
}

// Stage registers of one [64][HD] fp32 tile: 64 * HD / 4 float4 over 256
// threads; vector v = tid + 256 i covers row v / (HD/4), columns 4 (v % (HD/4)).
template <int HD>
struct Tile {
  static constexpr int NV = 64 * HD / 4 / 256;
  f32x4 v[NV];
  // rows r0 .. r0+63 of a [n][ld] matrix, columns col0 ..; rows >= n load 0
  __device__ __forceinline__ void load(const float* src, int ld, int col0, int r0, int n, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + 256 * i, r = vi / (HD / 4), c = 4 * (vi % (HD / 4));
      v[i] = r0 + r < n ? *(const f32x4*)(src + (int64_t)(r0 + r) * ld + col0 + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // row-major bf16 [64][HD]
  __device__ __forceinline__ void put_rows(unsigned char* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + 256 * i, r = vi / (HD / 4), c = 4 * (vi % (HD / 4));
      const bf16x4 b = {(bf16)v[i][0], (bf16)v[i][1], (bf16)v[i][2], (bf16)v[i][3]};
      *(bf16x4*)(dst + r * (HD * 2) + swzc<HD / 8>(r, c >> 3) * 16 + (c & 7) * 2) = b;
    }
  }
  // transposed bf16 [HD][64], the 64 rows of the tile permuted within groups of 16
  __device__ __forceinline__ void put_cols(unsigned char* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + 256 * i, r = vi / (HD / 4), c = 4 * (vi % (HD / 4));
      const int pr = perm16(r);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = c + t;
        *(bf16*)(dst + row * 128 + swzc<8>(row, pr >> 3) * 16 + (pr & 7) * 2) = (bf16)v[i][t];
      }
    }
  }
};

// A-operand fragment: row `row` of a row-major [.][HD] bf16 tile, 16-wide k
// step ks, lane half h
template <int HD>
__device__ __forceinline__ bf16x8 frag_rows(const unsigned char* t, int row, int ks, int h) {
  return *(const bf16x8*)(t + row * (HD * 2) + swzc<HD / 8>(row, 2 * ks + h) * 16);
}
// A-operand fragment of a transposed [HD][64] tile: row e, 16-group g
__device__ __forceinline__ bf16x8 frag_cols(const unsigned char* t, int e, int g, int h) {
  return *(const bf16x8*)(t + e * 128 + swzc<8>(e, 2 * g + h) * 16);
}
// B-operand fragment from global fp32: row `row` (clamped by caller), columns
// col0 + 16 ks + 8 h .. + 7
__device__ __forceinline__ bf16x8 frag_global(const float* src, int64_t ld, int row, int col0, int ks, int h) {
  const float* p = src + (int64_t)row * ld + col0 + 16 * ks + 8 * h;
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}
// scores of block kb, elements 8 ks .. 8 ks + 7, as a bf16 operand
__device__ __forceinline__ bf16x8 as_operand(const f32x16& s, int ks) {
  f32x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = s[8 * ks + j];
  return __builtin_convertvector(v, bf16x8);
}

}  // namespace

// ---------------------------------------------------------------------------
// Recomputed forward: O (fp32) and the row statistics m2, l of every query.
// Workgroup = (128 queries, query head, problem); wave w owns 32 queries.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_mfma_kernel(BwArgs a, const float* qkv, float* O, float* mx,
                                                            float* lsum, int64_t qkv_ps, int64_t o_ps,
                                                            int64_t st_ps) {
  constexpr int ES = HD / 16, DB = HD / 32;
  __shared__ __attribute__((aligned(16))) unsigned char kt[64 * HD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char vt[HD * 128];
  const int n = a.n, ld = a.qkv_ld, p = blockIdx.z, j = blockIdx.y;
  const int kv = j / (a.H / a.G);
  const float* base = qkv + p * qkv_ps;
  const int kc = (a.H + kv) * HD, vc = (a.H + a.G + kv) * HD;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int qb0 = blockIdx.x * 128, q0w = qb0 + 32 * w, q = q0w + r32;
  const int qc = q < n ? q : n - 1;
  const int q_end = qb0 + 128 < n ? qb0 + 128 : n;
  const int ntile = (q_end + 63) / 64;

  bf16x8 qf[ES];
#pragma unroll
  for (int ks = 0; ks < ES; ++ks) qf[ks] = frag_global(base, ld, qc, j * HD, ks, h);
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float mrun = -INFINITY, ls = 0.f;
  const float sl2 = a.scale * kLog2e;

  Tile<HD> tk, tv;
  tk.load(base, ld, kc, 0, n, tid);
  tv.load(base, ld, vc, 0, n, tid);
  for (int t = 0; t < ntile; ++t) {
    __syncthreads();   // every wave is done with tile t - 1
    tk.put_rows(kt, tid);
    tv.put_cols(vt, tid);
    __syncthreads();
    if (t + 1 < ntile) {
      tk.load(base, ld, kc, 64 * (t + 1), n, tid);
      tv.load(base, ld, vc, 64 * (t + 1), n, tid);
    }
    if (64 * t > q0w + 31 || q0w >= n) continue;   // tile entirely after this wave's queries
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < ES; ++ks)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<HD>(kt, 32 * kb + r32, ks, h), qf[ks], s[kb], 0, 0,
                                                        0);
    }
    // element e of block kb: key 64t + 32kb + 8(e/4) + 4h + e%4, query q
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 64 * t + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
        s[kb][e] = (key > q || key >= n) ? -INFINITY : s[kb][e] * sl2;
        mloc = fmaxf(mloc, s[kb][e]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float mnew = fmaxf(mrun, mloc);   // finite: key 0 <= q on the first tile
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    ls *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    mrun = mnew;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[kb][e] = __builtin_amdgcn_exp2f(s[kb][e] - mnew);
        ls += s[kb][e];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf = as_operand(s[kb], ks);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(vt, 32 * db + r32, 2 * kb + ks, h), pf, o[db], 0,
                                                          0, 0);
      }
    }
  }
  ls += __shfl_xor(ls, 32, kWave);
  if (q < n) {
    const float inv = 1.f / ls;
    float* out = O + p * o_ps + (int64_t)q * (a.H * HD) + j * HD;
    // element e of block db: head-dimension index 32db + 8(e/4) + 4h + e%4
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4*)(out + 32 * db + 8 * g4 + 4 * h) =
            f32x4{o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv};
    if (h == 0) {
      mx[p * st_ps + (int64_t)j * n + q] = mrun;
      lsum[p * st_ps + (int64_t)j * n + q] = ls;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ (and D = rowsum(dO * O) for the key side).  Workgroup = (128 queries,
// query head, problem).
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_dq_mfma_kernel(BwArgs a, const float* qkv, const float* O,
                                                           const float* dO, const float* mx, const float* lsum,
                                                           float* Dq, float* dqkv, int64_t qkv_ps, int64_t o_ps,
                                                           int64_t st_ps) {
  constexpr int ES = HD / 16, DB = HD / 32;
  __shared__ __attribute__((aligned(16))) unsigned char kt[64 * HD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char vt[64 * HD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char ktt[HD * 128];
  const int n = a.n, ld = a.qkv_ld, p = blockIdx.z, j = blockIdx.y, hh = a.H * HD;
  const int kv = j / (a.H / a.G);
  const float* base = qkv + p * qkv_ps;
  const float* dOp = dO + p * o_ps;
  const float* Op = O + p * o_ps;
  const int kc = (a.H + kv) * HD, vc = (a.H + a.G + kv) * HD;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int qb0 = blockIdx.x * 128, q0w = qb0 + 32 * w, q = q0w + r32;
  const int qc = q < n ? q : n - 1;
  const int q_end = qb0 + 128 < n ? qb0 + 128 : n;
  const int ntile = (q_end + 63) / 64;

  bf16x8 qf[ES], df[ES];
#pragma unroll
  for (int ks = 0; ks < ES; ++ks) {
    qf[ks] = frag_global(base, ld, qc, j * HD, ks, h);
    df[ks] = frag_global(dOp, hh, qc, j * HD, ks, h);
  }
  // D = dO . O for query q (fp32): each lane half sums half the head
  float dd = 0.f;
  for (int e = 8 * h; e < HD; e += 16) {
    const float* x = dOp + (int64_t)qc * hh + j * HD + e;
    const float* y = Op + (int64_t)qc * hh + j * HD + e;
#pragma unroll
    for (int t = 0; t < 8; ++t) dd = fmaf(x[t], y[t], dd);
  }
  dd += __shfl_xor(dd, 32, kWave);
  const float m2 = mx[p * st_ps + (int64_t)j * n + qc], il = 1.f / lsum[p * st_ps + (int64_t)j * n + qc];
  if (q < n && h == 0) Dq[p * st_ps + (int64_t)j * n + q] = dd;
  const float sl2 = a.scale * kLog2e;
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  Tile<HD> tk, tv;
  tk.load(base, ld, kc, 0, n, tid);
  tv.load(base, ld, vc, 0, n, tid);
  for (int t = 0; t < ntile; ++t) {
    __syncthreads();
    tk.put_rows(kt, tid);
    tk.put_cols(ktt, tid);
    tv.put_rows(vt, tid);
    __syncthreads();
    if (t + 1 < ntile) {
      tk.load(base, ld, kc, 64 * (t + 1), n, tid);
      tv.load(base, ld, vc, 64 * (t + 1), n, tid);
    }
    if (64 * t > q0w + 31 || q0w >= n) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < ES; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<HD>(kt, 32 * kb + r32, ks, h), qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<HD>(vt, 32 * kb + r32, ks, h), df[ks], dp, 0, 0, 0);
      }
      // dS^T for keys 64t + 32kb + 8(e/4) + 4h + e%4 of query q
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 64 * t + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
        const float pe = (key > q || key >= n) ? 0.f : __builtin_amdgcn_exp2f(s[e] * sl2 - m2) * il;
        s[e] = pe * (dp[e] - dd);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 sf = as_operand(s, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(ktt, 32 * db + r32, 2 * kb + ks, h), sf, dq[db],
                                                           0, 0, 0);
      }
    }
  }
  if (q < n) {
    float* out = dqkv + p * qkv_ps + (int64_t)q * ld + j * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(f32x4*)(out + 32 * db + 8 * g4 + 4 * h) =
            f32x4{dq[db][4 * g4] * a.scale, dq[db][4 * g4 + 1] * a.scale, dq[db][4 * g4 + 2] * a.scale,
                  dq[db][4 * g4 + 3] * a.scale};
  }
}

// ---------------------------------------------------------------------------
// dK and dV.  Workgroup = (128 keys, key/value head, problem); wave w owns 32
// keys and sums over the query heads of its group and the queries at or after
// its keys.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void attn_dkv_mfma_kernel(BwArgs a, const float* qkv, const float* dO,
                                                            const float* mx, const float* lsum, const float* Dq,
                                                            float* dqkv, int64_t qkv_ps, int64_t o_ps,
                                                            int64_t st_ps) {
  constexpr int ES = HD / 16, DB = HD / 32;
  __shared__ __attribute__((aligned(16))) unsigned char qt[64 * HD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char dt[64 * HD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char qtt[HD * 128];
  __shared__ __attribute__((aligned(16))) unsigned char dtt[HD * 128];
  __shared__ float stm[64], stl[64], std_[64];
  const int n = a.n, ld = a.qkv_ld, p = blockIdx.z, g = blockIdx.y, hh = a.H * HD, rep = a.H / a.G;
  const float* base = qkv + p * qkv_ps;
  const float* dOp = dO + p * o_ps;
  const int kc = (a.H + g) * HD, vc = (a.H + a.G + g) * HD;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int kb0 = blockIdx.x * 128, k0w = kb0 + 32 * w, key = k0w + r32;
  const int kcl = key < n ? key : n - 1;
  const int t0 = kb0 / 64, ntile = (n + 63) / 64;

  bf16x8 kf[ES], vf[ES];
#pragma unroll
  for (int ks = 0; ks < ES; ++ks) {
    kf[ks] = frag_global(base, ld, kcl, kc, ks, h);
    vf[ks] = frag_global(base, ld, kcl, vc, ks, h);
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float sl2 = a.scale * kLog2e;
  const int nsteps = rep * (ntile - t0);
  Tile<HD> tq, td;
  auto load_step = [&](int it) {
    const int jj = g * rep + it / (ntile - t0), t = t0 + it % (ntile - t0);
    tq.load(base, ld, jj * HD, 64 * t, n, tid);
    td.load(dOp, hh, jj * HD, 64 * t, n, tid);
  };
  load_step(0);
  for (int it = 0; it < nsteps; ++it) {
    const int jj = g * rep + it / (ntile - t0), t = t0 + it % (ntile - t0);
    __syncthreads();
    tq.put_rows(qt, tid);
    tq.put_cols(qtt, tid);
    td.put_rows(dt, tid);
    td.put_cols(dtt, tid);
    if (tid < 64) {
      const int qq = 64 * t + tid < n ? 64 * t + tid : n - 1;
      const int64_t o = p * st_ps + (int64_t)jj * n + qq;
      stm[tid] = mx[o];
      stl[tid] = 1.f / lsum[o];
      std_[tid] = Dq[o];
    }
    __syncthreads();
    if (it + 1 < nsteps) load_step(it + 1);
    if (64 * t + 63 < k0w || k0w >= n) continue;   // every query of the tile is before this wave's keys
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < ES; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<HD>(qt, 32 * qb + r32, ks, h), kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<HD>(dt, 32 * qb + r32, ks, h), vf[ks], dp, 0, 0, 0);
      }
      // element e: query 64t + 32qb + 8(e/4) + 4h + e%4 of key `key`
      f32x16 pp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ql = 32 * qb + 8 * (e >> 2) + 4 * h + (e & 3), qq = 64 * t + ql;
        const float pe = (qq < key || qq >= n) ? 0.f : __builtin_amdgcn_exp2f(s[e] * sl2 - stm[ql]) * stl[ql];
        pp[e] = pe;
        s[e] = pe * (dp[e] - std_[ql]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf = as_operand(pp, ks), sf = as_operand(s, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(dtt, 32 * db + r32, 2 * qb + ks, h), pf, dv[db],
                                                           0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(qtt, 32 * db + r32, 2 * qb + ks, h), sf, dk[db],
                                                           0, 0, 0);
        }
      }
    }
  }
  if (key < n) {
    float* ok = dqkv + p * qkv_ps + (int64_t)key * ld + kc;
    float* ov = dqkv + p * qkv_ps + (int64_t)key * ld + vc;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        *(f32x4*)(ok + 32 * db + 8 * g4 + 4 * h) = f32x4{dk[db][4 * g4] * a.scale, dk[db][4 * g4 + 1] * a.scale,
                                                         dk[db][4 * g4 + 2] * a.scale, dk[db][4 * g4 + 3] * a.scale};
        *(f32x4*)(ov + 32 * db + 8 * g4 + 4 * h) =
            f32x4{dv[db][4 * g4], dv[db][4 * g4 + 1], dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]};
      }
  }
}

// ---------------------------------------------------------------------------
bool bw_attn_mfma_ok(const BwArgs& a) {
  return (a.hd == 64 || a.hd == 128) && a.qkv_ld % 4 == 0 && a.H % a.G == 0;
}

hipError_t bw_attn_mfma_fwd(const BwArgs& a, const float* qkv, float* O, float* mx, float* ls, int64_t qkv_ps,
                            int64_t o_ps, int64_t st_ps, int P, hipStream_t st) {
  if (!bw_attn_mfma_ok(a) || qkv_ps % 4 || o_ps % 4) return hipErrorInvalidValue;
  const dim3 grid((a.n + 127) / 128, a.H, P);
  if (a.hd == 64)
    hipLaunchKernelGGL(attn_fwd_mfma_kernel<64>, grid, dim3(256), 0, st, a, qkv, O, mx, ls, qkv_ps, o_ps, st_ps);
  else
    hipLaunchKernelGGL(attn_fwd_mfma_kernel<128>, grid, dim3(256), 0, st, a, qkv, O, mx, ls, qkv_ps, o_ps, st_ps);
  return hipGetLastError();
}

hipError_t bw_attn_mfma_bwd(const BwArgs& a, const float* qkv, const float* O, const float* dO, const float* mx,
                            const float* ls, float* Dq, float* dqkv, int64_t qkv_ps, int64_t o_ps, int64_t st_ps,
                            int P, hipStream_t st) {
  if (!bw_attn_mfma_ok(a) || qkv_ps % 4 || o_ps % 4) return hipErrorInvalidValue;
  const dim3 gq((a.n + 127) / 128, a.H, P), gk((a.n + 127) / 128, a.G, P);
  if (a.hd == 64) {
    hipLaunchKernelGGL(attn_dq_mfma_kernel<64>, gq, dim3(256), 0, st, a, qkv, O, dO, mx, ls, Dq, dqkv, qkv_ps, o_ps,
                       st_ps);
    hipLaunchKernelGGL(attn_dkv_mfma_kernel<64>, gk, dim3(256), 0, st, a, qkv, dO, mx, ls, Dq, dqkv, qkv_ps, o_ps,
                       st_ps);
  } else {
    hipLaunchKernelGGL(attn_dq_mfma_kernel<128>, gq, dim3(256), 0, st, a, qkv, O, dO, mx, ls, Dq, dqkv, qkv_ps, o_ps,
                       st_ps);
    hipLaunchKernelGGL(attn_dkv_mfma_kernel<128>, gk, dim3(256), 0, st, a, qkv, dO, mx, ls, Dq, dqkv, qkv_ps, o_ps,
                       st_ps);
  }
  return hipGetLastError();
}

}  // namespace armt
