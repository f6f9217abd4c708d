// Backward pass of the fp32 forward (vector-Jacobian product), run over the
// diagonal waves in reverse order: node (s, l) needs the gradient of its
// output from node (s, l+1) and the gradient of the state it wrote from node
// (s+1, l), so the reversed grid is again S + L - 1 waves of independent
// nodes (Pith review of arXiv 2506.05229, "What carries the argument", Lemma
// 3.1, applied to the transposed dependency graph; the pages' appendix
// describes the grouped backward).  Each launch covers every active layer of
// a wave (problem p = layer l0 + p); every buffer is a per-layer slab, so the
// per-layer weight gradients take one node's contribution per wave with
// plain read-modify-write and the result does not depend on the wave width.
//
// These are fp32 kernels on the vector ALU (no matrix cores, no packed fp32):
// a generic strided GEMM with coalesced tile loads for either operand
// orientation, attention kernels that form each (query, key) score once and
// keep a row of probabilities in LDS, and row / element kernels.
#include <cmath>
#include <type_traits>
#include <utility>

#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time
// (register-array indices stay static).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float dphi_f(float u) { return u > 0.f ? 1.f : __expf(u); }

// ---------------------------------------------------------------------------
// Generic strided GEMM, P problems: C = beta * C + A B with
// A(m, k) = A + p*a_ps + m*a_rs + k*a_cs, B(k, n) likewise, C(m, n) likewise.
// TM x TN outputs per workgroup of 16 x 16 threads, (TM/16) x (TN/16) per
// thread; K in steps of 16 staged in LDS k-major.  Tile loads put consecutive
// threads on whichever index of the operand is contiguous in memory, so both
// a matrix and its transpose load coalesced.  Every output accumulates its
// products one k at a time in increasing k with fused multiply-adds, whatever
// the tile shape.  B may hold bf16 values (the weights of a bf16 model),
// widened exactly on load.
// ---------------------------------------------------------------------------
template <int TM, int TN, typename BT>
__global__ __launch_bounds__(256) void gemm_gen_kernel(GenGemm g) {
  constexpr int KS = 16, RM = TM / 16, RN = TN / 16;
  __shared__ __attribute__((aligned(16))) float As[KS][TM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[KS][TN + 4];
  const int p = blockIdx.z;
  const float* A = g.A + (int64_t)p * g.a_ps;
  const BT* B = (const BT*)g.B + (int64_t)p * g.b_ps;
  float* C = g.C + (int64_t)p * g.c_ps;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const bool a_kc = g.a_cs == 1, b_nc = g.b_cs == 1;   // contiguous along k (A) / along n (B)
  float acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += KS) {
#pragma unroll
    for (int t = 0; t < TM * KS / 256; ++t) {
      const int idx = tid + 256 * t;
      const int r = a_kc ? idx / KS : idx % TM, c = a_kc ? idx % KS : idx / TM;
      const int m = m0 + r, k = k0 + c;
      As[c][r] = (m < g.M && k < g.K) ? A[(int64_t)m * g.a_rs + (int64_t)k * g.a_cs] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < TN * KS / 256; ++t) {
      const int idx = tid + 256 * t;
      const int c = b_nc ? idx % TN : idx / KS, r = b_nc ? idx / TN : idx % KS;
      const int kk = k0 + r, n = n0 + c;
      Bs[r][c] = (kk < g.K && n < g.N) ? (float)B[(int64_t)kk * g.b_rs + (int64_t)n * g.b_cs] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float av[RM], bv[RN];
#pragma unroll
      for (int i = 0; i < RM; ++i) av[i] = As[k][ty * RM + i];
#pragma unroll
      for (int j = 0; j < RN; ++j) bv[j] = Bs[k][tx * RN + j];
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const int m = m0 + ty * RM + i, n = n0 + tx * RN + j;
      if (m < g.M && n < g.N) {
        float* c = C + (int64_t)m * g.c_rs + (int64_t)n * g.c_cs;
        *c = g.accumulate ? *c + acc[i][j] : acc[i][j];
      }
    }
}

// ---------------------------------------------------------------------------
// The same strided GEMM on the matrix cores (v_mfma_f32_32x32x16_bf16), for
// the backward of bf16 models.  Every fp32 operand enters as a bf16 pair
// (hi = R(v), lo = R(v - hi), |v - hi - lo| <= 2^-17 |v|): the products are
// A_hi B_hi + A_lo B_hi + A_hi B_lo for an fp32 B, A_hi B + A_lo B for a bf16
// B (weights, exact), so about 16 bits of each operand survive; fp32
// accumulation.  Tile 128 x 128, four waves of 64 x 64 (2 x 2 blocks of
// 32 x 32); K in steps of 32.  LDS holds each operand tile as 128 rows (m of
// A, n of B) of 32 k (64 bytes = four 16-byte chunks, XOR-swizzled so
// fragment reads of 16 consecutive rows are conflict-free).  Tile loads take
// 16-byte vectors along whichever index is contiguous in memory when the
// shape and alignment allow (VK: along k, VR: along the rows), else single
// elements; stages are loaded into registers one or two steps ahead of the
// one being multiplied (two or three register sets, two LDS buffers).
// ---------------------------------------------------------------------------
namespace mm {
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int BM = 128, BN = 128, BK = 32, ROWB = BK * 2, OPB = BM * ROWB;
enum { GEN = 0, VK = 1, VR = 2 };
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1); }
// byte offset of k (even) in row r
__device__ __forceinline__ int koff(int r, int k) { return r * ROWB + swz(r, k >> 3) * 16 + (k & 7) * 2; }
__device__ __forceinline__ unsigned bits(bf16 v) { return (unsigned)__builtin_bit_cast(unsigned short, v); }
__device__ __forceinline__ unsigned pack2(bf16 a, bf16 b) { return bits(a) | (bits(b) << 16); }
__device__ __forceinline__ bf16 lo_of(float v, bf16 hi) { return (bf16)(v - (float)hi); }

// One operand tile: element (r, k) of the 128 x 32 tile at rows r0.., k0..
// sits at base + r * rs + k * cs.  raw: 16 words of stage registers.
template <typename T, int MODE, bool LO>   // LO: an fp32 tile also stores its low parts
struct Opnd {
  const T* base;
  int64_t rs, cs;
  int rows, K;   // valid extent
  __device__ __forceinline__ void load(int r0, int k0, unsigned (&raw)[16], int tid) const {
    if constexpr (MODE == GEN) {
      // 2048 k pairs; consecutive lanes on the contiguous index
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = tid + 256 * j;
        const int r = cs == 1 ? i >> 4 : i & 127, kp = cs == 1 ? i & 15 : i >> 7;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int k = k0 + 2 * kp + t;
          const float v = (r0 + r < rows && k < K) ? (float)base[(int64_t)(r0 + r) * rs + (int64_t)k * cs] : 0.f;
          raw[2 * j + t] = __builtin_bit_cast(unsigned, v);
        }
      }
    } else if constexpr (MODE == VK && sizeof(T) == 4) {
      // 1024 vectors of 4 k: row i / 8, k 4 (i % 8)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = tid + 256 * j, r = i >> 3, k = k0 + 4 * (i & 7);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r0 + r < rows && k < K) v = *(const u32x4*)(base + (int64_t)(r0 + r) * rs + k);
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[4 * j + t] = v[t];
      }
    } else if constexpr (MODE == VK) {
      // 512 vectors of 8 k: row i / 4, k 8 (i % 4)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j, r = i >> 2, k = k0 + 8 * (i & 3);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r0 + r < rows && k < K) v = *(const u32x4*)(base + (int64_t)(r0 + r) * rs + k);
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[4 * j + t] = v[t];
      }
    } else if constexpr (sizeof(T) == 4) {
      // VR: 512 units of 4 rows x k pair: rows 4 (i % 32), k pair i / 32
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j, r = 4 * (i & 31), k = k0 + 2 * (i >> 5);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (r0 + r < rows && k + t < K) v = *(const u32x4*)(base + (int64_t)(r0 + r) + (int64_t)(k + t) * cs);
#pragma unroll
          for (int e = 0; e < 4; ++e) raw[8 * j + 4 * t + e] = v[e];
        }
      }
    } else {
      // VR, 2-byte elements: 256 units of 8 rows x k pair: rows 8 (i % 16), k pair i / 16
      const int i = tid, r = 8 * (i & 15), k = k0 + 2 * (i >> 4);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r0 + r < rows && k + t < K) v = *(const u32x4*)(base + (int64_t)(r0 + r) + (int64_t)(k + t) * cs);
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[4 * t + e] = v[e];
      }
    }
  }
  // raw -> LDS (hi part at hi, lo part at lo when T is fp32)
  __device__ __forceinline__ void store(const unsigned (&raw)[16], unsigned char* hi, unsigned char* lo,
                                        int tid) const {
    constexpr bool F32 = sizeof(T) == 4 && LO;
    if constexpr (MODE == GEN) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = tid + 256 * j;
        const int r = cs == 1 ? i >> 4 : i & 127, kp = cs == 1 ? i & 15 : i >> 7;
        const float v0 = __builtin_bit_cast(float, raw[2 * j]), v1 = __builtin_bit_cast(float, raw[2 * j + 1]);
        const bf16 h0 = (bf16)v0, h1 = (bf16)v1;
        const int o = koff(r, 2 * kp);
        *(unsigned*)(hi + o) = pack2(h0, h1);
        if (F32) *(unsigned*)(lo + o) = pack2(lo_of(v0, h0), lo_of(v1, h1));
      }
    } else if constexpr (MODE == VK && sizeof(T) == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = tid + 256 * j, r = i >> 3, k = 4 * (i & 7);
        bf16 h[4], l[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float v = __builtin_bit_cast(float, raw[4 * j + t]);
          h[t] = (bf16)v;
          l[t] = lo_of(v, h[t]);
        }
        const int o = koff(r, k);
        *(uint2*)(hi + o) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
        if (F32) *(uint2*)(lo + o) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
      }
    } else if constexpr (MODE == VK) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j, r = i >> 2;
        *(u32x4*)(hi + r * ROWB + swz(r, i & 3) * 16) =
            u32x4{raw[4 * j], raw[4 * j + 1], raw[4 * j + 2], raw[4 * j + 3]};
      }
    } else if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + 256 * j, r = 4 * (i & 31), k = 2 * (i >> 5);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = __builtin_bit_cast(float, raw[8 * j + e]), v1 = __builtin_bit_cast(float, raw[8 * j + 4 + e]);
          const bf16 h0 = (bf16)v0, h1 = (bf16)v1;
          const int o = koff(r + e, k);
          *(unsigned*)(hi + o) = pack2(h0, h1);
          if (F32) *(unsigned*)(lo + o) = pack2(lo_of(v0, h0), lo_of(v1, h1));
        }
      }
    } else {
      const int i = tid, r = 8 * (i & 15), k = 2 * (i >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned w0 = raw[e >> 1], w1 = raw[4 + (e >> 1)];
        const unsigned b0 = (e & 1) ? w0 >> 16 : w0 & 0xffffu, b1 = (e & 1) ? w1 >> 16 : w1 & 0xffffu;
        *(unsigned*)(hi + koff(r + e, k)) = b0 | (b1 << 16);
      }
    }
  }
};
}  // namespace mm

template <int AM, int BMODE, bool B16>
__global__ __launch_bounds__(256, (AM == mm::GEN || BMODE == mm::GEN) ? 1 : 2) void gemm_mfma_kernel(GenGemm g) {
  using namespace mm;
  using BT = typename std::conditional<B16, bf16, float>::type;
  constexpr bool ALO = true, BL = !B16;   // fp32 operands as hi/lo pairs
  constexpr int NB = BL ? 4 : 3;               // A_hi, A_lo, B_hi (, B_lo)
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][NB * OPB];
  const int p = blockIdx.z;
  const Opnd<float, AM, ALO> opa{g.A + (int64_t)p * g.a_ps, g.a_rs, g.a_cs, g.M, g.K};
  const Opnd<BT, BMODE, BL> opb{(const BT*)g.B + (int64_t)p * g.b_ps, g.b_cs, g.b_rs, g.N, g.K};
  float* C = g.C + (int64_t)p * g.c_ps;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // register sets for staged tiles: loads run PD = NSET - 1 stages ahead
  // (two fp32 operands take more registers: one stage ahead keeps two
  // workgroups per CU)
  constexpr int NSET = (B16 || AM == GEN || BMODE == GEN) ? 3 : 2;
  unsigned ra[NSET][16], rb[NSET][16];
  auto put = [&](int buf, const unsigned (&xa)[16], const unsigned (&xb)[16]) {
    unsigned char* base = lds[buf];
    opa.store(xa, base, base + OPB, tid);
    opb.store(xb, base + 2 * OPB, base + 3 * OPB, tid);
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](int buf) {
    const unsigned char* base = lds[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + r32;
        const int o = r * ROWB + swz(r, 2 * ks + h) * 16;
        ah[i] = *(const bf16x8*)(base + o);
        if (ALO) al[i] = *(const bf16x8*)(base + OPB + o);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 64 * wn + 32 * j + r32;
        const int o = r * ROWB + swz(r, 2 * ks + h) * 16;
        bh[j] = *(const bf16x8*)(base + 2 * OPB + o);
        if (BL) bl[j] = *(const bf16x8*)(base + 3 * OPB + o);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
          if (ALO) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
          if (BL) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
        }
    }
  };

  // stage s: register set s % NSET, LDS buffer s % 2
  constexpr int PD = NSET - 1;
  const int nst = (g.K + BK - 1) / BK;
  static_for<PD>([&](auto I) {
    constexpr int t = decltype(I)::value;
    if (t < nst) {
      opa.load(m0, t * BK, ra[t], tid);
      opb.load(n0, t * BK, rb[t], tid);
    }
  });
  put(0, ra[0], rb[0]);
  __syncthreads();
  for (int s0 = 0; s0 < nst; s0 += NSET) {
    static_for<NSET>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const int s = s0 + u;
      if (s < nst) {
        if (s + PD < nst) {
          opa.load(m0, (s + PD) * BK, ra[(u + PD) % NSET], tid);
          opb.load(n0, (s + PD) * BK, rb[(u + PD) % NSET], tid);
        }
        compute(s & 1);
        if (s + 1 < nst) put((s + 1) & 1, ra[(u + 1) % NSET], rb[(u + 1) % NSET]);
        __syncthreads();
      }
    });
  }
  // element e of block (i, j) in lane (r32, h): row 8(e/4) + 4h + e%4, column r32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        const int n = n0 + 64 * wn + 32 * j + r32;
        if (m < g.M && n < g.N) {
          float* c = C + (int64_t)m * g.c_rs + (int64_t)n * g.c_cs;
          *c = g.accumulate ? *c + acc[i][j][e] : acc[i][j][e];
        }
      }
}

// ---------------------------------------------------------------------------
// Row kernels.  One wave per row (rows of every problem: blockIdx.y = p).
// ---------------------------------------------------------------------------

// q = phi(u) (u kept), den = q . z + eps
__global__ __launch_bounds__(256) void phi_den_kernel(BwArgs a, const float* u, float* q, float* den,
                                                      const float* z, int64_t u_ps, int64_t z_ps, int rows) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + w;
  if (r >= rows) return;
  const float* ur = u + p * u_ps + (int64_t)r * 64;
  float* qr = q + p * u_ps + (int64_t)r * 64;
  const float qq = phi_f(ur[lane]);
  qr[lane] = qq;
  const float s = wave_sum(qq * z[p * z_ps + lane]);
  if (lane == 0) den[p * (int64_t)a.row_ps + r] = s + a.mem_eps;
}

// out = base + num / den[row]   (d columns)
__global__ __launch_bounds__(256) void add_div_kernel(BwArgs a, const float* base, const float* num, const float* den,
                                                      float* out, int64_t ps, int rows) {
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * a.d) return;
  const int r = (int)(i / a.d);
  out[p * ps + i] = base[p * ps + i] + num[p * ps + i] / den[p * (int64_t)a.row_ps + r];
}

// out = x * rs * g, rs[row] = 1 / sqrt(mean(x^2) + eps)
__global__ __launch_bounds__(256) void rms_fwd_kernel(BwArgs a, const float* x, const float* g, float* out, float* rs,
                                                      int64_t ps, int64_t g_ps, int rows) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + w;
  if (r >= rows) return;
  const float* xr = x + p * ps + (int64_t)r * a.d;
  float ss = 0.f;
  for (int i = lane; i < a.d; i += 64) ss = fmaf(xr[i], xr[i], ss);
  ss = wave_sum(ss);
  const float rr = 1.f / sqrtf(ss / (float)a.d + a.rms_eps);
  const float* gg = g + p * g_ps;
  float* o = out + p * ps + (int64_t)r * a.d;
  for (int i = lane; i < a.d; i += 64) o[i] = xr[i] * rr * gg[i];
  if (lane == 0) rs[p * (int64_t)a.row_ps + r] = rr;
}

// dx (+)= rs * (g . dy) - x * rs^3 * mean(x . g . dy)
__global__ __launch_bounds__(256) void rms_bwd_kernel(BwArgs a, const float* x, const float* g, const float* rs,
                                                      const float* dy, float* dx, int64_t ps, int64_t g_ps, int rows,
                                                      int accumulate) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + w;
  if (r >= rows) return;
  const float* xr = x + p * ps + (int64_t)r * a.d;
  const float* dr = dy + p * ps + (int64_t)r * a.d;
  const float* gg = g + p * g_ps;
  float dot = 0.f;
  for (int i = lane; i < a.d; i += 64) dot = fmaf(xr[i], gg[i] * dr[i], dot);
  dot = wave_sum(dot);
  const float rr = rs[p * (int64_t)a.row_ps + r];
  const float c = rr * rr * rr * dot / (float)a.d;
  float* o = dx + p * ps + (int64_t)r * a.d;
  for (int i = lane; i < a.d; i += 64) {
    const float v = rr * gg[i] * dr[i] - xr[i] * c;
    o[i] = accumulate ? o[i] + v : v;
  }
}

// dg[i] += sum over rows of dy[r, i] * x[r, i] * rs[r]   (one column per thread)
__global__ __launch_bounds__(64) void rms_dgain_kernel(BwArgs a, const float* x, const float* rs, const float* dy,
                                                        float* dg, int64_t ps, int64_t g_ps, int rows) {
  const int p = blockIdx.y;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= a.d) return;
  const float* dyp = dy + p * ps + i;
  const float* xp = x + p * ps + i;
  const float* rp = rs + p * (int64_t)a.row_ps;
  float s = 0.f;
  int r = 0;
  // rows in order; the loads of 8 rows are issued before their products
  for (; r + 8 <= rows; r += 8) {
    float dv[8], xv[8], rv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dv[u] = dyp[(int64_t)(r + u) * a.d];
      xv[u] = xp[(int64_t)(r + u) * a.d];
      rv[u] = rp[r + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s = fmaf(dv[u], xv[u] * rv[u], s);
  }
  for (; r < rows; ++r) s = fmaf(dyp[(int64_t)r * a.d], xp[(int64_t)r * a.d] * rp[r], s);
  dg[p * g_ps + i] += s;
}

// RoPE on the first `heads` heads of rows of width ld (in place); sign -1
// rotates back (the transpose, for gradients).
__global__ __launch_bounds__(256) void rope_kernel(BwArgs a, float* x, int64_t ps, int ld, int col0, int heads,
                                                   float sign, int rows) {
  const int p = blockIdx.y;
  const int hd = a.hd, half = hd / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * heads * half) return;
  const int r = (int)(i / (heads * half)), rem = (int)(i % (heads * half));
  const int hh = rem / half, f = rem % half;
  float* row = x + p * ps + (int64_t)r * ld + col0 + hh * hd;
  const float c = a.rope[((int64_t)r * half + f) * 2], s = sign * a.rope[((int64_t)r * half + f) * 2 + 1];
  const float x0 = row[f], x1 = row[f + half];
  row[f] = x0 * c - x1 * s;
  row[f + half] = x1 * c + x0 * s;
}

// Causal attention forward with the row statistics kept: one wave per
// (query, head).  O[q, j] = sum_k P[q, k] V[k, kv], P = softmax(scale q.k).
// The lanes first take keys (scores, max, sum of exponentials; P kept in the
// wave's LDS row), then head-dimension elements (the weighted sum over keys
// in key order).
__global__ __launch_bounds__(256) void attn_fwd_kernel(BwArgs a, const float* qkv, float* O, float* mx, float* lsum,
                                                       int64_t qkv_ps, int64_t o_ps, int64_t st_ps) {
  extern __shared__ float wrow[];   // [4][n]
  const int p = blockIdx.z, j = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + w;
  const int n = a.n, hd = a.hd, ld = a.qkv_ld;
  const bool active = q < n;
  const int kv = j / (a.H / a.G);
  const float* base = qkv + p * qkv_ps;
  const int kc = (a.H + kv) * hd, vc = (a.H + a.G + kv) * hd;
  float* pr = wrow + w * n;
  float m = -INFINITY, l = 0.f;
  if (active) {
    const float* qv = base + (int64_t)q * ld + j * hd;
    for (int k = lane; k <= q; k += 64) {
      float s = 0.f;
      for (int e = 0; e < hd; ++e) s = fmaf(qv[e], base[(int64_t)k * ld + kc + e], s);
      pr[k] = s * a.scale;
      m = fmaxf(m, s * a.scale);
    }
    m = wave_max(m);
    for (int k = lane; k <= q; k += 64) {
      const float e = __expf(pr[k] - m);
      pr[k] = e;
      l += e;
    }
    l = wave_sum(l);
    for (int k = lane; k <= q; k += 64) pr[k] = pr[k] / l;
  }
  __syncthreads();   // P rows written by one lane, read by all lanes of the wave
  if (!active) return;
  for (int e = lane; e < hd; e += 64) {
    float acc = 0.f;
    for (int k = 0; k <= q; ++k) acc = fmaf(pr[k], base[(int64_t)k * ld + vc + e], acc);
    O[p * o_ps + (int64_t)q * (a.H * hd) + j * hd + e] = acc;
  }
  if (lane == 0) {
    mx[p * st_ps + (int64_t)j * n + q] = m;
    lsum[p * st_ps + (int64_t)j * n + q] = l;
  }
}

__device__ __forceinline__ float att_score(const BwArgs& a, const float* base, int q, int k, int j, int kv) {
  const int hd = a.hd, ld = a.qkv_ld;
  const float* qv = base + (int64_t)q * ld + j * hd;
  const float* kvp = base + (int64_t)k * ld + (a.H + kv) * hd;
  float s = 0.f;
  for (int e = 0; e < hd; ++e) s = fmaf(qv[e], kvp[e], s);
  return s * a.scale;
}
__device__ __forceinline__ float att_dp(const BwArgs& a, const float* base, const float* dO, int q, int k, int j,
                                        int kv) {
  const int hd = a.hd, ld = a.qkv_ld;
  const float* dov = dO + (int64_t)q * (a.H * hd) + j * hd;
  const float* vv = base + (int64_t)k * ld + (a.H + a.G + kv) * hd;
  float s = 0.f;
  for (int e = 0; e < hd; ++e) s = fmaf(dov[e], vv[e], s);
  return s;
}

// Attention backward, part 1: one wave per (query, head):
// Dq = sum_k P dP (= dO . O), dQ[q] = scale * sum_k P (dP - Dq) K[k].
// Lanes take keys for dS = P (dP - Dq) (kept in the wave's LDS row), then
// head-dimension elements for the sum over keys in key order.
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(BwArgs a, const float* qkv, const float* O, const float* dO,
                                                         const float* mx, const float* lsum, float* Dq, float* dqkv,
                                                         int64_t qkv_ps, int64_t o_ps, int64_t st_ps) {
  extern __shared__ float wrow[];   // [4][n]
  const int p = blockIdx.z, j = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + w;
  const int n = a.n, hd = a.hd, ld = a.qkv_ld;
  const bool active = q < n;
  const int kv = j / (a.H / a.G);
  const float* base = qkv + p * qkv_ps;
  const float* dOp = dO + p * o_ps;
  float* ds = wrow + w * n;
  float dd = 0.f;
  if (active) {
    for (int e = lane; e < hd; e += 64)
      dd = fmaf(dOp[(int64_t)q * (a.H * hd) + j * hd + e], O[p * o_ps + (int64_t)q * (a.H * hd) + j * hd + e], dd);
    dd = wave_sum(dd);
    const float m = mx[p * st_ps + (int64_t)j * n + q], l = lsum[p * st_ps + (int64_t)j * n + q];
    for (int k = lane; k <= q; k += 64) {
      const float P = __expf(att_score(a, base, q, k, j, kv) - m) / l;
      ds[k] = P * (att_dp(a, base, dOp, q, k, j, kv) - dd);
    }
  }
  __syncthreads();
  if (!active) return;
  for (int e = lane; e < hd; e += 64) {
    float acc = 0.f;
    for (int k = 0; k <= q; ++k) acc = fmaf(ds[k], base[(int64_t)k * ld + (a.H + kv) * hd + e], acc);
    dqkv[p * qkv_ps + (int64_t)q * ld + j * hd + e] = acc * a.scale;
  }
  if (lane == 0) Dq[p * st_ps + (int64_t)j * n + q] = dd;
}

// Attention backward, part 2: one wave per (key, kv-head), summing over the
// query heads of its group and the queries at or after the key:
// dK[k] = scale * sum P (dP - Dq) Q[q],  dV[k] = sum P dO[q].
// Per query head, lanes take queries for P and dS (kept in the wave's LDS
// rows), then head-dimension elements for the sums over queries in order.
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(BwArgs a, const float* qkv, const float* dO, const float* mx,
                                                          const float* lsum, const float* Dq, float* dqkv,
                                                          int64_t qkv_ps, int64_t o_ps, int64_t st_ps) {
  extern __shared__ float wrow[];   // [4][2n]
  const int p = blockIdx.z, kv = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + w;
  const int n = a.n, hd = a.hd, ld = a.qkv_ld, rep = a.H / a.G;
  const bool active = k < n;
  const float* base = qkv + p * qkv_ps;
  const float* dOp = dO + p * o_ps;
  float* pr = wrow + w * 2 * n;
  float* ds = pr + n;
  float dk[2] = {0.f, 0.f}, dv[2] = {0.f, 0.f};   // e = lane, lane + 64 (hd <= 128)
  for (int j = kv * rep; j < (kv + 1) * rep; ++j) {
    if (active) {
      for (int q = k + lane; q < n; q += 64) {
        const float m = mx[p * st_ps + (int64_t)j * n + q], l = lsum[p * st_ps + (int64_t)j * n + q];
        const float P = __expf(att_score(a, base, q, k, j, kv) - m) / l;
        pr[q] = P;
        ds[q] = P * (att_dp(a, base, dOp, q, k, j, kv) - Dq[p * st_ps + (int64_t)j * n + q]);
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = lane + 64 * t;
        if (e < hd) {
          for (int q = k; q < n; ++q) {
            dk[t] = fmaf(ds[q], base[(int64_t)q * ld + j * hd + e], dk[t]);
            dv[t] = fmaf(pr[q], dOp[(int64_t)q * (a.H * hd) + j * hd + e], dv[t]);
          }
        }
      }
    }
    __syncthreads();   // the rows are rewritten for the next query head
  }
  if (!active) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int e = lane + 64 * t;
    if (e < hd) {
      dqkv[p * qkv_ps + (int64_t)k * ld + (a.H + kv) * hd + e] = dk[t] * a.scale;
      dqkv[p * qkv_ps + (int64_t)k * ld + (a.H + a.G + kv) * hd + e] = dv[t];
    }
  }
}

// Uo = silu(G) * Up   /   dG, dUp from dUo
__global__ __launch_bounds__(256) void swiglu_kernel(const float* Gt, const float* Up, float* Uo, int64_t count,
                                                     int64_t ps) {
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float g = Gt[p * ps + i];
  Uo[p * ps + i] = g / (1.f + __expf(-g)) * Up[p * ps + i];
}
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* Gt, const float* Up, const float* dUo, float* dG,
                                                         float* dUp, int64_t count, int64_t ps) {
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float g = Gt[p * ps + i], u = Up[p * ps + i], d = dUo[p * ps + i];
  const float sg = 1.f / (1.f + __expf(-g));
  dG[p * ps + i] = d * u * sg * (1.f + g * (1.f - sg));
  dUp[p * ps + i] = d * g * sg;
}

// Memory write, recomputed per memory row m (one wave each):
// k = phi(uk), beta = sigmoid(bl), denw = k . z + eps, vbar = kA / denw,
// e = beta (v - vbar).
__global__ __launch_bounds__(256) void memw_fwd_kernel(BwArgs a, const float* uk, float* k, const float* bl,
                                                       float* beta, const float* z, float* denw, const float* kA,
                                                       const float* v, float* e, int64_t z_ps) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + w;
  if (m >= a.M) return;
  const int64_t km = ((int64_t)p * a.M + m) * 64;
  const float kk = phi_f(uk[km + lane]);
  k[km + lane] = kk;
  const float dn = wave_sum(kk * z[p * z_ps + lane]) + a.mem_eps;
  const float b = 1.f / (1.f + __expf(-bl[p * a.M + m]));
  if (lane == 0) {
    denw[p * a.M + m] = dn;
    beta[p * a.M + m] = b;
  }
  const int64_t vm = ((int64_t)p * a.M + m) * a.d;
  for (int i = lane; i < a.d; i += 64) e[vm + i] = b * (v[vm + i] - kA[vm + i] / dn);
}

// Memory write backward, per memory row m (one wave each), given
// de = k dA'^T: dbeta, dv = beta de, dkA = -beta de / denw,
// ddenw = sum_i beta de_i kA_i / denw^2, dbl = dbeta beta (1 - beta).
__global__ __launch_bounds__(256) void memw_bwd_kernel(BwArgs a, const float* de, const float* v, const float* kA,
                                                       const float* beta, const float* denw, float* dv, float* dkA,
                                                       float* ddenw, float* dbl) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + w;
  if (m >= a.M) return;
  const int64_t vm = ((int64_t)p * a.M + m) * a.d;
  const float b = beta[p * a.M + m], dn = denw[p * a.M + m];
  float db = 0.f, dden = 0.f;
  for (int i = lane; i < a.d; i += 64) {
    const float dei = de[vm + i], kai = kA[vm + i];
    db = fmaf(dei, v[vm + i] - kai / dn, db);
    dv[vm + i] = b * dei;
    dkA[vm + i] = -b * dei / dn;
    dden = fmaf(b * dei, kai, dden);
  }
  db = wave_sum(db);
  dden = wave_sum(dden);
  if (lane == 0) {
    ddenw[p * a.M + m] = dden / (dn * dn);
    dbl[p * a.M + m] = db * b * (1.f - b);
  }
}

// dk += ddenw[m] z + dz' (and -> duk = dk phi'(uk)); dz = dz' + sum_m ddenw[m] k[m]
// (in place on the layer's dz, which held dz').  One workgroup per problem.
__global__ __launch_bounds__(64) void memw_dk_kernel(BwArgs a, float* dk, const float* uk, const float* k,
                                                     const float* ddenw, const float* z, float* dz, int64_t z_ps,
                                                     int64_t dz_ps) {
  const int p = blockIdx.x, j = threadIdx.x;
  const float dzp = dz[p * dz_ps + j], zj = z[p * z_ps + j];
  float acc = dzp;
  for (int m = 0; m < a.M; ++m) {
    const int64_t km = ((int64_t)p * a.M + m) * 64 + j;
    const float dd = ddenw[p * a.M + m];
    const float g = dk[km] + dd * zj + dzp;
    dk[km] = g * dphi_f(uk[km]);
    acc = fmaf(dd, k[km], acc);
  }
  dz[p * dz_ps + j] = acc;
}

// dY += dbl[m] w_beta, dw_beta += sum_m dbl[m] Y[m]
__global__ __launch_bounds__(256) void memw_beta_kernel(BwArgs a, const float* dbl, const float* wb, const float* Y,
                                                        float* dY, float* dwb, int64_t y_ps, int64_t wb_ps) {
  const int p = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.d) return;
  float s = 0.f;
  for (int m = 0; m < a.M; ++m) {
    const float d = dbl[p * a.M + m];
    dY[p * y_ps + (int64_t)m * a.d + i] += d * wb[p * wb_ps + i];
    s = fmaf(d, Y[p * y_ps + (int64_t)m * a.d + i], s);
  }
  dwb[p * wb_ps + i] += s;
}

// Memory read backward, per row (one wave each): dnum = dh1 / den,
// dden = -sum_i dh1_i num_i / den^2.
__global__ __launch_bounds__(256) void memr_bwd_kernel(BwArgs a, const float* dh1, const float* num, const float* den,
                                                       float* dnum, float* dden, int64_t ps, int rows) {
  const int p = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + w;
  if (r >= rows) return;
  const float dn = den[p * (int64_t)a.row_ps + r];
  const int64_t o = p * ps + (int64_t)r * a.d;
  float s = 0.f;
  for (int i = lane; i < a.d; i += 64) {
    dnum[o + i] = dh1[o + i] / dn;
    s = fmaf(dh1[o + i], num[o + i], s);
  }
  s = wave_sum(s);
  if (lane == 0) dden[p * (int64_t)a.row_ps + r] = -s / (dn * dn);
}

// dq += dden[r] z, du = dq phi'(u)  (in place on dq); dz += sum_r dden[r] q[r]
__global__ __launch_bounds__(64) void memr_dq_kernel(BwArgs a, float* dq, const float* u, const float* q,
                                                     const float* dden, const float* z, float* dz, int64_t u_ps,
                                                     int64_t z_ps, int64_t dz_ps, int rows) {
  const int p = blockIdx.x, j = threadIdx.x;
  const float zj = z[p * z_ps + j];
  float acc = 0.f;
  int r = 0;
  // rows in order; the loads of 8 rows are issued before their updates
  for (; r + 8 <= rows; r += 8) {
    float dqv[8], uv[8], qv[8], ddv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t o = p * u_ps + (int64_t)(r + t) * 64 + j;
      dqv[t] = dq[o];
      uv[t] = u[o];
      qv[t] = q[o];
      ddv[t] = dden[p * (int64_t)a.row_ps + r + t];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      dq[p * u_ps + (int64_t)(r + t) * 64 + j] = (dqv[t] + ddv[t] * zj) * dphi_f(uv[t]);
      acc = fmaf(ddv[t], qv[t], acc);
    }
  }
  for (; r < rows; ++r) {
    const int64_t o = p * u_ps + (int64_t)r * 64 + j;
    const float dd = dden[p * (int64_t)a.row_ps + r];
    dq[o] = (dq[o] + dd * zj) * dphi_f(u[o]);
    acc = fmaf(dd, q[o], acc);
  }
  dz[p * dz_ps + j] += acc;
}

// Gather / scatter between the tape, the layer slabs and the caller's
// arrays.  Node (s, l) of problem p: layer l0 + p, segment s = c - l.
__global__ __launch_bounds__(256) void bw_copy_kernel(const float* src, float* dst, int64_t count, int64_t src_ps,
                                                      int64_t dst_ps, int accumulate) {
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  dst[p * dst_ps + i] = accumulate ? dst[p * dst_ps + i] + src[p * src_ps + i] : src[p * src_ps + i];
}

// dst = R(src) (bf16), count a multiple of 4, per-problem strides ps
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* src, bf16* dst, int64_t count4, int64_t ps) {
  const int p = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count4) return;
  const f32x4 v = *(const f32x4*)(src + p * ps + 4 * i);
  *(bf16x4*)(dst + p * ps + 4 * i) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// dst[c][r] = src[r][c] for r < rows_pad (zero for r >= rows), c < cols:
// bf16 hi part (and lo part when dst_lo) of an fp32 or bf16 source.  Tiles of
// 64 x 64 through LDS; reads coalesced along c, writes along r.
template <typename T>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const T* src, int64_t ld_src, int64_t src_ps, int rows,
                                                             int cols, bf16* dst_hi, bf16* dst_lo, int64_t ld_dst,
                                                             int64_t dst_ps) {
  __shared__ float tile[64][65];
  const int p = blockIdx.z, r0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
  const T* sp = src + p * src_ps;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * i + (tid >> 6), c = tid & 63;
    tile[r][c] = (r0 + r < rows && c0 + c < cols) ? (float)sp[(int64_t)(r0 + r) * ld_src + c0 + c] : 0.f;
  }
  __syncthreads();
  const int c = tid >> 2, r16 = (tid & 3) * 16;
  if (c0 + c >= cols) return;
  bf16x8 h[2], l[2];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const float v = tile[r16 + t][c];
    const bf16 hv = (bf16)v;
    h[t >> 3][t & 7] = hv;
    l[t >> 3][t & 7] = (bf16)(v - (float)hv);
  }
  bf16* dh = dst_hi + p * dst_ps + (int64_t)(c0 + c) * ld_dst + r0 + r16;
  *(bf16x8*)dh = h[0];
  *(bf16x8*)(dh + 8) = h[1];
  if (dst_lo) {
    bf16* dl = dst_lo + p * dst_ps + (int64_t)(c0 + c) * ld_dst + r0 + r16;
    *(bf16x8*)dl = l[0];
    *(bf16x8*)(dl + 8) = l[1];
  }
}

// dst[r][c] = hi(src[r][c]), dst[r][lo_off + c] = lo(src[r][c]) (bf16 pair);
// cols a multiple of 4
__global__ __launch_bounds__(256) void split_bf16_kernel(const float* src, int64_t ld_src, int64_t src_ps, int rows,
                                                         int cols, bf16* dst, int64_t ld_dst, int64_t dst_ps,
                                                         int lo_off) {
  const int p = blockIdx.y, c4n = cols / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * c4n) return;
  const int r = (int)(i / c4n), c = 4 * (int)(i % c4n);
  const f32x4 v = *(const f32x4*)(src + p * src_ps + (int64_t)r * ld_src + c);
  bf16x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (bf16)v[e];
    l[e] = (bf16)(v[e] - (float)h[e]);
  }
  bf16* d = dst + p * dst_ps + (int64_t)r * ld_dst + c;
  *(bf16x4*)d = h;
  *(bf16x4*)(d + lo_off) = l;
}

}  // namespace

hipError_t bw_split_bf16(const float* src, int64_t ld_src, int64_t src_ps, int rows, int cols, bf16* dst,
                         int64_t ld_dst, int64_t dst_ps, int lo_off, int P, hipStream_t st) {
  if (cols % 4 || ld_src % 4 || src_ps % 4 || ld_dst % 4 || dst_ps % 4 || lo_off % 4 || ((uintptr_t)src & 15) ||
      ((uintptr_t)dst & 7))
    return hipErrorInvalidValue;
  const int64_t items = (int64_t)rows * (cols / 4);
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)((items + 255) / 256), P), dim3(256), 0, st, src, ld_src,
                     src_ps, rows, cols, dst, ld_dst, dst_ps, lo_off);
  return hipGetLastError();
}

hipError_t bw_transpose_bf16(const void* src, bool src_bf16, int64_t ld_src, int64_t src_ps, int rows, int rows_pad,
                             int cols, bf16* dst_hi, bf16* dst_lo, int64_t ld_dst, int64_t dst_ps, int P,
                             hipStream_t st) {
  // rows_pad: whole 64-row tiles; 16-byte aligned destination rows
  if (rows_pad % 64 || rows_pad < rows || ld_dst < rows_pad || ld_dst % 8 || dst_ps % 8 || ((uintptr_t)dst_hi & 15) ||
      ((uintptr_t)dst_lo & 15))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(rows_pad / 64), (unsigned)((cols + 63) / 64), P);
  if (src_bf16)
    hipLaunchKernelGGL(transpose_bf16_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)src, ld_src, src_ps, rows,
                       cols, dst_hi, dst_lo, ld_dst, dst_ps);
  else
    hipLaunchKernelGGL(transpose_bf16_kernel<float>, grid, dim3(256), 0, st, (const float*)src, ld_src, src_ps, rows,
                       cols, dst_hi, dst_lo, ld_dst, dst_ps);
  return hipGetLastError();
}

hipError_t bw_to_bf16(const float* src, bf16* dst, int64_t count, int64_t ps, int P, hipStream_t st) {
  if (count % 4 || ps % 4 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 7)) return hipErrorInvalidValue;
  const int64_t c4 = count / 4;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((c4 + 255) / 256), P), dim3(256), 0, st, src, dst, c4, ps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_gemm_gen(const GenGemm& g, int P, bool matrix_cores, hipStream_t st) {
  if (P <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0) return hipErrorInvalidValue;
  if (matrix_cores) {
    const dim3 grid((g.N + mm::BN - 1) / mm::BN, (g.M + mm::BM - 1) / mm::BM, P);
    // 16-byte vectors along the contiguous index where every vector is whole
    // and aligned
    auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    int am = mm::GEN, bm = mm::GEN;
    if (al16(g.A) && g.a_ps % 4 == 0) {
      if (g.a_cs == 1 && g.a_rs % 4 == 0 && g.K % 4 == 0) am = mm::VK;
      else if (g.a_rs == 1 && g.a_cs % 4 == 0 && g.M % 4 == 0) am = mm::VR;
    }
    const int vb = g.b_bf16 ? 8 : 4;
    if (al16(g.B) && g.b_ps % vb == 0) {
      if (g.b_rs == 1 && g.b_cs % vb == 0 && g.K % vb == 0) bm = mm::VK;
      else if (g.b_cs == 1 && g.b_rs % vb == 0 && g.N % vb == 0) bm = mm::VR;
    }
#define MM_LAUNCH(AM_, BM_)                                                                             \
  do {                                                                                                 \
    if (g.b_bf16) hipLaunchKernelGGL((gemm_mfma_kernel<AM_, BM_, true>), grid, dim3(256), 0, st, g);  \
    else hipLaunchKernelGGL((gemm_mfma_kernel<AM_, BM_, false>), grid, dim3(256), 0, st, g);          \
  } while (0)
    switch (am * 3 + bm) {
      case 0: MM_LAUNCH(mm::GEN, mm::GEN); break;
      case 1: MM_LAUNCH(mm::GEN, mm::VK); break;
      case 2: MM_LAUNCH(mm::GEN, mm::VR); break;
      case 3: MM_LAUNCH(mm::VK, mm::GEN); break;
      case 4: MM_LAUNCH(mm::VK, mm::VK); break;
      case 5: MM_LAUNCH(mm::VK, mm::VR); break;
      case 6: MM_LAUNCH(mm::VR, mm::GEN); break;
      case 7: MM_LAUNCH(mm::VR, mm::VK); break;
      default: MM_LAUNCH(mm::VR, mm::VR); break;
    }
#undef MM_LAUNCH
    return hipGetLastError();
  }
  // 64 x 64 tiles only where they still give two workgroups per CU; the
  // products here are small, and the number of workgroups sets their speed
  const int64_t big = (int64_t)((g.M + 63) / 64) * ((g.N + 63) / 64) * P;
  const dim3 g64((g.N + 63) / 64, (g.M + 63) / 64, P), g32((g.N + 31) / 32, (g.M + 31) / 32, P);
  if (g.M >= 64 && g.N >= 64 && big >= 512) {
    if (g.b_bf16) hipLaunchKernelGGL((gemm_gen_kernel<64, 64, bf16>), g64, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_gen_kernel<64, 64, float>), g64, dim3(256), 0, st, g);
  } else {
    if (g.b_bf16) hipLaunchKernelGGL((gemm_gen_kernel<32, 32, bf16>), g32, dim3(256), 0, st, g);
    else hipLaunchKernelGGL((gemm_gen_kernel<32, 32, float>), g32, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

static dim3 rows_grid(int rows, int P) { return dim3((rows + 3) / 4, P); }
static dim3 elem_grid(int64_t count, int P) { return dim3((unsigned)((count + 255) / 256), P); }

hipError_t bw_phi_den(const BwArgs& a, const float* u, float* q, float* den, const float* z, int64_t u_ps,
                      int64_t z_ps, int rows, int P, hipStream_t st) {
  hipLaunchKernelGGL(phi_den_kernel, rows_grid(rows, P), dim3(256), 0, st, a, u, q, den, z, u_ps, z_ps, rows);
  return hipGetLastError();
}
hipError_t bw_add_div(const BwArgs& a, const float* base, const float* num, const float* den, float* out, int64_t ps,
                      int rows, int P, hipStream_t st) {
  hipLaunchKernelGGL(add_div_kernel, elem_grid((int64_t)rows * a.d, P), dim3(256), 0, st, a, base, num, den, out, ps,
                     rows);
  return hipGetLastError();
}
hipError_t bw_rms_fwd(const BwArgs& a, const float* x, const float* g, float* out, float* rs, int64_t ps,
                      int64_t g_ps, int rows, int P, hipStream_t st) {
  hipLaunchKernelGGL(rms_fwd_kernel, rows_grid(rows, P), dim3(256), 0, st, a, x, g, out, rs, ps, g_ps, rows);
  return hipGetLastError();
}
hipError_t bw_rms_bwd(const BwArgs& a, const float* x, const float* g, const float* rs, const float* dy, float* dx,
                      float* dg, int64_t ps, int64_t g_ps, int rows, int accumulate, int P, hipStream_t st) {
  hipLaunchKernelGGL(rms_dgain_kernel, dim3((a.d + 63) / 64, P), dim3(64), 0, st, a, x, rs, dy, dg, ps, g_ps, rows);
  hipLaunchKernelGGL(rms_bwd_kernel, rows_grid(rows, P), dim3(256), 0, st, a, x, g, rs, dy, dx, ps, g_ps, rows,
                     accumulate);
  return hipGetLastError();
}
hipError_t bw_rope(const BwArgs& a, float* x, int64_t ps, int ld, int col0, int heads, float sign, int rows, int P,
                   hipStream_t st) {
  hipLaunchKernelGGL(rope_kernel, elem_grid((int64_t)rows * heads * (a.hd / 2), P), dim3(256), 0, st, a, x, ps, ld,
                     col0, heads, sign, rows);
  return hipGetLastError();
}
hipError_t bw_attn_fwd(const BwArgs& a, const float* qkv, float* O, float* mx, float* ls, int64_t qkv_ps,
                       int64_t o_ps, int64_t st_ps, int P, hipStream_t st) {
  if (a.n > 4096 || a.hd > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((a.n + 3) / 4, a.H, P), dim3(256), 4 * a.n * sizeof(float), st, a, qkv, O,
                     mx, ls, qkv_ps, o_ps, st_ps);
  return hipGetLastError();
}
hipError_t bw_attn_bwd(const BwArgs& a, const float* qkv, const float* O, const float* dO, const float* mx,
                       const float* ls, float* Dq, float* dqkv, int64_t qkv_ps, int64_t o_ps, int64_t st_ps, int P,
                       hipStream_t st) {
  if (a.n > 4096 || a.hd > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bwd_q_kernel, dim3((a.n + 3) / 4, a.H, P), dim3(256), 4 * a.n * sizeof(float), st, a, qkv,
                     O, dO, mx, ls, Dq, dqkv, qkv_ps, o_ps, st_ps);
  hipLaunchKernelGGL(attn_bwd_kv_kernel, dim3((a.n + 3) / 4, a.G, P), dim3(256), 8 * a.n * sizeof(float), st, a, qkv,
                     dO, mx, ls, Dq, dqkv, qkv_ps, o_ps, st_ps);
  return hipGetLastError();
}
hipError_t bw_swiglu(const float* G, const float* Up, float* Uo, int64_t count, int64_t ps, int P, hipStream_t st) {
  hipLaunchKernelGGL(swiglu_kernel, elem_grid(count, P), dim3(256), 0, st, G, Up, Uo, count, ps);
  return hipGetLastError();
}
hipError_t bw_swiglu_bwd(const float* G, const float* Up, const float* dUo, float* dG, float* dUp, int64_t count,
                         int64_t ps, int P, hipStream_t st) {
  hipLaunchKernelGGL(swiglu_bwd_kernel, elem_grid(count, P), dim3(256), 0, st, G, Up, dUo, dG, dUp, count, ps);
  return hipGetLastError();
}
hipError_t bw_memw_fwd(const BwArgs& a, const float* uk, float* k, const float* bl, float* beta, const float* z,
                       float* denw, const float* kA, const float* v, float* e, int64_t z_ps, int P, hipStream_t st) {
  hipLaunchKernelGGL(memw_fwd_kernel, rows_grid(a.M, P), dim3(256), 0, st, a, uk, k, bl, beta, z, denw, kA, v, e,
                     z_ps);
  return hipGetLastError();
}
hipError_t bw_memw_bwd(const BwArgs& a, const float* de, const float* v, const float* kA, const float* beta,
                       const float* denw, float* dv, float* dkA, float* ddenw, float* dbl, int P, hipStream_t st) {
  hipLaunchKernelGGL(memw_bwd_kernel, rows_grid(a.M, P), dim3(256), 0, st, a, de, v, kA, beta, denw, dv, dkA, ddenw,
                     dbl);
  return hipGetLastError();
}
hipError_t bw_memw_dk(const BwArgs& a, float* dk, const float* uk, const float* k, const float* ddenw, const float* z,
                      float* dz, int64_t z_ps, int64_t dz_ps, int P, hipStream_t st) {
  hipLaunchKernelGGL(memw_dk_kernel, dim3(P), dim3(64), 0, st, a, dk, uk, k, ddenw, z, dz, z_ps, dz_ps);
  return hipGetLastError();
}
hipError_t bw_memw_beta(const BwArgs& a, const float* dbl, const float* wb, const float* Y, float* dY, float* dwb,
                        int64_t y_ps, int64_t wb_ps, int P, hipStream_t st) {
  hipLaunchKernelGGL(memw_beta_kernel, dim3((a.d + 255) / 256, P), dim3(256), 0, st, a, dbl, wb, Y, dY, dwb, y_ps,
                     wb_ps);
  return hipGetLastError();
}
hipError_t bw_memr_bwd(const BwArgs& a, const float* dh1, const float* num, const float* den, float* dnum, float* dden,
                       int64_t ps, int rows, int P, hipStream_t st) {
  hipLaunchKernelGGL(memr_bwd_kernel, rows_grid(rows, P), dim3(256), 0, st, a, dh1, num, den, dnum, dden, ps, rows);
  return hipGetLastError();
}
hipError_t bw_memr_dq(const BwArgs& a, float* dq, const float* u, const float* q, const float* dden, const float* z,
                      float* dz, int64_t u_ps, int64_t z_ps, int64_t dz_ps, int rows, int P, hipStream_t st) {
  hipLaunchKernelGGL(memr_dq_kernel, dim3(P), dim3(64), 0, st, a, dq, u, q, dden, z, dz, u_ps, z_ps, dz_ps, rows);
  return hipGetLastError();
}
hipError_t bw_copy(const float* src, float* dst, int64_t count, int64_t src_ps, int64_t dst_ps, int accumulate, int P,
                   hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(bw_copy_kernel, elem_grid(count, P), dim3(256), 0, st, src, dst, count, src_ps, dst_ps,
                     accumulate);
  return hipGetLastError();
}

}  // namespace armt
