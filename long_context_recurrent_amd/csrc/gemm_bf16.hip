// Grouped bf16 GEMM for one diagonal wave: problem p multiplies layer
// (l0 + p)'s activations by layer (l0 + p)'s weights, C = A * B^T with
// A [M, K] (row-major, K contiguous) and B [N, K] (weights, row-major
// [out, in]).  One launch covers every active layer of the wave -- the
// grouped layer of diagonal batching (Pith review of arXiv 2506.05229, "What
// carries the argument"; Figure 4 caption on grouped GEMM scaling; skill page
// "Diagonal Batching for Recurrent Memory Transformers", Implementation).
//
// CDNA4 mapping.  A workgroup of 4 waves owns a BM x 256 tile (BM = 16*MB
// rows, chosen per workload so that the n = T + M node rows split with little
// padding: 1040 = 5 * 208).  Each wave owns all BM rows and 64 of the 256
// columns and issues v_mfma_f32_16x16x32_bf16 on 16x16 blocks (fp32
// accumulators, MB*16 registers per lane).  K advances 64 at a time through a
// double-buffered LDS tile with padded rows (144 B pitch: conflict-free 16-byte
// fragment reads); the next K slice is loaded into registers while the current
// one is multiplied.  Tiles are ordered so that each of the 8 XCDs gets a
// contiguous range (same weights, neighbouring rows), keeping shared operands
// in that XCD's L2.  The epilogue stages fp32 results through LDS, so every
// global store is a coalesced 16-byte write and every bf16 rounding happens
// once, on the fp32 value:
//   EPI_QKV   : RoPE on the Q and K heads (pairs i, i + hd/2 are kept in the
//               same lane by the column map), bf16 store; V heads are stored
//               transposed ([G][hd][n_pad]) for the attention kernel.
//   EPI_RESID : C = R(C + acc) in place (residual add); for the last layer the
//               segment-token rows are also written to the caller's y.
//   EPI_SWIGLU: B holds gate rows then up rows; U = R(silu(gate) * up).
#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

constexpr int BK = 64;
constexpr int PITCH = BK + 8;   // bf16 elements per LDS row (144 bytes)
constexpr int BNB = 256;        // B-tile rows held in LDS
constexpr int RC = 64;          // epilogue rows staged per pass
constexpr int CPITCH_PAD = 4;

// Column-block map: block j (0..3) of wave w -> first B-tile row it uses.
// MAP_LINEAR (also hd 32 and 64): 64w + 16j.  MAP_HD128: a 128-wide head split
// so that block j and j + 2 are hd/2 = 64 apart.  MAP_DUAL: j < 2 gate rows
// 32w + 16j, j >= 2 the matching up rows 128 + 32w + 16(j - 2).
enum { MAP_LINEAR = 0, MAP_HD32 = 1, MAP_HD64 = 2, MAP_HD128 = 3, MAP_DUAL = 4 };

template <int MAP>
__device__ __forceinline__ int col_block(int w, int j) {
  if (MAP == MAP_HD128) return 128 * (w >> 1) + 32 * (w & 1) + (j & 1) * 16 + (j >> 1) * 64;
  if (MAP == MAP_DUAL) return (j < 2) ? (32 * w + 16 * j) : (128 + 32 * w + 16 * (j - 2));
  return 64 * w + 16 * j;
}

// Output column (relative to the tile's first output column) of block j's
// lane column 0.
template <int MAP>
__device__ __forceinline__ int out_col_block(int w, int j) {
  if (MAP == MAP_DUAL) return 32 * w + 16 * (j & 1);
  return col_block<MAP>(w, j);
}

// RoPE partner of block j (hd/2 columns to the right) under each head map.
template <int MAP>
constexpr int rope_pmask() { return MAP == MAP_HD32 ? 1 : 2; }
template <int MAP>
constexpr int rope_hd() { return MAP == MAP_HD32 ? 32 : (MAP == MAP_HD64 ? 64 : 128); }

__device__ __forceinline__ void xcd_tile(int id, int total, int& logical) {
  // Hardware dispatches workgroup id to XCD id % 8.  Give XCD x the
  // contiguous logical range [start(x), start(x) + count(x)).
  const int q = total >> 3, r = total & 7;
  const int x = id & 7, j = id >> 3;
  logical = x * q + (x < r ? x : r) + j;
}

}  // namespace

template <int MB, int EPI, int MAP>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = 16 * MB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  constexpr int A_CHUNKS = BM * (BK / 8);              // 16-byte chunks per A tile
  constexpr int A_ITERS = (A_CHUNKS + 255) / 256;
  constexpr int B_ITERS = BNB * (BK / 8) / 256;        // = 8
  constexpr int LDS_TILE = (BM + BNB) * PITCH;         // bf16 elements per stage
  constexpr int CPITCH = BN_OUT + CPITCH_PAD;
  static_assert(2 * LDS_TILE * 2 <= 160 * 1024, "LDS budget");
  static_assert(RC * CPITCH * 4 <= 2 * LDS_TILE * 2, "epilogue staging fits");

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * LDS_TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN_OUT - 1) / BN_OUT;
  const int total = tiles_m * tiles_n * g.P;
  int logical;
  xcd_tile(blockIdx.x, total, logical);
  const int tm = logical % tiles_m;
  const int tn = (logical / tiles_m) % tiles_n;
  const int p = logical / (tiles_m * tiles_n);
  const int layer = g.l0 + p;
  const int m0 = tm * BM;
  const int n0 = tn * BN_OUT;

  const bf16* __restrict__ A = (const bf16*)g.A + (int64_t)layer * g.a_stride;
  const bf16* __restrict__ B = (const bf16*)g.B + (int64_t)layer * g.b_stride;
  const bf16* __restrict__ B2 =
      (EPI == EPI_SWIGLU) ? (const bf16*)g.B2 + (int64_t)layer * g.b_stride : B;

  // ---- global -> register staging (element offsets; chunk c = tid + 256 i
  // covers tile row c / 8, 16-byte column chunk c % 8) ----
  int a_off[A_ITERS];
  int b_off[B_ITERS];
#pragma unroll
  for (int i = 0; i < A_ITERS; ++i) {
    const int c = tid + 256 * i;
    int row = m0 + c / 8;
    row = row < g.M ? row : g.M - 1;
    a_off[i] = row * g.lda + (c % 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_ITERS; ++i) {
    const int c = tid + 256 * i;
    // dual: tile rows 0..127 (i < 4) are gate rows, 128..255 the up rows
    int nrow = n0 + ((EPI == EPI_SWIGLU) ? ((c / 8) & 127) : (c / 8));
    nrow = nrow < g.N ? nrow : g.N - 1;
    b_off[i] = nrow * g.K + (c % 8) * 8;
  }

  u32x4 ra[A_ITERS], rb[B_ITERS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i)
      if (A_CHUNKS % 256 == 0 || tid + 256 * i < A_CHUNKS)
        ra[i] = *(const u32x4*)(A + a_off[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const bf16* base = (EPI == EPI_SWIGLU && i >= B_ITERS / 2) ? B2 : B;
      rb[i] = *(const u32x4*)(base + b_off[i] + kt * BK);
    }
  };
  auto lstore = [&](int buf) {
    bf16* As = smem + buf * LDS_TILE;
    bf16* Bs = As + BM * PITCH;
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int c = tid + 256 * i;
      if (A_CHUNKS % 256 == 0 || c < A_CHUNKS)
        *(u32x4*)(As + (c / 8) * PITCH + (c % 8) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const int c = tid + 256 * i;
      *(u32x4*)(Bs + (c / 8) * PITCH + (c % 8) * 8) = rb[i];
    }
  };

  f32x4 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = g.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const bf16* As = smem + buf * LDS_TILE;
    const bf16* Bs = As + BM * PITCH;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *(const bf16x8*)(Bs + (col_block<MAP>(w, j) + frag_row) * PITCH + kk + frag_k);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const bf16x8 afr = *(const bf16x8*)(As + (16 * i + frag_row) * PITCH + kk + frag_k);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- register epilogue: RoPE (QKV) or SiLU * up (SWIGLU) ----
  const int lrow = (lane >> 4) * 4;    // first of the lane's 4 accumulator rows
  const int lcol = lane & 15;
  if (EPI == EPI_QKV) {
    constexpr int hd = rope_hd<MAP>(), half = hd / 2, pmask = rope_pmask<MAP>();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((j & pmask) != 0) continue;
      const int pj = j ^ pmask;
      const int c = n0 + col_block<MAP>(w, j) + lcol;      // global output column
      if (c < g.rope_cols) {
        const int e = c % hd;                                // < half
#pragma unroll
        for (int i = 0; i < MB; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int m = m0 + 16 * i + lrow + r;
            m = m < g.M ? m : g.M - 1;
            const float2 cs = *(const float2*)(g.rope_cs + ((int64_t)m * half + e) * 2);
            const float x1 = acc[i][j][r], x2 = acc[i][pj][r];
            acc[i][j][r] = x1 * cs.x - x2 * cs.y;
            acc[i][pj][r] = x2 * cs.x + x1 * cs.y;
          }
        }
      }
    }
  }

  // ---- staged store ----
  float* Cs = (float*)smem;
  for (int rc0 = 0; rc0 < BM; rc0 += RC) {
    // waves write their fp32 results for rows [rc0, rc0 + RC) of the tile
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (16 * i < rc0 || 16 * i >= rc0 + RC) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int oc = out_col_block<MAP>(w, j) + lcol;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[i][j][r], up = acc[i][j + 2][r];
            Cs[(16 * i - rc0 + lrow + r) * CPITCH + oc] = gt * sigmoid_f(gt) * up;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int oc = out_col_block<MAP>(w, j) + lcol;
#pragma unroll
          for (int r = 0; r < 4; ++r) Cs[(16 * i - rc0 + lrow + r) * CPITCH + oc] = acc[i][j][r];
        }
      }
    }
    __syncthreads();
    const int rows_here = (BM - rc0) < RC ? (BM - rc0) : RC;
    constexpr int PIECES_ROW = BN_OUT / 8;
    bf16* C = (bf16*)g.C + (int64_t)layer * g.c_stride;
    if (EPI == EPI_QKV) {
      // row-major pieces for Q and K columns
      for (int pc = tid; pc < rows_here * PIECES_ROW; pc += 256) {
        const int r = pc / PIECES_ROW, c8 = (pc % PIECES_ROW) * 8;
        const int m = m0 + rc0 + r, n = n0 + c8;
        if (m >= g.M || n >= g.v_col0) continue;
        const float* src = Cs + r * CPITCH + c8;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)src[e];
        *(bf16x8*)(C + (int64_t)m * g.ldc + n) = o;
      }
      // transposed pieces for V columns: 8 consecutive rows of one column
      bf16* Vt = (bf16*)g.vt + (int64_t)layer * g.vt_stride;
      const int rgroups = (rows_here + 7) / 8;
      for (int pc = tid; pc < rgroups * BN_OUT; pc += 256) {
        const int col = pc % BN_OUT, rg = pc / BN_OUT;
        const int n = n0 + col;
        if (n < g.v_col0 || n >= g.N) continue;
        const int m = m0 + rc0 + rg * 8;
        if (m >= g.M) continue;
        const int vc = n - g.v_col0;                       // kv_head * hd + e
        bf16* dst = Vt + (int64_t)vc * g.vt_ld + m;
        const float* src = Cs + (rg * 8) * CPITCH + col;
        if (m + 8 <= g.M) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)src[e * CPITCH];
          *(bf16x8*)dst = o;
        } else {
          for (int e = 0; m + e < g.M; ++e) dst[e] = (bf16)src[e * CPITCH];
        }
      }
    } else {
      bf16* Y = nullptr;
      int y_rows = 0;
      if (EPI == EPI_RESID && g.desc != nullptr && layer == g.last_layer) {
        const int s = g.desc->c - layer;
        Y = (bf16*)g.desc->y + (int64_t)s * g.T * g.ldc;
        y_rows = g.T;
      }
      for (int pc = tid; pc < rows_here * PIECES_ROW; pc += 256) {
        const int r = pc / PIECES_ROW, c8 = (pc % PIECES_ROW) * 8;
        const int m = m0 + rc0 + r, n = n0 + c8;
        if (m >= g.M || n >= g.N) continue;
        const float* src = Cs + r * CPITCH + c8;
        bf16* dst = C + (int64_t)m * g.ldc + n;
        bf16x8 o;
        if (EPI == EPI_RESID) {
          const bf16x8 res = *(const bf16x8*)dst;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)res[e] + src[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)src[e];
        }
        *(bf16x8*)dst = o;
        if (m < y_rows) *(bf16x8*)(Y + (int64_t)m * g.ldc + n) = o;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <int MB, int EPI, int MAP>
static hipError_t launch_mb(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 16 * MB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN_OUT - 1) / BN_OUT) * g.P;
  hipLaunchKernelGGL((gemm_bf16_kernel<MB, EPI, MAP>), dim3(tiles), dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int EPI, int MAP>
static hipError_t launch_map(const GemmArgs& g, int mb, hipStream_t st) {
  switch (mb) {
    case 4: return launch_mb<4, EPI, MAP>(g, st);
    case 8: return launch_mb<8, EPI, MAP>(g, st);
    case 9: return launch_mb<9, EPI, MAP>(g, st);
    case 11: return launch_mb<11, EPI, MAP>(g, st);
    case 12: return launch_mb<12, EPI, MAP>(g, st);
    case 13: return launch_mb<13, EPI, MAP>(g, st);
    default: return hipErrorInvalidValue;
  }
}

const int kGemmRowBlocks[] = {4, 8, 9, 11, 12, 13};
const int kGemmRowBlocksCount = 6;

hipError_t launch_gemm_bf16(const GemmArgs& g, int epi, int mb, hipStream_t st) {
  if (g.P <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % BK) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV:
      if (g.head_dim == 128) return launch_map<EPI_QKV, MAP_HD128>(g, mb, st);
      if (g.head_dim == 64) return launch_map<EPI_QKV, MAP_HD64>(g, mb, st);
      if (g.head_dim == 32) return launch_map<EPI_QKV, MAP_HD32>(g, mb, st);
      return hipErrorInvalidValue;
    case EPI_RESID: return launch_map<EPI_RESID, MAP_LINEAR>(g, mb, st);
    case EPI_SWIGLU: return launch_map<EPI_SWIGLU, MAP_DUAL>(g, mb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace armt
