// Grouped bf16 GEMM for one diagonal wave: problem p multiplies layer
// (l0 + p)'s activations by layer (l0 + p)'s weights, C = A * B^T with
// A [M, K] (row-major, K contiguous) and B [N, K] (weights, row-major
// [out, in]).  One launch covers every active layer of the wave -- the
// grouped layer of diagonal batching (Pith review of arXiv 2506.05229, "What
// carries the argument"; Figure 4 caption on grouped GEMM scaling; skill page
// "Diagonal Batching for Recurrent Memory Transformers", Implementation).
//
// CDNA4 mapping.
//  * Matrix core: v_mfma_f32_16x16x32_bf16 (fp32 accumulation).  With enough
//    independent accumulators in flight it sustains the same dense bf16 rate
//    as the 32x32x16 form on MI355X, and its 16-row granularity lets a node's
//    n = T + M rows split into tiles with little padding (1040 = 5 x 208).
//  * Tile: a workgroup of 4 waves owns BM x 256 outputs, BM = 16 * RB rows,
//    chosen per workload.  Each wave owns all BM rows and 64 columns: RB x 4
//    accumulator blocks of 16 x 16 (16 * RB accumulator registers per lane).
//  * Operands: K advances 32 per pipeline step (one MFMA per block).
//    Operand tiles are filled straight from global memory into LDS by
//    global_load_lds_dwordx4 (no staging registers): the A tile in four
//    stages of k = 32 (64-byte rows), issued three steps ahead; the weight
//    tile in three double stages of k = 64 (128-byte rows), issued every
//    other step at least three steps ahead, so its loads fetch whole cache
//    lines.  Rows keep their 16-byte chunks XOR-swizzled; a fragment read
//    covers one 16-row block and its lanes hit 16 different bank groups.
//    The fragments of the next step are read while the MFMAs of the current
//    one run.
//  * Schedule: tiles are numbered so that each of the 8 XCDs works through a
//    contiguous range (same layer, same weight columns, neighbouring rows of
//    every sequence of the batch), keeping the shared operand tiles in that
//    XCD's L2.
//  * Epilogue: every bf16 rounding happens once, on the fp32 value; except
//    for SwiGLU, fp32 results are staged through LDS, so every global store
//    is a coalesced 16-byte write:
//      EPI_QKV   : RoPE on the Q and K heads (partner column i + hd/2 read from
//                  the staged tile), bf16 store; V heads are stored transposed
//                  ([G * hd][n_pad], keys reordered within groups of 16) for
//                  the attention kernel.
//      EPI_RESID : C += acc in place on the fp32 residual stream; for the
//                  last layer the segment-token rows (fewer in a short last
//                  segment) are also written to the caller's y, rounded to bf16.
//      EPI_SWIGLU: the B tile holds 128 gate rows then the 128 matching up
//                  rows; a wave's gate and up blocks of the same output
//                  columns sit in the same lanes; U = R(silu(gate) * up),
//                  computed and stored straight from the registers (the
//                  products run with the operands swapped, so a lane holds
//                  four consecutive columns of one row).
//      EPI_STORE : fp32 store (LM-head logits; N a multiple of 8).
//  Every output element accumulates over K in the same order whatever RB or
//  the number of problems, so results do not depend on the wave width.
#include <type_traits>
#include <utility>

#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time
// (array indices stay static where a loop body holds barriers).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int BK = 32;          // k per pipeline stage
constexpr int ROWB = BK * 2;    // bytes per tile row in a stage (64)
constexpr int BNB = 256;        // B-tile rows per stage
constexpr int RC = 64;          // epilogue rows staged per pass
constexpr int CPITCH = 256 + 4; // staged tile pitch (floats)
constexpr int LDS_BYTES = 160 * 1024;

// Operand staging in LDS: NSA stages of the A tile (k = 32: BM rows of 64
// bytes) and NSB double stages of the B tile (k = 64: 256 rows of 128
// bytes, whole cache lines per row, so each B wave load covers 8 full lines
// instead of 16 half lines).
constexpr int NSA = 4;
constexpr int NSB = 3;
constexpr int B_STAGE = BNB * 2 * ROWB;   // 32 KB

// 16-byte chunk c (0..3) of tile row r sits at physical chunk
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1): the same logical chunk of any 8 (or 16)
// consecutive rows lands in 8 (16) different 16-byte bank groups, so fragment
// reads (lane L: row 16i + L % 16, chunk L / 16) are conflict-free whether the
// LDS serves 128 or 256 bytes per cycle.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// 16-byte chunk c (0..7) of a 128-byte B row r sits at physical chunk
// c ^ ((r >> 1) & 7): the same logical chunk of 16 consecutive rows covers
// all sixteen 16-byte bank groups of 256 bytes.
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
// Word 3 of a raw buffer resource on gfx9 parts (no format conversion), and a
// store offset past any bound used here (the store is dropped).
constexpr int kRawBuffer = 0x00020000;
constexpr int kDropOffset = 0x7fffff00;

// s_waitcnt immediate (gfx9 layout): vmcnt <= n, lgkmcnt = 0, expcnt free.
__host__ __device__ constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier without the release fence of __syncthreads(), which would
// also wait for every outstanding global->LDS load.  Callers wait for exactly
// what they need with s_waitcnt first; the empty asm statements keep the
// compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// First B-tile row (output column) of wave w's 16-column block j (0..3).
// SwiGLU: blocks 0, 1 are gate rows and blocks 2, 3 the up rows of the same
// output columns.
template <int EPI>
__device__ __forceinline__ int col_block(int w, int j) {
  if (EPI == EPI_SWIGLU) return (j < 2 ? 32 * w : 128 + 32 * w) + 16 * (j & 1);
  return 64 * w + 16 * j;
}

// Stored position of key k in a V^T row: keys 4..7 and 8..11 of every
// aligned group of 16 trade places.
__device__ __forceinline__ int vt_pos(int k) {
  const int a = (k >> 2) & 3;
  return (k & ~15) + 4 * (a == 1 ? 2 : a == 2 ? 1 : a) + (k & 3);
}

__device__ __forceinline__ int xcd_tile(int id, int total) {
  // Hardware dispatches workgroup id to XCD id % 8.  Give XCD x the
  // contiguous logical range [start(x), start(x) + count(x)).
  const int q = total >> 3, r = total & 7;
  const int x = id & 7, j = id >> 3;
  return x * q + (x < r ? x : r) + j;
}

// Raw buffer resource over [p, p + bytes) for wave-uniform p and bytes.  The
// parts go through readfirstlane so the compiler keeps the resource in
// scalar registers: a resource it cannot prove uniform wraps every buffer
// access in a loop over the distinct values in the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const unsigned long long a = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), kRawBuffer);
}

}  // namespace

template <int RB, int EPI, bool TAIL>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = 16 * RB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  constexpr int A_STAGE = BM * ROWB;                   // bytes per A stage
  constexpr int B_BASE = NSA * A_STAGE;                 // first B double stage
  constexpr int LDS_USED = B_BASE + NSB * B_STAGE;
  static_assert(LDS_USED <= LDS_BYTES, "operand stages fit");
  static_assert(RC * CPITCH * 4 <= LDS_USED, "epilogue staging fits");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_USED];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // logical tile order: row tile fastest, then sequence, then column tile,
  // then layer -- the row tiles of every sequence that share one weight tile
  // are neighbours
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_mb = tiles_m * g.batch;
  const int tiles_n = (g.N + BN_OUT - 1) / BN_OUT;
  const int logical = xcd_tile(blockIdx.x, tiles_mb * tiles_n * g.P);
  const int tmb = logical % tiles_mb;
  const int tm = tmb % tiles_m, seq = tmb / tiles_m;
  const int tn = (logical / tiles_mb) % tiles_n;
  const int layer = g.l0 + logical / (tiles_mb * tiles_n);   // model layer (weights)
  const int prob = layer * g.batch + seq;                      // (layer, sequence) problem
  const int m0 = tm * BM;
  const int n0 = tn * BN_OUT;

  const bf16* __restrict__ A = (const bf16*)g.A + (int64_t)prob * g.a_stride;
  const bf16* __restrict__ B = (const bf16*)g.B + (int64_t)layer * g.b_stride;
  const bf16* __restrict__ B2 =
      (EPI == EPI_SWIGLU) ? (const bf16*)g.B2 + (int64_t)layer * g.b_stride : B;

  // ---- direct global -> LDS loads (wave loads of 1 KB, lane L's 16 bytes
  // at byte 16 L of the block).
  // A stage: RB blocks of 16 rows; in block q lane L brings row 16q + L/4,
  // physical chunk L%4 (= logical chunk swz(row, L%4)).  Wave w issues the
  // blocks q = w, w + 4, ... below 4 NFA (NFA = RB / 4), and waves
  // w < EXA = RB % 4 one more whole block, 4 NFA + w.  (The choice is
  // wave-uniform: a load under a lane mask lets the compiler merge it with
  // the next load across the branch, and the LDS address of the merged load
  // is then taken from the wrong lanes.)
  // B double stage: 32 blocks of 8 rows; in block b lane L brings row
  // 8b + L/8, physical chunk L%8 (= logical chunk swz8(row, L%8)); wave w
  // issues blocks w, w + 4, ..., w + 28.
  // The vmcnt waits count this wave's own loads: NB per B double stage and
  // NFA or NFA + 1 per A stage.
  constexpr int EXA = RB % 4;
  constexpr int NFA = RB / 4;
  constexpr int NA = NFA + (EXA ? 1 : 0);              // A loads per stage, at most
  constexpr int NB = 8;                                // B loads per wave per double stage
  const bool a_extra = EXA != 0 && w < EXA;            // wave-uniform
  const bf16* srca[NA];
  int dsta[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const int q = t < NFA ? w + 4 * t : (a_extra ? 4 * NFA + w : 0);
    dsta[t] = 1024 * q;
    const int r = 16 * q + (lane >> 2);
    int row = m0 + r;
    row = row < g.M ? row : g.M - 1;
    srca[t] = A + (int64_t)row * g.lda + swz(r, lane & 3) * 8;
  }
  const bf16* srcb[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int r = 8 * (w + 4 * t) + (lane >> 3);        // B-tile row 0..255
    int nrow = n0 + ((EPI == EPI_SWIGLU) ? (r & 127) : r);
    nrow = nrow < g.N ? nrow : g.N - 1;
    const bf16* base = (EPI == EPI_SWIGLU && r >= 128) ? B2 : B;
    srcb[t] = base + (int64_t)nrow * (g.ldb ? g.ldb : g.K) + swz8(r, lane & 7) * 8;
  }
  const int KT = g.K / BK;                              // even: K is a multiple of 64
  // A stage kt / B double stage d (k = 64 d .. 64 d + 63); in short K loops,
  // stages past the end re-fetch the last one into a buffer nobody reads.
  auto issue_a = [&](int kt) {
    const int kc = kt < KT ? kt : KT - 1;
    unsigned char* st = smem + (kt % NSA) * A_STAGE;
#pragma unroll
    for (int t = 0; t < NFA; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(srca[t] + kc * BK),
                                       (__attribute__((address_space(3))) void*)(st + dsta[t]), 16, 0, 0);
    if (a_extra)
      __builtin_amdgcn_global_load_lds((const void*)(srca[NA - 1] + kc * BK),
                                       (__attribute__((address_space(3))) void*)(st + dsta[NA - 1]), 16, 0, 0);
  };
  auto issue_b = [&](int d) {
    const int dc = d < KT / 2 ? d : KT / 2 - 1;
    unsigned char* st = smem + B_BASE + (d % NSB) * B_STAGE;
#pragma unroll
    for (int t = 0; t < NB; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(srcb[t] + dc * 2 * BK),
                                       (__attribute__((address_space(3))) void*)(st + 1024 * (w + 4 * t)), 16, 0,
                                       0);
  };

  f32x4 acc[RB][4];

  // Fragments of one step (k = 32): lane (r16 = lane % 16, c = lane / 16)
  // holds k = 8c..8c+7 of row r16 of each 16-row A block and of each
  // 16-column B block -- one 16-byte read per block (B: half kt % 2 of its
  // double stage).
  const int r16 = lane & 15, kc = lane >> 4;
  bf16x8 fa0[RB], fb0[4], fa1[RB], fb1[4];
  auto read_frags = [&](int kt, bf16x8* fa, bf16x8* fb) {
    const unsigned char* sa = smem + (kt % NSA) * A_STAGE;
    const unsigned char* sb = smem + B_BASE + ((kt >> 1) % NSB) * B_STAGE;
    const int h4 = 4 * (kt & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = col_block<EPI>(w, j) + r16;
      fb[j] = *(const bf16x8*)(sb + r * (2 * ROWB) + swz8(r, h4 + kc) * 16);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = 16 * i + r16;
      fa[i] = *(const bf16x8*)(sa + r * ROWB + swz(r, kc) * 16);
    }
  };
  // vmcnt waits (lgkmcnt 0 as well: this wave's LDS reads drained, so nobody
  // refills a buffer another wave still reads once past the barrier).  A step
  // kt waits for A stage kt+1 (issued two steps earlier); loads issued after
  // it: even kt: the B double stage issued with it, one A stage, then this
  // step's A stage and B double stage; odd kt: one A stage with its B double
  // stage, then this step's A stage.  The B double stage holding k-step kt+1
  // was issued before that A stage.
  // wait_loads(S, E): at most S A stages and E other loads of this wave
  // younger than what is waited for.
  auto wait_loads = [&](auto nstages, auto nother) {
    constexpr int S = decltype(nstages)::value, E = decltype(nother)::value;
    if (a_extra)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(S * (NFA + 1) + E));
    else
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(S * NFA + E));
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using INB = std::integral_constant<int, NB>;
  using I2NB = std::integral_constant<int, 2 * NB>;

  // prologue, in the order the steady state would have issued it: B double
  // stage 0, A stages 0 and 1, B double stage 1, A stage 2; then A stage 0
  // and B double stage 0 landed and the first fragments read
  issue_b(0);
  issue_a(0);
  issue_a(1);
  issue_b(1);
  issue_a(2);
  wait_loads(I2{}, INB{});
  lds_barrier();
  read_frags(0, fa0, fb0);
  // One pipeline step kt: multiply part of the fragments already in
  // registers, refill A stage kt+3 (the one read two steps ago) and, on even
  // steps, B double stage kt/2 + 2 (the one read by steps kt-2 and kt-1),
  // wait until this wave's loads of k-step kt+1 landed, barrier, read k-step
  // kt+1's fragments into the other register set, and multiply the rest.
  // The first H row blocks' products of a step go out before the refill,
  // the wait and the barrier, so the matrix core has work while the waves
  // meet; the rest interleave with the next stage's fragment reads.  (Best
  // split measured per GEMM: a quarter of the rows for gate/up and QKV, a
  // third for the residual GEMMs; a third or half for gate/up, half or a
  // quarter for the residual GEMMs measured slower.)
  constexpr int H = (EPI == EPI_RESID) ? RB / 3 : RB / 4;
  // Products of row blocks I0 .. I1-1.  The first stage's products start
  // from zero (an explicit zero-initialised accumulator makes the register
  // allocator rotate the accumulators through copies on every trip of the K
  // loop).
  // SwiGLU multiplies with the operands swapped (weights as the first), so
  // its accumulator blocks hold C^T: the epilogue then finds one output row
  // and four consecutive columns per lane (see there).
  auto mfma_rows = [&](const bf16x8* fa, const bf16x8* fb, auto first, auto I0, auto I1) {
#pragma unroll
    for (int i = decltype(I0)::value; i < decltype(I1)::value; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 c = decltype(first)::value ? f32x4{} : acc[i][j];
        acc[i][j] = (EPI == EPI_SWIGLU) ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], c, 0, 0, 0)
                                        : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], c, 0, 0, 0);
      }
  };
  // Residual epilogue: each 64-row pass's fp32 residual rows are loaded into
  // registers one pass ahead; the first pass's loads go out in the K loop's
  // tail where registers allow (below), so they land while the last
  // products run.
  constexpr int PPT = RC * (BN_OUT / 8) / 256;     // pieces per thread per pass
  float* const Cf = (float*)g.C + (int64_t)prob * g.c_stride;
  f32x4 rb[2][PPT][2];
  // Every lane loads (a piece past the tile or the node reads a row that
  // exists and drops the value): loads in conditional blocks would leave
  // the compiler unsure which are in flight, and it would then wait for
  // all of them before every store, prefetched rows included.
  auto load_pass = [&](int rc0, f32x4 (&dstv)[PPT][2]) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pc = tid + 256 * k, r = pc >> 5, c8 = (pc & 31) * 8;
      int m = m0 + rc0 + r, n = n0 + c8;
      m = m < g.M ? m : g.M - 1;
      n = n < g.N ? n : g.N - 8;
      dstv[k][0] = *(const f32x4*)(Cf + (int64_t)m * g.ldc + n);
      dstv[k][1] = *(const f32x4*)(Cf + (int64_t)m * g.ldc + n + 4);
    }
  };
  // Residual loads issued in the tail (up to 176-row tiles: taller ones have
  // no registers to spare for them beside the two fragment sets).
  constexpr bool PREFETCH = EPI == EPI_RESID && TAIL && RB <= 11;
  constexpr int PF = PREFETCH ? 2 * PPT : 0;
  static_assert(NSA == 4 && NSB == 3, "step kinds assume four A stages and three B double stages");
  // Step kinds: 0 = steady state (even / odd k-step); for K >= 192 the last
  // four steps stop refilling what lies past K:
  //   4 (kt = KT-4): refills A stage KT-1 only; waits for A stage KT-3 with
  //     B double stage KT/2 - 1 and two A stages younger;
  //   1 (kt = KT-3): the residual epilogue may issue its first pass's loads
  //     instead; waits for A stage KT-2 with A stage KT-1 and those loads
  //     younger;
  //   2 (kt = KT-2): waits for A stage KT-1, the last one, with only the
  //     residual loads younger;
  //   3 (kt = KT-1): products only.
  auto step = [&](int kt, const bf16x8* fa_cur, const bf16x8* fb_cur, bf16x8* fa_nxt, bf16x8* fb_nxt,
                  auto first, auto kind) {
    constexpr int KIND = decltype(kind)::value;
    if constexpr (KIND == 3) {
      mfma_rows(fa_cur, fb_cur, first, std::integral_constant<int, 0>{}, std::integral_constant<int, RB>{});
      return;
    }
    mfma_rows(fa_cur, fb_cur, first, std::integral_constant<int, 0>{}, std::integral_constant<int, H>{});
    if constexpr (KIND == 0) {
      issue_a(kt + 3);
      if ((kt & 1) == 0) {
        issue_b((kt >> 1) + 2);
        wait_loads(I2{}, I2NB{});
      } else {
        wait_loads(I2{}, INB{});
      }
    } else if constexpr (KIND == 4) {
      issue_a(kt + 3);
      wait_loads(I2{}, INB{});
    } else if constexpr (KIND == 1) {
      if constexpr (PREFETCH) load_pass(0, rb[0]);
      wait_loads(I1{}, std::integral_constant<int, PF>{});
    } else {
      wait_loads(I0{}, std::integral_constant<int, PF>{});
    }
    lds_barrier();
    read_frags(kt + 1, fa_nxt, fb_nxt);
    mfma_rows(fa_cur, fb_cur, first, std::integral_constant<int, H>{}, std::integral_constant<int, RB>{});
    constexpr int NREAD = RB + 4, NMFMA = 4 * (RB - H);
    constexpr int PER = NMFMA / NREAD;
#pragma unroll
    for (int i = 0; i < NREAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - PER * NREAD, 0);
  };
  using K0 = std::integral_constant<int, 0>;
  step(0, fa0, fb0, fa1, fb1, std::true_type{}, K0{});
  step(1, fa1, fb1, fa0, fb0, std::false_type{}, K0{});
  if constexpr (TAIL) {   // K >= 192
    for (int kt = 2; kt < KT - 4; kt += 2) {
      step(kt, fa0, fb0, fa1, fb1, std::false_type{}, K0{});
      step(kt + 1, fa1, fb1, fa0, fb0, std::false_type{}, K0{});
    }
    step(KT - 4, fa0, fb0, fa1, fb1, std::false_type{}, std::integral_constant<int, 4>{});
    step(KT - 3, fa1, fb1, fa0, fb0, std::false_type{}, std::integral_constant<int, 1>{});
    step(KT - 2, fa0, fb0, fa1, fb1, std::false_type{}, std::integral_constant<int, 2>{});
    step(KT - 1, fa1, fb1, fa0, fb0, std::false_type{}, std::integral_constant<int, 3>{});
  } else {
    // short K (64 or 128): every step refills (past the end: a re-fetch of
    // the last stage into a buffer nobody reads)
    for (int kt = 2; kt < KT; kt += 2) {
      step(kt, fa0, fb0, fa1, fb1, std::false_type{}, K0{});
      step(kt + 1, fa1, fb1, fa0, fb0, std::false_type{}, K0{});
    }
  }
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
  __syncthreads();

  // ---- epilogue: stage RC rows at a time as fp32 in LDS, then store.
  // Accumulator element e of block (i, j) in lane (r16, kc) is output row
  // 16i + 4kc + e, column col_block(w, j) + r16.
  float* Cs = (float*)smem;
  if (EPI == EPI_RESID) {
    // Residual stream (fp32) += acc.  Each pass's residual rows are loaded
    // into registers while the previous pass is stored, and the barriers
    // wait only for LDS traffic, so the loads overlap the staging and the
    // stores.  The last layer's segment-token rows also go to the caller's y,
    // rounded once to bf16.
    constexpr int NPASS = (BM + RC - 1) / RC;
    bf16* Y = nullptr;
    int y_rows = 0;
    if (g.desc != nullptr && layer == g.last_layer) {
      Y = (bf16*)g.desc->y + ((int64_t)seq * g.desc->seq_rows + (int64_t)(g.desc->c - layer) * g.T) * g.ldc;
      y_rows = seg_tokens(g.desc, g.desc->c - layer, g.T);
    }
    // Stores go through buffer resources bounded to the tile's rows (and to
    // y's rows), every lane issuing each one: a piece outside the node or the
    // tile gets an offset past the bound and the hardware drops it.  Stores
    // in conditional blocks would again leave the compiler unsure what is in
    // flight (and it would wait for everything before the next piece).
    const int c_rows = max(0, min(BM, g.M - m0));
    const __amdgpu_buffer_rsrc_t c_rs = uniform_rsrc(Cf + (int64_t)m0 * g.ldc, c_rows * g.ldc * 4);
    const int y_tile_rows = Y != nullptr ? max(0, min(BM, y_rows - m0)) : 0;
    const __amdgpu_buffer_rsrc_t y_rs =
        uniform_rsrc(Y != nullptr ? (const void*)(Y + (int64_t)m0 * g.ldc) : (const void*)Cf, y_tile_rows * g.ldc * 2);
    if constexpr (!PREFETCH) load_pass(0, rb[0]);   // (else issued in the K loop's tail)
    static_for<NPASS>([&](auto PI) {
      constexpr int p = decltype(PI)::value, rc0 = RC * p;
      if (p + 1 < NPASS) load_pass(rc0 + RC, rb[(p + 1) & 1]);
      static_for<RB>([&](auto II) {
        constexpr int i = decltype(II)::value;
        if (16 * i >= rc0 && 16 * i < rc0 + RC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rl = 16 * i - rc0 + 4 * kc + e;
#pragma unroll
            for (int j = 0; j < 4; ++j) Cs[rl * CPITCH + col_block<EPI>(w, j) + r16] = acc[i][j][e];
          }
        }
      });
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(63));
      lds_barrier();
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int pc = tid + 256 * k, r = pc >> 5, c8 = (pc & 31) * 8;
        const int m = m0 + rc0 + r, n = n0 + c8;
        const bool ok = r < BM - rc0 && m < g.M && n < g.N;
        const float* sv = Cs + r * CPITCH + c8;
        const f32x4 x0 = rb[p & 1][k][0], x1 = rb[p & 1][k][1];
        const f32x4 o0 = f32x4{x0[0] + sv[0], x0[1] + sv[1], x0[2] + sv[2], x0[3] + sv[3]};
        const f32x4 o1 = f32x4{x1[0] + sv[4], x1[1] + sv[5], x1[2] + sv[6], x1[3] + sv[7]};
        const bf16x8 o = {(bf16)o0[0], (bf16)o0[1], (bf16)o0[2], (bf16)o0[3],
                          (bf16)o1[0], (bf16)o1[1], (bf16)o1[2], (bf16)o1[3]};
        const int eo = (m - m0) * g.ldc + n;   // element offset from the tile's first row
        const int cf_off = ok ? 4 * eo : kDropOffset;
        const int y_off = ok && m < y_rows ? 2 * eo : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0), c_rs, cf_off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1), c_rs, cf_off + 16, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), y_rs, y_off, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(63));
      lds_barrier();
    });
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    // U = R(silu(gate) * up) straight from the registers: with the operands
    // swapped, element e of block (i, j) in lane (r16, kc) is output row
    // 16i + r16, column col_block(w, j) + 4kc + e, and the up block j + 2
    // holds the same positions as the gate block j.  Each lane stores four
    // consecutive bf16 outputs (8 bytes) per block pair through a buffer
    // resource bounded to the tile's rows (rows past the node are dropped by
    // the bound; N is a multiple of 4).
    bf16* C = (bf16*)g.C + (int64_t)prob * g.c_stride;
    const int c_rows = max(0, min(BM, g.M - m0));
    const __amdgpu_buffer_rsrc_t u_rs = uniform_rsrc(C + (int64_t)m0 * g.ldc, c_rows * g.ldc * 2);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gt = acc[i][j][e], up = acc[i][j + 2][e];
          o[e] = (bf16)(gt * sigmoid_f(gt) * up);
        }
        const int n = n0 + 32 * w + 16 * j + 4 * kc;
        const int off = n < g.N ? 2 * ((16 * i + r16) * g.ldc + n) : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), u_rs, off, 0, 0);
      }
    return;
  }
  // Passes are separated by barriers that wait for LDS traffic only; the
  // global stores of one pass drain while the next is staged.
  constexpr int EP_PITCH = CPITCH;
  constexpr int EP_RC = RC;
  static_assert(EP_RC * EP_PITCH * 4 <= LDS_USED, "epilogue staging fits");
  for (int rc0 = 0; rc0 < BM; rc0 += EP_RC) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (16 * i < rc0 || 16 * i >= rc0 + EP_RC) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 16 * i - rc0 + 4 * kc + e;
#pragma unroll
        for (int j = 0; j < 4; ++j) Cs[rl * EP_PITCH + col_block<EPI>(w, j) + r16] = acc[i][j][e];
      }
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(63));
    lds_barrier();
    const int rows_here = (BM - rc0) < EP_RC ? (BM - rc0) : EP_RC;
    constexpr int PIECES_ROW = BN_OUT / 8;
    bf16* C = (bf16*)g.C + (int64_t)prob * g.c_stride;
    if (EPI == EPI_QKV) {
      // Q and K columns: RoPE with the partner column i +- hd/2 of the same
      // head (heads never straddle the 256-column tile: hd divides 256).  The
      // 8 columns of a piece lie in one half of one head (hd is a power of
      // two, a multiple of 16), so they share the partner offset and read 8
      // consecutive (cos, sin) pairs of the row's table.
      const int hd = g.head_dim, half = hd >> 1;
      // Work unit = (row, head, 8-wide frequency chunk): the chunk's columns
      // in both halves of the head, i and i + hd/2, rotated by the same 8
      // (cos, sin) pairs.  A row has 256 / 16 = 16 units; thread t takes row
      // t / 4 and units t % 4 + 4k, which share their frequency chunk (all of
      // them when hd = 64 or 32, two chunks when hd = 128), so the table
      // loads of a row are issued once and together.
      static_assert(EPI != EPI_QKV || EP_RC % 64 == 0, "four threads per staged row");
      const int nfc = half >> 3;                      // frequency chunks per head
#pragma unroll
      for (int rp = 0; rp < EP_RC / 64; ++rp) {
        const int r = (tid >> 2) + 64 * rp;
        const int m = m0 + rc0 + r;
        if (r >= rows_here || m >= g.M) continue;
        const float* srow = Cs + r * EP_PITCH;
        bf16* crow = C + (int64_t)m * g.ldc;
        f32x4 tcs[2][4];   // (cos, sin) x 8 for up to two frequency chunks
        int tfc[2] = {-1, -1};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int u = (tid & 3) + 4 * k;
          const int fc = u % nfc;
          const int slot = (k == 0 || fc == tfc[0]) ? 0 : 1;
          if (tfc[slot] != fc) {
            tfc[slot] = fc;
            const f32x4* cs = (const f32x4*)(g.rope_cs + ((int64_t)m * half + 8 * fc) * 2);
#pragma unroll
            for (int q = 0; q < 4; ++q) tcs[slot][q] = cs[q];
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int u = (tid & 3) + 4 * k;
          const int head = u / nfc, fc = u % nfc;
          const int c1 = head * hd + 8 * fc, c2 = c1 + half;   // tile columns of the two pieces
          const int n1 = n0 + c1, n2 = n0 + c2;
          if (n1 >= g.v_col0) continue;                       // V heads: transposed below
          const f32x4 a0 = *(const f32x4*)(srow + c1), a1 = *(const f32x4*)(srow + c1 + 4);
          const f32x4 b0 = *(const f32x4*)(srow + c2), b1 = *(const f32x4*)(srow + c2 + 4);
          const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          bf16x8 o1, o2;
          if (n1 < g.rope_cols) {
            const f32x4* t = tcs[fc == tfc[0] ? 0 : 1];
            const float cv[8] = {t[0][0], t[0][2], t[1][0], t[1][2], t[2][0], t[2][2], t[3][0], t[3][2]};
            const float sv[8] = {t[0][1], t[0][3], t[1][1], t[1][3], t[2][1], t[2][3], t[3][1], t[3][3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              o1[e] = (bf16)(av[e] * cv[e] - bv[e] * sv[e]);   // first half: x cos - partner sin
              o2[e] = (bf16)(bv[e] * cv[e] + av[e] * sv[e]);   // second half: x cos + partner sin
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              o1[e] = (bf16)av[e];
              o2[e] = (bf16)bv[e];
            }
          }
          if (n1 < g.N) *(bf16x8*)(crow + n1) = o1;
          if (n2 < g.N) *(bf16x8*)(crow + n2) = o2;
        }
      }
      // V columns, transposed: one aligned group of 16 keys of one column per
      // item.  Within the group the stored order is 0-3, 8-11, 4-7, 12-15 (the
      // k-slot order of the attention kernel's P V product), so a full group
      // is two 16-byte stores; consecutive threads take consecutive columns
      // (conflict-free LDS reads down the staged columns).
      bf16* Vt = (bf16*)g.vt + (int64_t)prob * g.vt_stride;
      const int kgroups = (rows_here + 15) / 16;
      for (int it = tid; it < kgroups * BN_OUT; it += 256) {
        const int col = it % BN_OUT, grp = it / BN_OUT;
        const int n = n0 + col;
        if (n < g.v_col0 || n >= g.N) continue;
        const int m = m0 + rc0 + 16 * grp;           // a multiple of 16
        if (m >= g.M) continue;
        bf16* dstp = Vt + (int64_t)(n - g.v_col0) * g.vt_ld;
        const float* sp = Cs + (16 * grp) * EP_PITCH + col;
        if (m + 16 <= g.M) {
          bf16x8 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = (bf16)sp[e * EP_PITCH];              // keys 0-3
            a[4 + e] = (bf16)sp[(8 + e) * EP_PITCH];    // keys 8-11
            b[e] = (bf16)sp[(4 + e) * EP_PITCH];        // keys 4-7
            b[4 + e] = (bf16)sp[(12 + e) * EP_PITCH];   // keys 12-15
          }
          *(bf16x8*)(dstp + m) = a;
          *(bf16x8*)(dstp + m + 8) = b;
        } else {
          for (int e = 0; m + e < g.M; ++e) dstp[vt_pos(m + e)] = (bf16)sp[e * EP_PITCH];
        }
      }
    } else if (EPI == EPI_STORE) {
      // fp32 output (LM-head logits)
      float* Cf = (float*)g.C + (int64_t)prob * g.c_stride;
      for (int pc = tid; pc < rows_here * PIECES_ROW; pc += 256) {
        const int r = pc / PIECES_ROW, c8 = (pc % PIECES_ROW) * 8;
        const int m = m0 + rc0 + r, n = n0 + c8;
        if (m >= g.M || n >= g.N) continue;
        const float* s = Cs + r * EP_PITCH + c8;
        float* dstp = Cf + (int64_t)m * g.ldc + n;
        *(f32x4*)dstp = f32x4{s[0], s[1], s[2], s[3]};
        *(f32x4*)(dstp + 4) = f32x4{s[4], s[5], s[6], s[7]};
      }
    } else {
      for (int pc = tid; pc < rows_here * PIECES_ROW; pc += 256) {
        const int r = pc / PIECES_ROW, c8 = (pc % PIECES_ROW) * 8;
        const int m = m0 + rc0 + r, n = n0 + c8;
        if (m >= g.M || n >= g.N) continue;
        const float* s = Cs + r * EP_PITCH + c8;
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)s[e];
        *(bf16x8*)(C + (int64_t)m * g.ldc + n) = o;
      }
    }
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(63));
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <int RB, int EPI>
static hipError_t launch_rb(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 16 * RB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN_OUT - 1) / BN_OUT) * g.P * g.batch;
  // K loops of at least six stages end with three steps that refill nothing
  if (g.K >= 6 * BK)
    hipLaunchKernelGGL((gemm_bf16_kernel<RB, EPI, true>), dim3(tiles), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<RB, EPI, false>), dim3(tiles), dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, int rb, hipStream_t st) {
  switch (rb) {
    case 4: return launch_rb<4, EPI>(g, st);
    case 6: return launch_rb<6, EPI>(g, st);
    case 8: return launch_rb<8, EPI>(g, st);
    case 9: return launch_rb<9, EPI>(g, st);
    case 10: return launch_rb<10, EPI>(g, st);
    case 11: return launch_rb<11, EPI>(g, st);
    case 12: return launch_rb<12, EPI>(g, st);
    case 13: return launch_rb<13, EPI>(g, st);
    case 14: return launch_rb<14, EPI>(g, st);
    default: return hipErrorInvalidValue;
  }
}

// Tile heights offered, in 16-row blocks.
const int kGemmRowBlocks[] = {4, 6, 8, 9, 10, 11, 12, 13, 14};
const int kGemmRowBlocksCount = 9;

hipError_t launch_gemm_bf16(const GemmArgs& g, int epi, int rb, hipStream_t st) {
  // K must be a multiple of 64 (two pipeline stages per loop trip)
  if (g.P <= 0 || g.batch <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % (2 * BK)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV:
      if (g.head_dim <= 0 || 256 % g.head_dim) return hipErrorInvalidValue;
      return launch_epi<EPI_QKV>(g, rb, st);
    case EPI_RESID: return launch_epi<EPI_RESID>(g, rb, st);
    case EPI_SWIGLU:
      // four-column output pieces
      if (g.N % 4) return hipErrorInvalidValue;
      return launch_epi<EPI_SWIGLU>(g, rb, st);
    case EPI_STORE:
      // whole 8-column output pieces
      if (g.N % 8) return hipErrorInvalidValue;
      return launch_epi<EPI_STORE>(g, rb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace armt
