// Grouped bf16 GEMM for one diagonal wave: problem p multiplies layer
// (l0 + p)'s activations by layer (l0 + p)'s weights, C = A * B^T with
// A [M, K] (row-major, K contiguous) and B [N, K] (weights, row-major
// [out, in]).  One launch covers every active layer of the wave -- the
// grouped layer of diagonal batching (Pith review of arXiv 2506.05229, "What
// carries the argument"; Figure 4 caption on grouped GEMM scaling; skill page
// "Diagonal Batching for Recurrent Memory Transformers", Implementation).
//
// CDNA4 mapping.
//  * Matrix core: v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  On MI355X it
//    sustains the full dense bf16 rate, twice that of the 16x16x32 form.
//  * Tile: a workgroup of 4 waves owns BM x 256 outputs, BM = 32 * MB rows,
//    chosen per workload to pad the n = T + M node rows little.  Each wave owns
//    all BM rows and 64 columns: MB x 2 accumulator blocks of 32 x 32
//    (32 * MB accumulator registers per lane).
//  * Operands: K advances 32 per pipeline stage.  Stages are filled straight
//    from global memory into LDS by global_load_lds_dwordx4 (no staging
//    registers), issued NS - 1 stages ahead; each 64-byte tile row keeps its
//    four 16-byte chunks XOR-swizzled so the fragment reads of 16 consecutive
//    rows hit 16 different bank groups.  The fragments of the next stage are
//    read while the MFMAs of the current one run.
//  * Schedule: tiles are numbered so that each of the 8 XCDs works through a
//    contiguous range (same layer, same weight columns, neighbouring rows of
//    every sequence of the batch), keeping the shared operand tiles in that
//    XCD's L2.
//  * Epilogue: fp32 results are staged through LDS, so every global store is a
//    coalesced 16-byte write and every bf16 rounding happens once, on the fp32
//    value:
//      EPI_QKV   : RoPE on the Q and K heads (partner column i + hd/2 read from
//                  the staged tile), bf16 store; V heads are stored transposed
//                  ([G * hd][n_pad], keys reordered within groups of 16) for
//                  the attention kernel.
//      EPI_RESID : C += acc in place on the fp32 residual stream; for the
//                  last layer the segment-token rows (fewer in a short last
//                  segment) are also written to the caller's y, rounded to bf16.
//      EPI_SWIGLU: the B tile holds 128 gate rows then the 128 matching up
//                  rows; U = R(silu(gate) * up).
//      EPI_STORE : fp32 store (LM-head logits; N a multiple of 8).
//  Every output element accumulates over K in the same order whatever MB or
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32;          // k per pipeline stage
constexpr int ROWB = BK * 2;    // bytes per tile row in a stage (64)
constexpr int BNB = 256;        // B-tile rows per stage
constexpr int RC = 64;          // epilogue rows staged per pass
constexpr int CPITCH = 256 + 4; // staged tile pitch (floats)
constexpr int LDS_BYTES = 160 * 1024;

// Stages that fit in LDS (at most 4); each holds BM + 256 rows of 64 bytes.
template <int MB>
constexpr int n_stages() {
  return (LDS_BYTES / ((32 * MB + BNB) * ROWB)) > 4 ? 4 : (LDS_BYTES / ((32 * MB + BNB) * ROWB));
}

// 16-byte chunk c (0..3) of tile row r sits at physical chunk
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1): the same logical chunk of any 8 (or 16)
// consecutive rows lands in 8 (16) different 16-byte bank groups, so fragment
// reads are conflict-free whether the LDS serves 128 or 256 bytes per cycle.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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

// First B-tile row (output column) of wave w's column block j (0, 1).
template <int EPI>
__device__ __forceinline__ int col_block(int w, int j) {
  if (EPI == EPI_SWIGLU) return j == 0 ? 32 * w : 128 + 32 * w;   // gate, matching up
  return 64 * w + 32 * j;
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

}  // namespace

template <int MB, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = 32 * MB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  constexpr int NS = n_stages<MB>();
  constexpr int STAGE = (BM + BNB) * ROWB;             // bytes per stage
  constexpr int A_INSTR = BM / 16;                     // 1 KB wave loads per stage
  constexpr int INSTR = A_INSTR + BNB / 16;
  constexpr int MAXQ = (INSTR + 3) / 4;                // loads per wave per stage
  static_assert(NS >= 3, "pipeline depth");
  static_assert(RC * CPITCH * 4 <= NS * STAGE, "epilogue staging fits");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * STAGE];

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

  // ---- direct global -> LDS loads.  A stage holds INSTR blocks of 16 tile
  // rows (A rows, then B rows), each filled by one 1 KB wave load in which
  // lane L brings tile row 16q + L/4, physical chunk L%4 (= logical chunk
  // swz(row, L%4)).  Wave w issues blocks q = w, w + 4, ...; every wave issues
  // exactly MAXQ loads per stage (a wave with fewer blocks repeats its first
  // one, rewriting identical bytes), so the vmcnt waits are constants.
  const bf16* src[MAXQ];
  int dst[MAXQ];
#pragma unroll
  for (int t = 0; t < MAXQ; ++t) {
    int q = w + 4 * t;
    q = q < INSTR ? q : w;
    const int rl = lane >> 2, pc = lane & 3;
    if (q < A_INSTR) {
      const int r = 16 * q + rl;
      int row = m0 + r;
      row = row < g.M ? row : g.M - 1;
      src[t] = A + (int64_t)row * g.lda + swz(r, pc) * 8;
      dst[t] = 16 * q * ROWB;
    } else {
      const int r = 16 * (q - A_INSTR) + rl;          // B-tile row 0..255
      int nrow = n0 + ((EPI == EPI_SWIGLU) ? (r & 127) : r);
      nrow = nrow < g.N ? nrow : g.N - 1;
      const bf16* base = (EPI == EPI_SWIGLU && r >= 128) ? B2 : B;
      src[t] = base + (int64_t)nrow * g.K + swz(r, pc) * 8;
      dst[t] = (BM + 16 * (q - A_INSTR)) * ROWB;
    }
  }
  const int KT = g.K / BK;
  // Stage kt of the K loop; tiles past the end re-fetch the last tile into a
  // stage nobody reads any more.
  auto issue = [&](int kt) {
    const int kc = kt < KT ? kt : KT - 1;
    unsigned char* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int t = 0; t < MAXQ; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(src[t] + kc * BK),
                                       (__attribute__((address_space(3))) void*)(st + dst[t]), 16, 0, 0);
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // Fragments of one stage: two 16-wide k-steps; lane (r32 = lane % 32,
  // h = lane / 32) holds k = 8h..8h+7 of its row, i.e. logical chunk 2ks + h.
  const int r32 = lane & 31, h = lane >> 5;
  bf16x8 fa0[2][MB], fb0[2][2], fa1[2][MB], fb1[2][2];
  auto read_frags = [&](int kt, bf16x8 (*fa)[MB], bf16x8 (*fb)[2]) {
    const unsigned char* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = col_block<EPI>(w, j) + r32;
        fb[ks][j] = *(const bf16x8*)(st + (BM + r) * ROWB + swz(r, 2 * ks + h) * 16);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = 32 * i + r32;
        fa[ks][i] = *(const bf16x8*)(st + r * ROWB + swz(r, 2 * ks + h) * 16);
      }
    }
  };
  auto mfma_all = [&](bf16x8 (*fa)[MB], bf16x8 (*fb)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
  };

  // prologue: stages 0 .. NS-2 in flight; stage 0 landed; its fragments read
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait((NS - 2) * MAXQ));
  lds_barrier();
  read_frags(0, fa0, fb0);
  // One pipeline step: refill the stage freed two steps ago, wait until this
  // wave's loads of stage kt+1 landed (the wait also drains this wave's LDS
  // reads, so nobody refills a stage another wave still reads), barrier, read
  // stage kt+1's fragments into the other register set, and multiply the
  // fragments of stage kt already in registers.  After the last step the
  // fragments read belong to a re-fetched stage and are never used; KT is even
  // because K is a multiple of 64.
  auto step = [&](int kt, bf16x8 (*fa_cur)[MB], bf16x8 (*fb_cur)[2], bf16x8 (*fa_nxt)[MB],
                  bf16x8 (*fb_nxt)[2]) {
    issue(kt + NS - 1);
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait((NS - 2) * MAXQ));
    lds_barrier();
    read_frags(kt + 1, fa_nxt, fb_nxt);
    mfma_all(fa_cur, fb_cur);
    // Interleave the reads with the MFMAs (one read, then one MFMA) so the
    // LDS and the matrix core work side by side; left alone, the scheduler
    // sinks each read next to the MFMA of the following step that uses it.
    constexpr int NREAD = 2 * (MB + 2), NMFMA = 4 * MB;
#pragma unroll
    for (int i = 0; i < NREAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NREAD, 0);
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, fa0, fb0, fa1, fb1);
    step(kt + 1, fa1, fb1, fa0, fb0);
  }
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
  __syncthreads();

  // ---- epilogue: stage RC rows at a time as fp32 in LDS, then store.
  // Accumulator element e of block (i, j) in lane (r32, h) is output row
  // 32i + 8(e/4) + 4h + e%4, column col_block(w, j) + r32.
  float* Cs = (float*)smem;
  if (EPI == EPI_RESID) {
    // Residual stream (fp32) += acc.  Each pass's residual rows are loaded
    // into registers while the previous pass is stored, and the barriers
    // wait only for LDS traffic, so the loads overlap the staging and the
    // stores.  The last layer's segment-token rows also go to the caller's y,
    // rounded once to bf16.
    constexpr int NPASS = (BM + RC - 1) / RC;
    constexpr int PPT = RC * (BN_OUT / 8) / 256;     // pieces per thread per pass
    float* Cf = (float*)g.C + (int64_t)prob * g.c_stride;
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
    const __amdgpu_buffer_rsrc_t c_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Cf + (int64_t)m0 * g.ldc), 0, c_rows * g.ldc * 4, kRawBuffer);
    const int y_tile_rows = Y != nullptr ? max(0, min(BM, y_rows - m0)) : 0;
    const __amdgpu_buffer_rsrc_t y_rs = __builtin_amdgcn_make_buffer_rsrc(
        Y != nullptr ? (void*)(Y + (int64_t)m0 * g.ldc) : (void*)Cf, 0, y_tile_rows * g.ldc * 2, kRawBuffer);
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
    load_pass(0, rb[0]);
    static_for<NPASS>([&](auto PI) {
      constexpr int p = decltype(PI)::value, rc0 = RC * p;
      if (p + 1 < NPASS) load_pass(rc0 + RC, rb[(p + 1) & 1]);
      static_for<MB>([&](auto II) {
        constexpr int i = decltype(II)::value;
        if (32 * i >= rc0 && 32 * i < rc0 + RC) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = 32 * i - rc0 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
            for (int j = 0; j < 2; ++j) Cs[rl * CPITCH + col_block<EPI>(w, j) + r32] = acc[i][j][e];
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
  // The SwiGLU tile has 128 output columns: with a 132-float pitch all BM rows
  // fit the stage buffers at once, so it takes a single pass.  Passes are
  // separated by barriers that wait for LDS traffic only; the global stores
  // of one pass drain while the next is staged.
  constexpr int EP_PITCH = (EPI == EPI_SWIGLU) ? 128 + 4 : CPITCH;
  constexpr int EP_RC = (EPI == EPI_SWIGLU) ? BM : RC;
  static_assert(EP_RC * EP_PITCH * 4 <= NS * STAGE, "epilogue staging fits");
  for (int rc0 = 0; rc0 < BM; rc0 += EP_RC) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (32 * i < rc0 || 32 * i >= rc0 + EP_RC) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = 32 * i - rc0 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (EPI == EPI_SWIGLU) {
          const float gt = acc[i][0][e], up = acc[i][1][e];
          Cs[rl * EP_PITCH + 32 * w + r32] = gt * sigmoid_f(gt) * up;
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) Cs[rl * EP_PITCH + col_block<EPI>(w, j) + r32] = acc[i][j][e];
        }
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

template <int MB, int EPI>
static hipError_t launch_mb(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 32 * MB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN_OUT - 1) / BN_OUT) * g.P * g.batch;
  hipLaunchKernelGGL((gemm_bf16_kernel<MB, EPI>), dim3(tiles), dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, int mb, hipStream_t st) {
  switch (mb) {
    case 2: return launch_mb<2, EPI>(g, st);
    case 3: return launch_mb<3, EPI>(g, st);
    case 4: return launch_mb<4, EPI>(g, st);
    case 5: return launch_mb<5, EPI>(g, st);
    case 6: return launch_mb<6, EPI>(g, st);
    case 7: return launch_mb<7, EPI>(g, st);
    default: return hipErrorInvalidValue;
  }
}

const int kGemmRowBlocks[] = {2, 3, 4, 5, 6, 7};
const int kGemmRowBlocksCount = 6;

hipError_t launch_gemm_bf16(const GemmArgs& g, int epi, int mb, hipStream_t st) {
  // K must be a multiple of 64 (two pipeline stages per loop trip)
  if (g.P <= 0 || g.batch <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % (2 * BK)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV:
      if (g.head_dim <= 0 || 256 % g.head_dim) return hipErrorInvalidValue;
      return launch_epi<EPI_QKV>(g, mb, st);
    case EPI_RESID: return launch_epi<EPI_RESID>(g, mb, st);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(g, mb, st);
    case EPI_STORE:
      // whole 8-column output pieces
      if (g.N % 8) return hipErrorInvalidValue;
      return launch_epi<EPI_STORE>(g, mb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace armt
