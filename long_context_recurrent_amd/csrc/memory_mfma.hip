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

// s_waitcnt immediates (gfx9 layout): vmcnt <= n with lgkmcnt = 0; lgkmcnt = 0 only
__host__ __device__ constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }
constexpr int kLgkmOnly = 0xc07f;

// Workgroup barrier that does not wait for outstanding global->LDS loads
// (callers wait for exactly what they need with s_waitcnt first).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
// Memory read fused with the attention RMSNorm, for 32 rows of one node:
//   q  = phi(h_in W_mq^T),  h = h_in + (q A^T) * (1 / (q . z + eps))   (fp32 stream)
//   a  = R(rms(h) * g_attn)                                             (bf16)
// Workgroup = 8 waves: row group rg = w / 4 (16 rows) x column set cq = w % 4.
// Columns come in 128-wide chunks s = 0 .. d/128 - 1; wave (rg, cq) owns
// columns 128 s + 32 cq .. + 31 of every chunk and keeps its 16 rows of them
// in registers from the first load to the last store: lane (c16, g) holds row
// c16, columns 128 s + 32 cq + 8 g .. + 7.  The operands of a chunk -- the
// W_mq columns [64 keys x 128] bf16 for the first product, then 128 rows of
// the state as bf16 hi / lo halves [128 x (64 + 64)] for the second -- stream
// into LDS by buffer->LDS DMA in whole 256-byte rows and are shared by both
// row groups.
//  * u = h W_mq^T on v_mfma_f32_16x16x32_bf16 with h as a bf16 pair
//    (hi = R(h), lo = R(h - hi)); the four column sets' partial u are added
//    in LDS in a fixed order.
//  * r^T = A q^T on the same instruction as three hi/lo products
//    (A_hi q_hi + A_hi q_lo + A_lo q_hi, relative error ~2^-16).  The split of
//    the fp32 state is kept beside it (A2, written by every memory update), so
//    it is formed once per node instead of by every workgroup.  The A rows
//    feeding 16x16 output block sb are the columns 8(i/4) + 4 sb + i%4 of the
//    wave's 32, so lane (c16, g) receives r for exactly the columns it holds.
// Tile rows keep their 16-byte chunks XOR-swizzled (W_mq rows by key & 15, A
// rows by (r & 3) | ((r >> 3) & 3) << 2) so the fragment reads are free of
// bank conflicts.
//
// Vector-memory operations complete in issue order, so a wait for one of
// them is "at most n outstanding" with n the operations issued after it; the
// kernel counts what it issues (a lower bound wherever a count could vary, so
// a wait is never short) and waits for exactly what the next step reads.
// Operands stay NW (phase 1) or NA (phase 2) chunks ahead of the products and
// h HA chunks ahead; each updated h chunk is stored as soon as it is formed;
// the gains and z reach LDS early, so the bf16 output waits for nothing but
// its row's RMS.  With the chunk count a template constant every wait is a
// single instruction.
template <int I = 0>
__device__ __forceinline__ void wait_vm_le(int n) {   // n wave-uniform
  if constexpr (I >= 31) {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(31));
  } else {
    if (n <= I) __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(I));
    else wait_vm_le<I + 1>(n);
  }
}

// Word 3 of a raw buffer resource on gfx9 parts (no format conversion).
constexpr int kRawBuffer = 0x00020000;

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte LDS reads of the chunk buffers, issued together and waited for in
// the same block.  Written as asm because the compiler would otherwise wait
// for every buffer->LDS load in flight before each read (it cannot tell which
// buffer a DMA fills); the explicit vmcnt waits already cover the chunk read.
__device__ __forceinline__ void lds_read4(unsigned a0, unsigned a1, unsigned a2, unsigned a3, bf16x8& r0, bf16x8& r1,
                                          bf16x8& r2, bf16x8& r3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3));
}

constexpr int kMrW = 16 * 1024;   // W_mq chunk: 64 keys x 128 columns bf16
constexpr int kMrA = 32 * 1024;   // A chunk: 128 rows x 64 keys fp32
constexpr int kMrNW = 6;          // W_mq chunk buffers (phase 1)
constexpr int kMrNA = 3;          // A chunk buffers (phase 2), same LDS
constexpr int kMrOps = kMrNW * kMrW;
static_assert(kMrNA * kMrA <= kMrOps, "operand buffers");

template <int NBM, bool EXACT, bool L0>   // EXACT: d == 128 NBM (every count below is a constant)
__device__ __forceinline__ void memread_norm_body(const MemArgs& a, unsigned char* ops, float (&ured)[2][4][16][65],
                                                  float (&qs)[32][68], float (&dens)[32], float (&ssq)[2][4][16],
                                                  float (&zs)[64], unsigned char* gsh) {
  constexpr int LW = kMrW / 1024 / 8;   // 1 KB DMA loads per wave per W_mq chunk (2)
  constexpr int LA = kMrA / 1024 / 8;   // ... per A chunk (4)
  constexpr int HO = L0 ? 1 : 2;        // loads per h chunk (bf16 x / fp32 stream)
  constexpr int SO = 2;                 // stores per h chunk
  constexpr int HA = 6;                 // h chunks loaded ahead

  const int layer = a.l0 + blockIdx.y;          // (layer, sequence) problem
  const int wl = layer / a.batch;                // model layer
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int rg = w >> 2, cq = w & 3;
  const int d = EXACT ? 128 * NBM : a.d, nb = d >> 7;
  const int rl = 16 * rg + c16;                  // row within the workgroup's 32
  const int row = blockIdx.x * 32 + rl;
  const int rowc = row < a.n ? row : a.n - 1;
  const int colw = 32 * cq + 8 * g;              // + 128 s
  // the wave holds at least one row of the node (its stores are issued)
  const bool live = blockIdx.x * 32 + 16 * rg < a.n;

  // z, for the denominators (one value per lane of wave 0)
  const float zv = w == 0 ? a.z[(int64_t)layer * 64 + lane] : 0.f;

  // h_in rows (fp32 stream, or bf16 x / memory embeddings at layer 0; the
  // rows after a short last segment's memory tokens are zero padding).  Every
  // lane loads (padding lanes from a valid row), so each chunk is HO loads.
  float hv[NBM][8];
  bf16x8 hx[NBM];
  const bf16* h0p = nullptr;
  bool pad = false;
  if constexpr (L0) {
    const int ts0 = seg_tokens(a.desc, a.desc->c, a.T);
    // at layer 0 the problem index is the sequence index
    const bf16* xs = (const bf16*)a.desc->x + (int64_t)layer * a.desc->seq_rows * d;
    pad = rowc >= ts0 + a.M;
    h0p = rowc < ts0 ? xs + ((int64_t)a.desc->c * a.T + rowc) * d
                     : (const bf16*)a.mem_emb + (int64_t)(pad ? 0 : rowc - ts0) * d;
  }
  const float* hp = L0 ? nullptr
                       : (const float*)a.act_prev + (int64_t)(layer - a.batch) * a.act_stride + (int64_t)rowc * d;
  auto load_h = [&](int s) {
    const int c = 128 * s + colw;
    if constexpr (L0) hx[s] = *(const bf16x8*)(h0p + c);
    else load8f(hp + c, hv[s]);
  };

  // chunk DMA: 1 KB block q = w + 8t covers 4 rows of 256 bytes; lane L
  // brings row 4q + L/16, physical chunk L%16.  Buffer (not global) DMA: with
  // global->LDS loads in flight the compiler waits for every outstanding
  // operation before any use of a register load (the h rows).
  const __amdgpu_buffer_rsrc_t wq_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)a.w_mq + (int64_t)wl * 64 * d), 0, 64 * d * 2, kRawBuffer);
  const __amdgpu_buffer_rsrc_t a_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.A2 + (int64_t)layer * d * 128), 0, d * 128 * 2, kRawBuffer);
  auto issue_wq = [&](int s) {
    unsigned char* buf = ops + (s % kMrNW) * kMrW;
#pragma unroll
    for (int t = 0; t < LW; ++t) {
      const int q = w + 8 * t, key = 4 * q + (lane >> 4), pc = lane & 15;
      const int off = 2 * (key * d + 128 * s + 8 * (pc ^ (key & 15)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wq_rs, (__attribute__((address_space(3))) void*)(buf + q * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  auto aswz = [](int r) { return (r & 3) | (((r >> 3) & 3) << 2); };
  // A buffer j overlays W_mq buffers 2j, 2j+1 and is free once the last W_mq
  // chunk held there has been multiplied (after phase-1 step fr[j]; -1: never
  // used).  Update-phase chunk s goes to A buffer abuf[s % NA], the first
  // chunks to the buffers freed first, so they load during phase 1.
  auto last_w = [&](int b) { return b < nb ? b + kMrNW * ((nb - 1 - b) / kMrNW) : -1; };
  int fr[kMrNA], abuf[kMrNA];
#pragma unroll
  for (int j = 0; j < kMrNA; ++j) {
    fr[j] = max(last_w(2 * j), last_w(2 * j + 1));
    abuf[j] = j;
  }
#pragma unroll
  for (int i = 0; i < kMrNA; ++i)
#pragma unroll
    for (int j = 0; j + 1 < kMrNA; ++j)
      if (fr[abuf[j]] > fr[abuf[j + 1]]) {
        const int t = abuf[j];
        abuf[j] = abuf[j + 1];
        abuf[j + 1] = t;
      }
  auto issue_a = [&](int s) {
    unsigned char* buf = ops + abuf[s % kMrNA] * kMrA;
#pragma unroll
    for (int t = 0; t < LA; ++t) {
      const int q = w + 8 * t, r = 4 * q + (lane >> 4), pc = lane & 15;
      const int off = (128 * s + r) * 256 + 16 * (pc ^ aswz(r));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (__attribute__((address_space(3))) void*)(buf + q * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  // memory operations keep the order of these calls
  auto fence = [] { asm volatile("" ::: "memory"); };
  int issued = 0;        // loads and DMA issued so far by this wave
  int stores = 0;        // h stores issued so far, counted as if the wave is live
  int tag[NBM];          // `issued` just after W_mq chunk s's DMA
  int atag[NBM];         // `issued` just after A chunk s's DMA
  int astag[NBM];        // `stores` at that point
  auto issue_a_tagged = [&](int s) {
    issue_a(s);
    issued += LA;
    atag[s] = issued;
    astag[s] = stores;
  };

  // the gains (one 1 KB block per wave, clamped into the row), needed last
  {
    const __amdgpu_buffer_rsrc_t g_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)a.gain + (int64_t)wl * d), 0, 2 * d, kRawBuffer);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g_rs, (__attribute__((address_space(3))) void*)(gsh + 1024 * w), 16,
                                             min(1024 * w + 16 * lane, 2 * d - 16), 0, 0, 0);
    issued += 1;
  }
  fence();

  // ---- u = h W_mq^T: chunk s from buffer s % NW.  Issue order: h 0..HA-1,
  // W_mq 0..NW-1; after step s: h s+HA, W_mq s+NW.
#pragma unroll
  for (int s = 0; s < HA && s < NBM; ++s)
    if (s < nb) { load_h(s); issued += HO; }
  fence();
#pragma unroll
  for (int s = 0; s < kMrNW && s < NBM; ++s)
    if (s < nb) { issue_wq(s); issued += LW; tag[s] = issued; fence(); }
  // A chunks whose buffer phase 1 never uses (all but the last of the first NA)
#pragma unroll
  for (int j = 0; j + 1 < kMrNA && j < NBM; ++j)
    if (j < nb && fr[abuf[j]] < 0) { issue_a_tagged(j); fence(); }
  f32x4 u[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) u[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NBM; ++s) {
    if (s < nb) {
      wait_vm_le(issued - tag[s]);   // W_mq chunk s in LDS (h chunk s: its registers are waited for)
      lds_barrier();
      if constexpr (L0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[s][e] = pad ? 0.f : (float)hx[s][e];
      }
      const unsigned char* buf = ops + (s % kMrNW) * kMrW;
      bf16x8 hi, lo;
      split8(hv[s], hi, lo);
      const int lc = 4 * cq + g;
      // key 16 jb + c16 of the chunk (key & 15 == c16)
      const unsigned b0 = lds_addr(buf) + c16 * 256 + ((lc ^ c16) << 4);
      bf16x8 bv[4];
      lds_read4(b0, b0 + 16 * 256, b0 + 32 * 256, b0 + 48 * 256, bv[0], bv[1], bv[2], bv[3]);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        u[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv[jb], u[jb], 0, 0, 0);
        u[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv[jb], u[jb], 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(kLgkmOnly);
      lds_barrier();
      if (s + HA < nb) { load_h(s + HA); issued += HO; }
      fence();
      if (s + kMrNW < nb) { issue_wq(s + kMrNW); issued += LW; tag[s + kMrNW] = issued; }
      fence();
      // A chunks whose buffer this step freed
#pragma unroll
      for (int j = 0; j + 1 < kMrNA && j < NBM; ++j)
        if (j < nb && fr[abuf[j]] == s) { issue_a_tagged(j); fence(); }
    }
  }
  // lane (c16, g) of block jb holds u[row 4g + i of its group][key 16 jb + c16]
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int i = 0; i < 4; ++i) ured[rg][cq][4 * g + i][16 * jb + c16] = u[jb][i];
  if (w == 0) zs[lane] = zv;
  __builtin_amdgcn_s_waitcnt(kLgkmOnly);
  lds_barrier();
  for (int idx = tid; idx < 32 * 64; idx += 512) {
    const int r = idx >> 6, k = idx & 63, gr = r >> 4, rr = r & 15;
    qs[r][k] = phi_f(((ured[gr][0][rr][k] + ured[gr][1][rr][k]) + ured[gr][2][rr][k]) + ured[gr][3][rr][k]);
  }
  __builtin_amdgcn_s_waitcnt(kLgkmOnly);
  lds_barrier();
  if (tid < 32) {
    float sd = 0.f;
    for (int k = 0; k < 64; ++k) sd = fmaf(qs[tid][k], zs[k], sd);
    dens[tid] = sd + a.mem_eps;
  }
  // q^T as the second operand of r^T = A q^T: lane (c16, g) brings
  // q[row c16 of its group][32 ks + 8 g .. + 7] as a bf16 pair
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = qs[rl][32 * ks + 8 * g + e];
    split8(v, qh[ks], ql[ks]);
  }
  __builtin_amdgcn_s_waitcnt(kLgkmOnly);
  lds_barrier();   // dens visible
  const float rden = 1.f / dens[rl];   // one division per row
  // the last of the first NA A chunks goes in after the LDS traffic above, so
  // that traffic does not wait for it (the compiler orders every LDS access
  // after all buffer->LDS loads in flight)
  fence();
  if (kMrNA - 1 < nb) issue_a_tagged(kMrNA - 1);
  fence();

  // ---- h += r^T / den, chunk by chunk from buffer s % NA, each chunk stored
  // once updated; partial sum of squares of the new h.  After step s: A s+NA,
  // then the store of h chunk s (issued by live waves only).
  float* ho = (float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)row * d;
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < NBM; ++s) {
    if (s < nb) {
      // A chunk s (and the gains before it) in LDS
      if (live) wait_vm_le(issued - atag[s] + stores - astag[s]);
      else wait_vm_le(issued - atag[s]);
      lds_barrier();
      const unsigned char* buf = ops + abuf[s % kMrNA] * kMrA;
      // A rows ar(sb) = 32 cq + 8 (c16 / 4) + 4 sb + c16 % 4 (aswz(ar) does
      // not depend on sb); keys 32 ks + 8 g .. + 7 are 16-byte chunk 4 ks + g
      // of the row's hi half and 8 + 4 ks + g of its lo half
      const int ar0 = 32 * cq + 8 * (c16 >> 2) + (c16 & 3), sw = aswz(ar0);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        bf16x8 ah[2], al[2];
        const unsigned rb = lds_addr(buf) + (ar0 + 4 * sb) * 256;
        lds_read4(rb + ((g ^ sw) << 4), rb + (((8 + g) ^ sw) << 4), rb + (((4 + g) ^ sw) << 4),
                  rb + (((12 + g) ^ sw) << 4), ah[0], al[0], ah[1], al[1]);
        f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], qh[ks], r, 0, 0, 0);
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], ql[ks], r, 0, 0, 0);
          r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], qh[ks], r, 0, 0, 0);
        }
        // lane (c16, g) holds r^T[block row 4g + i][row c16] = column 8g + 4sb + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float hn = fmaf(r[i], rden, hv[s][4 * sb + i]);
          hv[s][4 * sb + i] = hn;
          ss = fmaf(hn, hn, ss);
        }
      }
      __builtin_amdgcn_s_waitcnt(kLgkmOnly);
      lds_barrier();
      if (s + kMrNA < nb) issue_a_tagged(s + kMrNA);
      fence();
      if (row < a.n) {
        const int c = 128 * s + colw;
        const float* v = hv[s];
        *(f32x4*)(ho + c) = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4*)(ho + c + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
      stores += SO;
      fence();
    }
  }
  ss += __shfl_xor(ss, 16, kWave);
  ss += __shfl_xor(ss, 32, kWave);
  if (g == 0) ssq[rg][cq][c16] = ss;
  __builtin_amdgcn_s_waitcnt(kLgkmOnly);
  lds_barrier();
  const float rs = rsqrtf((((ssq[rg][0][c16] + ssq[rg][1][c16]) + ssq[rg][2][c16]) + ssq[rg][3][c16]) / (float)d +
                          a.rms_eps);
  if (row < a.n) {
    bf16* ao = (bf16*)a.abuf + (int64_t)layer * a.act_stride + (int64_t)row * d;
#pragma unroll
    for (int s = 0; s < NBM; ++s) {
      if (s < nb) {
        const int c = 128 * s + colw;
        const float* v = hv[s];
        const bf16x8 gv = *(const bf16x8*)(gsh + 2 * c);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * rs * (float)gv[e]);
        *(bf16x8*)(ao + c) = o;
      }
    }
  }
}

template <int NBM, bool EXACT>   // 128-column chunks: d / 128 <= NBM (EXACT: ==)
__global__ __launch_bounds__(512) void memread_norm_bf16_kernel(MemArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char ops[kMrOps];
  __shared__ __attribute__((aligned(1024))) unsigned char gsh[8 * 1024];
  __shared__ float ured[2][4][16][65];
  __shared__ float qs[32][68];
  __shared__ float dens[32];
  __shared__ float ssq[2][4][16];
  __shared__ float zs[64];
  if ((a.l0 + (int)blockIdx.y) / a.batch == 0) memread_norm_body<NBM, EXACT, true>(a, ops, ured, qs, dens, ssq, zs, gsh);
  else memread_norm_body<NBM, EXACT, false>(a, ops, ured, qs, dens, ssq, zs, gsh);
}

// ---------------------------------------------------------------------------
// Memory write, part 1.  Workgroup (jb < 4, node): keys k[:, 16jb .. 16jb+15]
// = phi(Y W_mk^T) with the 4 waves splitting d (interleaved 32-wide steps) and
// a fixed-order reduction in LDS; then the partial denominators
// sum_{j in block} k_mj z_j with the pre-update z, and z_j += sum_m k_mj for
// the block's own columns.  Workgroup jb = 4: the gates beta_m.
// ---------------------------------------------------------------------------
template <int MBK>   // 16-row blocks of memory tokens: M <= 16 * MBK
__global__ __launch_bounds__(256) void memkeys_bf16_kernel(MemArgs a) {
  __shared__ float red[4][4][64][4];   // [wave][m-block][lane][r]
  __shared__ float ks[64][17];
  const int layer = a.l0 + blockIdx.y;
  const int jb = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int d = a.d, M = a.M;
  const int wl = layer / a.batch;
  const int ts = seg_tokens(a.desc, a.desc->c - wl, a.T);      // memory rows start here
  if (jb == 0 && tid == 0) a.moff[layer] = ts;                 // for memupdate (next launch)
  const float* Y = (const float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)ts * d;
  if (jb < 4) {
    const int mblocks = MBK;
    // waves take interleaved 64-wide k chunks; lane group g brings
    // k0 + 16g .. +15 (same slot order for both operands, as in memupdate);
    // the next chunk's operands load while the current one multiplies
    const bf16* wk = (const bf16*)a.w_mk + ((int64_t)wl * 64 + 16 * jb + c16) * d + 16 * g;
    f32x4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int yrow[MBK];
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) yrow[mb] = 16 * mb + c16 < M ? 16 * mb + c16 : M - 1;
    bf16x8 bw[2][2];
    float yv[2][MBK][16];
    auto load = [&](int k0, bf16x8 (&b)[2], float (&y)[MBK][16]) {
      b[0] = *(const bf16x8*)(wk + k0);
      b[1] = *(const bf16x8*)(wk + k0 + 8);
#pragma unroll
      for (int mb = 0; mb < MBK; ++mb) {
        load8f(Y + (int64_t)yrow[mb] * d + k0 + 16 * g, y[mb]);
        load8f(Y + (int64_t)yrow[mb] * d + k0 + 16 * g + 8, y[mb] + 8);
      }
    };
    auto mul = [&](const bf16x8 (&b)[2], const float (&y)[MBK][16]) {
#pragma unroll
      for (int mb = 0; mb < MBK; ++mb) {
        bf16x8 hi0, lo0, hi1, lo1;
        split8(y[mb], hi0, lo0);
        split8(y[mb] + 8, hi1, lo1);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi0, b[0], acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo0, b[0], acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi1, b[1], acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo1, b[1], acc[mb], 0, 0, 0);
      }
    };
    int k0 = 64 * w;
    if (k0 < d) load(k0, bw[0], yv[0]);
    for (; k0 < d; k0 += 512) {
      if (k0 + 256 < d) load(k0 + 256, bw[1], yv[1]);
      mul(bw[0], yv[0]);
      if (k0 + 256 >= d) break;
      if (k0 + 512 < d) load(k0 + 512, bw[0], yv[0]);
      mul(bw[1], yv[1]);
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
    const bf16* wb = (const bf16*)a.w_beta + (int64_t)wl * d;
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
// k_mj, also stored as its bf16 hi / lo split for the next memory read.  W_mv
// is read exactly once per node.  Optionally advances the wave counter (no
// kernel of this launch reads it).
// ---------------------------------------------------------------------------
template <int MBK>   // 16-row blocks of memory tokens: M <= 16 * MBK
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
  // memory rows' offset from memkeys (this kernel advances the wave counter,
  // so it must not derive the segment from it)
  const float* Y = (const float*)a.act_cur + (int64_t)layer * a.act_stride + (int64_t)a.moff[layer] * d;
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

  // v = Y W_mv^T for the workgroup's 64 rows of W_mv.  The waves split k:
  // wave w takes the 64-wide steps w, w + 4, ...  In a step, lane group g
  // brings k0 + 16g .. +15 of a row (32 bytes of W_mv; a whole 128-byte line
  // per row across the four groups) and feeds them to two MFMAs (slots
  // k0 + 16g + j, then k0 + 16g + 8 + j); the Y operand, split into its bf16
  // pair once per step, uses the same slot order and serves the four 16-row
  // blocks of W_mv -- so each wave reads its quarter of Y once, not all of it.
  // The next step's operands load into a second register set while a step
  // multiplies; the four waves' partial sums are added in LDS in wave order.
  const bf16* wv = (const bf16*)a.w_mv + ((int64_t)(layer / a.batch) * d + i0 + c16) * d + 16 * g;
  f32x4 acc[4][MBK];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int yrow[MBK];
#pragma unroll
  for (int mb = 0; mb < MBK; ++mb) yrow[mb] = 16 * mb + c16 < M ? 16 * mb + c16 : M - 1;
  bf16x8 bw[2][4][2];
  float yv[2][MBK][16];
  auto load = [&](int k0, bf16x8 (&b)[4][2], float (&y)[MBK][16]) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      b[rb][0] = *(const bf16x8*)(wv + (int64_t)16 * rb * d + k0);
      b[rb][1] = *(const bf16x8*)(wv + (int64_t)16 * rb * d + k0 + 8);
    }
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) {
      load8f(Y + (int64_t)yrow[mb] * d + k0 + 16 * g, y[mb]);
      load8f(Y + (int64_t)yrow[mb] * d + k0 + 16 * g + 8, y[mb] + 8);
    }
  };
  auto mul = [&](const bf16x8 (&b)[4][2], const float (&y)[MBK][16]) {
#pragma unroll
    for (int mb = 0; mb < MBK; ++mb) {
      bf16x8 hi0, lo0, hi1, lo1;
      split8(y[mb], hi0, lo0);
      split8(y[mb] + 8, hi1, lo1);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi0, b[rb][0], acc[rb][mb], 0, 0, 0);
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo0, b[rb][0], acc[rb][mb], 0, 0, 0);
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi1, b[rb][1], acc[rb][mb], 0, 0, 0);
        acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo1, b[rb][1], acc[rb][mb], 0, 0, 0);
      }
    }
  };
  const int ksteps = d >> 6;
  int st = w;
  if (st < ksteps) load(64 * st, bw[0], yv[0]);
  for (; st < ksteps; st += 8) {
    if (st + 4 < ksteps) load(64 * (st + 4), bw[1], yv[1]);
    mul(bw[0], yv[0]);
    if (st + 4 >= ksteps) break;
    if (st + 8 < ksteps) load(64 * (st + 8), bw[0], yv[0]);
    mul(bw[1], yv[1]);
  }
  // lane holds wave w's partial v[m = 16mb + 4g + r][i = i0 + 16rb + c16];
  // vvs = ((w0 + w1) + w2) + w3
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 16 * mb + 4 * g + r;
            if (m < M) vvs[m][16 * rb + c16] = (ww == 0 ? 0.f : vvs[m][16 * rb + c16]) + acc[rb][mb][r];
          }
    }
    __syncthreads();
  }
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
    const float v = At[ii][j] + s;
    A[(int64_t)(i0 + ii) * 64 + j] = v;
    const bf16 hi = (bf16)v;
    bf16* a2 = a.A2 + ((int64_t)layer * d + i0 + ii) * 128 + j;
    a2[0] = hi;
    a2[64] = (bf16)(v - (float)hi);
  }
  if (a.advance != 0 && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) a.desc->c += a.advance;
}

// ---------------------------------------------------------------------------
hipError_t launch_mem_read_bf16(const MemArgs& m, hipStream_t st) {
  // 128-column chunks; up to 24 held per wave
  if (m.dk != 64 || m.d % 128 || m.d > 3072) return hipErrorInvalidValue;
  const dim3 grid((m.n + 31) / 32, m.P);
  const int nb = m.d / 128;
  switch (nb) {   // the common widths with constant wait counts, others counted at run time
    case 1: hipLaunchKernelGGL((memread_norm_bf16_kernel<1, true>), grid, dim3(512), 0, st, m); break;
    case 2: hipLaunchKernelGGL((memread_norm_bf16_kernel<2, true>), grid, dim3(512), 0, st, m); break;
    case 4: hipLaunchKernelGGL((memread_norm_bf16_kernel<4, true>), grid, dim3(512), 0, st, m); break;
    case 6: hipLaunchKernelGGL((memread_norm_bf16_kernel<6, true>), grid, dim3(512), 0, st, m); break;
    case 8: hipLaunchKernelGGL((memread_norm_bf16_kernel<8, true>), grid, dim3(512), 0, st, m); break;
    case 16: hipLaunchKernelGGL((memread_norm_bf16_kernel<16, true>), grid, dim3(512), 0, st, m); break;
    case 24: hipLaunchKernelGGL((memread_norm_bf16_kernel<24, true>), grid, dim3(512), 0, st, m); break;
    default:
      if (nb <= 8) hipLaunchKernelGGL((memread_norm_bf16_kernel<8, false>), grid, dim3(512), 0, st, m);
      else if (nb <= 16) hipLaunchKernelGGL((memread_norm_bf16_kernel<16, false>), grid, dim3(512), 0, st, m);
      else hipLaunchKernelGGL((memread_norm_bf16_kernel<24, false>), grid, dim3(512), 0, st, m);
  }
  return hipGetLastError();
}

namespace {
__global__ void split_state_kernel(const float* A, bf16* A2, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float v = A[i];
  const bf16 hi = (bf16)v;
  bf16* o = A2 + (i >> 6) * 128 + (i & 63);
  o[0] = hi;
  o[64] = (bf16)(v - (float)hi);
}
}  // namespace

hipError_t launch_split_state(const float* A, bf16* A2, int64_t rows, hipStream_t st) {
  const int64_t count = rows * 64;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, A, A2, count);
  return hipGetLastError();
}

hipError_t launch_mem_keys_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 64) return hipErrorInvalidValue;
  const dim3 grid(5, m.P);
  if (m.M <= 16) hipLaunchKernelGGL(memkeys_bf16_kernel<1>, grid, dim3(256), 0, st, m);
  else if (m.M <= 32) hipLaunchKernelGGL(memkeys_bf16_kernel<2>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(memkeys_bf16_kernel<4>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_mem_update_bf16(const MemArgs& m, hipStream_t st) {
  if (m.dk != 64 || m.M > 64 || m.d % 64) return hipErrorInvalidValue;
  const dim3 grid(m.d / 64, m.P);
  if (m.d % 128) return hipErrorInvalidValue;
  if (m.M <= 16) hipLaunchKernelGGL(memupdate_bf16_kernel<1>, grid, dim3(256), 0, st, m);
  else if (m.M <= 32) hipLaunchKernelGGL(memupdate_bf16_kernel<2>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(memupdate_bf16_kernel<4>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace armt
