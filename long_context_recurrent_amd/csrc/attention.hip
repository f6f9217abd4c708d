// Batched causal segment attention over the nodes of one wave: every node is
// one batch element and attends only over its own n = T + M rows (segment
// tokens, then memory tokens); query head j reads key/value head
// j / (H/G) (Pith review of arXiv 2506.05229, "What carries the argument":
// batched attention inside the grouped layer; Figure 5 caption: groups are
// treated as batches).
//
// bf16 path (flash-style, CDNA4 MFMA).  Workgroup = (128-query block, query
// head, node), each of its 4 waves owning 32 queries; with four query heads
// per key/value head, (32-query block, key/value head, node), wave w owning
// the block's queries of query head 4 kvh + w.  Key tiles of 64 rows
// and the matching V^T tiles (V is stored transposed by the QKV GEMM) stream
// into LDS through buffer->LDS DMA loads, two tiles ahead, and are shared
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
// at depth), and O is rounded to bf16 once at the end.  Tile rows keep their
// 16-byte chunks XOR-swizzled so the fragment reads are free of bank
// conflicts.  Query blocks end at n (the partial block is the first) and are
// launched heaviest first over the whole grid.
#include <type_traits>

#include "armt_common.h"
#include "armt_kernels.h"

namespace armt {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Physical 16-byte chunk of logical chunk c in row r of a tile whose rows
// hold CH chunks: the same logical chunk of 8 (and of 16) consecutive rows
// falls in distinct bank groups.
template <int CH>
__device__ __forceinline__ int swzc(int r, int c) {
  if (CH == 4) return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
  if (CH == 8) return c ^ ((r ^ (r >> 3)) & 7);
  return c ^ (r & 15);
}

// buffer resource flags for raw (unswizzled, stride 0) buffer loads
constexpr int kRawBuffer = 0x00020000;

// One 16-byte-per-lane DMA of a wave into LDS (lane i's bytes at lds + 16 i)
// through a raw buffer resource [base, base + bytes): reads past the end
// return zero.  (Kept out of the kernels' lambdas: a buffer resource built
// inside a lambda of a kernel template keeps the host compiler from emitting
// the kernel's launch stub.)
__device__ __forceinline__ void buffer_to_lds(const void* base, int bytes, unsigned char* lds, int voffset) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRawBuffer);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
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
__global__ __launch_bounds__(256, HD <= 64 ? 3 : 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = HD / 8;                  // 16-byte chunks per K row
  constexpr int K_BYTES = 64 * HD * 2;        // K tile: 64 keys x HD
  constexpr int V_BYTES = HD * 64 * 2;        // V^T tile: HD rows x 64 keys
  constexpr int TILE = K_BYTES + V_BYTES;
  constexpr int NBUF = HD >= 128 ? 2 : 3;
  constexpr int K_BLOCKS = K_BYTES / 1024;    // 1 KB wave loads per tile
  static_assert(K_BLOCKS % 4 == 0, "a wave's K and V^T blocks follow from the load index alone");
  constexpr int LOADS = (TILE / 1024) / 4;    // per wave per tile
  constexpr int KROWS = 1024 / (HD * 2);      // K rows per 1 KB load
  constexpr int ES = HD / 16, DB = HD / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NBUF * TILE];

  const int n = a.n;
  const int R = a.H / a.G;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r32 = lane & 31, hh = lane >> 5;
  int layer, kvh, head, q0w, q_end;
  if (R == 4) {
    // Four query heads per K/V head: a workgroup takes 32 queries of all
    // four (wave w: query head 4 kvh + w), so every wave needs the same key
    // tiles and none idles at the tile barriers near the diagonal.  Query
    // blocks of 32 end at n, n - 32, ... (the partial block is the first);
    // workgroups run heaviest block first.
    const int per_level = a.G * a.P;
    const int level = (int)blockIdx.x / per_level;
    const int grp = (int)blockIdx.x - level * per_level;   // (node, key/value head)
    kvh = grp % a.G;
    layer = a.l0 + grp / a.G;
    head = kvh * R + w;
    q_end = n - 32 * level;                                 // > 0
    q0w = q_end - 32;                                       // may be negative in the first block
  } else {
    // Query blocks of 128 end at n, n - 128, ...: the partial block is the
    // first one, whose queries see the fewest keys.  Workgroup order: the
    // blocks heaviest first across the whole grid (longest-processing-time
    // order, so no long block starts late), and within one block index the
    // R = H/G query heads that share a key/value head dispatched to one XCD
    // back to back (workgroup i runs on XCD i % 8), so they share its L2.
    const int nqb = (n + 127) / 128;
    const int per_level = a.H * a.P;
    const int level = (int)blockIdx.x / per_level;
    int li = (int)blockIdx.x - level * per_level;
    if (((a.G * a.P) & 7) == 0) {
      const int x = li & 7, j = li >> 3;
      li = (x + 8 * (j / R)) * R + j % R;
    }
    const int qb = nqb - 1 - level;
    const int grp = li / R;                       // (node, key/value head)
    kvh = grp % a.G;
    head = kvh * R + li % R;
    layer = a.l0 + grp / a.G;
    q0w = n - 128 * (nqb - qb) + 32 * w;          // may be negative in the first block
    q_end = n - 128 * (nqb - 1 - qb);             // > 0
  }
  const bf16* qkv = (const bf16*)a.qkv + (int64_t)layer * a.qkv_stride;
  const bf16* vt = (const bf16*)a.vt + (int64_t)layer * a.vt_stride + (int64_t)kvh * HD * a.vt_ld;
  const int kcol = (a.H + kvh) * HD;

  const int q = q0w + r32;                         // < n; rows q < 0 do not exist
  const int qc = q < 0 ? 0 : q;
  const int ntile = (q_end + 63) / 64;
  const int wtiles = q0w + 32 > 0 ? (q0w + 32 + 63) / 64 : 0;

  // DMA slots: 1 KB block b = w + 4i of a tile (K blocks first, then V^T);
  // byte offset of this lane's 16 bytes from the tile's first key row / V^T
  // column.  The loads are buffer loads whose resource starts at the tile
  // (key rows past n read as zero: they are masked anyway), so a tile's
  // addresses cost scalar work only.
  int voffs[LOADS], dst[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int b = w + 4 * i;
    dst[i] = b * 1024;
    if (4 * i < K_BLOCKS) {   // == (b < K_BLOCKS): K_BLOCKS is a multiple of 4 and w < 4
      const int r = b * KROWS + lane / CH;             // key row in the tile
      voffs[i] = 2 * (r * a.ld_qkv + kcol + swzc<CH>(r, lane % CH) * 8);
    } else {
      const int dim = (b - K_BLOCKS) * 8 + lane / 8;   // V^T row
      voffs[i] = 2 * (dim * a.vt_ld + swzc<8>(dim, lane % 8) * 8);
    }
  }
  const int k_bytes = n * a.ld_qkv * 2;   // the node's key rows 0..n-1
  const int v_bytes = HD * a.vt_ld * 2;
  auto issue = [&](int t) {
    const int tt = t < ntile ? t : ntile - 1;   // past the end: a harmless re-fetch
    unsigned char* st = smem + (t % NBUF) * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (4 * i < K_BLOCKS)   // compile-time: no branch per load and tile
        buffer_to_lds(qkv + (int64_t)tt * 64 * a.ld_qkv, k_bytes - tt * 64 * a.ld_qkv * 2, st + dst[i], voffs[i]);
      else
        buffer_to_lds(vt + tt * 64, v_bytes - tt * 128, st + dst[i], voffs[i]);
    }
  };

#pragma unroll
  for (int s = 0; s < NBUF - 1; ++s) issue(s);

  bf16x8 qf[ES];
#pragma unroll
  for (int ks = 0; ks < ES; ++ks)
    qf[ks] = *(const bf16x8*)(qkv + (int64_t)qc * a.ld_qkv + head * HD + 16 * ks + 8 * hh);

  // Per-lane LDS byte offsets of this lane's K and V^T fragments inside a
  // tile buffer; the buffer's own offset is a compile-time constant below
  // (the tile loop is unrolled by NBUF), so every fragment read is a single
  // ds_read with an immediate offset.
  int koff[2][ES], voff[2][2][DB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < ES; ++ks) {
      const int r = kb * 32 + r32;
      koff[kb][ks] = r * (HD * 2) + swzc<CH>(r, 2 * ks + hh) * 16;
    }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r = db * 32 + r32;
        const int c = 2 * (2 * kb + ks) + hh;    // logical chunk of the V^T row
        voff[kb][ks][db] = K_BYTES + r * 128 + swzc<8>(r, c) * 16;
      }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // Running row statistics, in scores scaled to log2 units (s * sl2).  The
  // subtracted offset mb is not the running maximum: it is raised (to the
  // maximum, with O and the row sum rescaled) only when a tile's exponentials
  // push some lane's row sum past 2^ROWSUM_LOG2 -- which the first tile
  // always does (mb starts at -1e30, so its exponentials are infinite) and
  // later tiles do only when a score exceeds mb by tens of binades.  Until
  // then every exponential lies in [0, 2^ROWSUM_LOG2], far inside fp32 and
  // bf16 range; bf16 keeps the same relative precision at any magnitude and
  // every row holds a term >= 1 after its first rescale, so O / l is
  // unchanged.  No tile needs its row maximum, which is the bulk of the
  // softmax's vector work besides the exponentials.
  constexpr float ROWSUM_LIMIT = 4294967296.f;   // 2^32
  float mb = -1e30f, lsum0 = 0.f, lsum1 = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;   // scores in log2 units
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

  auto tile = [&](int t, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    // tile t landed (this wave's loads; the barrier covers the others'),
    // and every wave is done with tile t - 1, whose buffer is refilled next
    __builtin_amdgcn_s_waitcnt(att_wait((NBUF - 2) * LOADS));
    att_barrier();
    issue(t + NBUF - 1);
    if (t >= wtiles) return;
    const unsigned char* tb = smem + buf * TILE;

    // S^T of the tile: every K fragment is read before the first product
    // (one LDS round trip per tile, not one per product pair).  Element e of
    // block kb: key t*64 + 32kb + 8(e/4) + 4hh + e%4, query q.  Only the
    // wave's last one or two tiles reach past its first query and need the
    // causal mask: key > q <=> 32kb + 8(e/4) + e%4 > q - 64t - 4hh (rows
    // q < 0 of the first block mask every key).
    auto scores = [&](f32x16* s) {
      if constexpr (HD <= 64) {
        bf16x8 kf[2][ES];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ks = 0; ks < ES; ++ks) kf[kb][ks] = *(const bf16x8*)(tb + koff[kb][ks]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < ES; ++ks)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][ks], qf[ks], s[kb], 0, 0, 0);
        }
        // keep the reads ahead of the products (the scheduler would
        // otherwise pair each read with its product to save registers)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * ES, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * ES, 0);
      } else {
        // HD = 128: 16 fragments would not fit beside the accumulators
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < ES; ++ks) {
            const bf16x8 kf = *(const bf16x8*)(tb + koff[kb][ks]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
          }
        }
      }
      if (t * 64 + 63 > q0w) {
        const int thr = q - t * 64 - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * kb + 8 * (e >> 2) + (e & 3) > thr) s[kb][e] = -INFINITY;
      }
    };
    // The first tile always raises the softmax offset (it starts at -1e30):
    // at hd <= 64 its scores are computed once, on the raising path below
    // (at hd 128 the extra path costs more registers than it saves).
    const bool first = HD <= 64 && t == 0;
    f32x16 s[2];
    if (!first) scores(s);
    // HD <= 64: the V^T fragments are read now and land while the
    // exponentials run (at HD = 128 each is read next to its product)
    bf16x8 vf[2][2][DB];
    if constexpr (HD <= 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db) vf[kb][ks][db] = *(const bf16x8*)(tb + voff[kb][ks][db]);
      asm volatile("" ::: "memory");
    }
    // P = 2^(s sl2 - mb) in bf16, as the second operand of O^T = V^T P^T:
    // 16-key group G = 2kb + ks, slot j = element 8ks + j of block kb.  The
    // row sum adds the bf16 P that enters the product (two products against
    // (1, 1) per dot instruction).
    bf16x8 ph[2][2];
    auto exps = [&](const f32x16* s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f32x8 pv;
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * ks + j], sl2, -mb));
          ph[kb][ks] = __builtin_convertvector(pv, bf16x8);
          float& ls = ks ? lsum1 : lsum0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{ph[kb][ks][2 * j], ph[kb][ks][2 * j + 1]}, ones, ls, false);
        }
    };
    const float l0 = lsum0, l1 = lsum1;
    bool raise = first;
    if (!first) {
      exps(s);
      // the negated test also catches an infinite or NaN sum
      raise = __any(!(lsum0 + lsum1 <= ROWSUM_LIMIT));
    }
    // (rare after the first tile: the scores are recomputed rather than kept
    // live through the exponentials)
    if (raise) {
      f32x16 s2[2];
      scores(s2);
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, s2[kb][e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave)) * sl2;
      const float mnew = fmaxf(mb, mloc);
      const float alpha = __builtin_amdgcn_exp2f(mb - mnew);   // 0 on the first tile
      lsum0 = l0 * alpha;
      lsum1 = l1 * alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      mb = mnew;
      exps(s2);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if constexpr (HD > 64) vf[kb][ks][db] = *(const bf16x8*)(tb + voff[kb][ks][db]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][ks][db], ph[kb][ks], o[db], 0, 0, 0);
        }
  };
  for (int t0 = 0; t0 < ntile; t0 += NBUF) {
    tile(t0, std::integral_constant<int, 0>{});
    if (t0 + 1 < ntile) tile(t0 + 1, std::integral_constant<int, 1>{});
    if (NBUF > 2 && t0 + 2 < ntile) tile(t0 + 2, std::integral_constant<int, 2 % NBUF>{});
  }
  float lsum = lsum0 + lsum1;
  __builtin_amdgcn_s_waitcnt(att_wait(0));
  lsum += __shfl_xor(lsum, 32, kWave);
  if (q >= 0) {
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
    // the tile loads address a node's keys and V^T with 32-bit buffer offsets
    if ((int64_t)a.n * a.ld_qkv * 2 > INT32_MAX || (int64_t)a.hd * a.vt_ld * 2 > INT32_MAX) return hipErrorInvalidValue;
    // four query heads per K/V head: one workgroup per 32 queries of the four;
    // otherwise one per 128 queries of one head
    dim3 grid(a.H == 4 * a.G ? ((a.n + 31) / 32) * a.G * a.P : ((a.n + 127) / 128) * a.H * a.P);
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
