// gfx950 kernels of the block-causal renderer attention backward.
//
//  bc_prep     per query row and head: -lse*log2(e) and rowsum(dO * O)
//  bc_dq<D>    dQ, query-major: item = (chunk, head, 256 queries); over the
//              chunk's key tiles S^T = K Q^T, dP^T = V dO^T,
//              dS^T = P^T * (dP^T - rowsum), dQ^T += K^T dS^T
//  bc_dkv<D,.> dK or dV, key-major: item = (source, head, 256 keys); over
//              the query tiles of every chunk that reads the source
//              S = Q K^T, then dV^T += dO^T P, or dP = dO V^T and dK^T += Q^T dS
//  *_f32       plain fp32 paths (one lane per row and head)
//
// The MFMA kernels split the work so that no gradient needs atomics: each
// query row's dQ and each key row's dK and dV are owned by one workgroup, at
// the price of computing S three times and dP twice.
//
// Page cited: [S] "In-Flight KV Cache with Clean Anchors for Faster
// Autoregressive Video Diffusion", Korean summary page, section "how it
// works", training paragraph: the renderer runs as one block-causal forward
// over the clip so that gradients reach earlier chunks and the anchors.
#include <hip/hip_runtime.h>

#include "../ff_internal.h"
#include "ff_prof.h"
#include "ff_tile.h"

namespace ff {
namespace {

constexpr int kDqWaves = 8;              // two per SIMD, 32 queries each
constexpr int kKeyWaves = 8;             // two per SIMD, 32 keys each
constexpr int kKeyBlock = kKeyWaves * 32;

// This wave's share of the copies of one rows tile (rows o .. o+63 of a
// [n][D] block) into LDS; rows at or past n read as zeros.
template <int D, int NW>
__device__ __forceinline__ void copy_rows(const __bf16* rows, int n, int o, const LaneConst<D, NW>& lc, uint8_t* buf,
                                          int w) {
  using Cfg = TileCfg<D, NW>;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(rows + int64_t(o) * D, uint32_t(n - o) * D * 2);
#pragma unroll
  for (int j = 0; j < Cfg::kKBlocks; ++j) dma16(r, lc.kdma[j], buf + (w * Cfg::kKBlocks + j) * 1024);
}

// Lane offsets of the transposed-tile copies for blocks with n columns.
template <int D, int NW, int NB>
__device__ __forceinline__ void tr_offsets(uint32_t (&off)[NB], int n, int w, int lane) {
  using Cfg = TileCfg<D, NW>;
  static_assert(NB == Cfg::kVBlocks, "one offset per transposed-tile copy of this wave");
#pragma unroll
  for (int j = 0; j < Cfg::kVBlocks; ++j) {
    const int dd = (w * Cfg::kVBlocks + j) * 8 + lane / 8;
    off[j] = uint32_t(dd * n * 2 + (((lane & 7) ^ vrow_swz(dd)) << 4));
  }
}

// This wave's share of the copies of one transposed tile (columns o .. o+63
// of a [D][n] block).  Columns past n read the next row's first values (or
// zeros after the last row); they meet zero weights.
template <int D, int NW, int NB>
__device__ __forceinline__ void copy_tr(const __bf16* tr, int n, int o, const uint32_t (&off)[NB], uint8_t* buf, int w) {
  using Cfg = TileCfg<D, NW>;
  static_assert(NB == Cfg::kVBlocks, "one offset per transposed-tile copy of this wave");
  const __amdgpu_buffer_rsrc_t r = make_rsrc(tr + o, uint32_t(D * n - o) * 2);
#pragma unroll
  for (int j = 0; j < Cfg::kVBlocks; ++j) dma16(r, off[j], buf + (w * Cfg::kVBlocks + j) * 1024);
}

// One 32-row half of a backward tile as a single stream of LDS operand
// reads, each issued kBwdAhead MFMAs before its use (every read feeds one
// MFMA, which alone does not cover the read's latency):
//   the score MFMAs  sc += A x areg (A = rows tile abuf) and, with kDP,
//                    dp += G x greg (G = rows tile gbuf), alternating so that
//                    the two accumulator chains interleave;
//   pre()            at the last score MFMA (loads the valu step's inputs);
//   valu(sc, dp, ob) the weights of the half as two bf16 B operands;
//   the accumulation acc[db] += T[32*db ..][half] x ob (T = transposed tile
//                    tbuf), whose first reads are in flight under the valu.
constexpr int kBwdAhead = 3;

template <int D, int NW, bool kDP, typename Pre, typename Valu>
__device__ __forceinline__ void bwd_half(const uint8_t* abuf, const uint8_t* gbuf, const uint8_t* tbuf, int half,
                                         const LaneConst<D, NW>& lc, const bf16x8 (&areg)[1][D / 16],
                                         const bf16x8 (&greg)[1][D / 16], f32x16 (&acc)[D / 32], Pre&& pre,
                                         Valu&& valu) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int NSC = kDP ? 2 * KS : KS;       // score MFMAs
  constexpr int N = NSC + 2 * DB;              // + accumulation MFMAs
  auto rd = [&](int k) {
    if (k < NSC) {
      const int ks = kDP ? k >> 1 : k;
      const uint8_t* buf = (kDP && (k & 1)) ? gbuf : abuf;
      return __builtin_bit_cast(bf16x8, ld16(buf + lc.kread[ks] + half * 32 * D * 2));
    }
    const int m = k - NSC, j = m / DB, db = m % DB;
    return __builtin_bit_cast(
        bf16x8, ld16(tbuf + (int32_t(lc.vread[half][j]) - int32_t(kLdsBias)) + db * 32 * kBlockN * 2));
  };
  f32x16 sc = {}, dp = {};
  bf16x8 ob[2];
  bf16x8 op[kBwdAhead + 1];
#pragma unroll
  for (int j = 0; j < kBwdAhead; ++j) op[j] = rd(j);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    op[kBwdAhead] = op[kBwdAhead - 1];
    if (k + kBwdAhead < N) op[kBwdAhead] = rd(k + kBwdAhead);
    if (k == NSC - 1) pre();
    __builtin_amdgcn_sched_barrier(0);
    if (k == NSC) {
      valu(sc, dp, ob);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (k < NSC) {
      const int ks = kDP ? k >> 1 : k;
      if (kDP && (k & 1)) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[0], greg[0][ks], dp, 0, 0, 0);
      else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[0], areg[0][ks], sc, 0, 0, 0);
    } else {
      const int m = k - NSC, j = m / DB, db = m % DB;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[0], ob[j], acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kBwdAhead; ++j) op[j] = op[j + 1];
  }
}

// Row r of a bf16 token-major tensor, head h, as this lane's B operand over
// head_dim: 8 values per 16-wide k-step (zeros when !ok).
template <int D>
__device__ __forceinline__ void load_b_operand(const void* base, int64_t row, int nh, int h, bool ok, int hl,
                                               bf16x8 (&reg)[1][D / 16]) {
  const __bf16* p = static_cast<const __bf16*>(base) + ((ok ? row : 0) * nh + h) * D + 8 * hl;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 v = ld16(p + 16 * ks);
    if (!ok) v = u32x4{0u, 0u, 0u, 0u};
    reg[0][ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Transposed accumulator (acc[db][r] = X^T[32*db + 8*(r/4) + 4*hl + r%4][lane
// column]) times `scale`, stored as bf16 row `row`, head h of a token-major tensor.
template <int D>
__device__ __forceinline__ void store_rows(void* base, int64_t row, int nh, int h, int hl, float scale,
                                           const f32x16 (&acc)[D / 32]) {
  __bf16* op = static_cast<__bf16*>(base) + (row * nh + h) * D + 4 * hl;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[db][4 * g + e] * scale);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g) = ov;
    }
}

// --------------------------------------------------------------------------
// Per-row statistics: stats[(i*nh + h)*L + q] = {-lse*log2(e), rowsum(dO*O)}.
// D/EPT consecutive lanes share a (row, head) and reduce with lane shuffles.
// --------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(256) void bc_prep_kernel(const BcLaunch b) {
  constexpr int EPT = 16 / sizeof(E);             // elements per lane
  constexpr int TPR = D / EPT;                    // lanes per (row, head), divides 64
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t g = t / TPR;                      // token row * nh + head
  const int c = int(t % TPR);
  if (g >= int64_t(b.n_chunk) * b.L * b.nh) return;   // whole groups leave together
  const u32x4 x = ld16(static_cast<const E*>(b.dO) + g * D + c * EPT);
  const u32x4 y = ld16(static_cast<const E*>(b.O) + g * D + c * EPT);
  const E* xe = reinterpret_cast<const E*>(&x);
  const E* ye = reinterpret_cast<const E*>(&y);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc = fmaf(float(xe[e]), float(ye[e]), acc);
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (c == 0) {
    const int64_t row = g / b.nh;
    const int h = int(g % b.nh);
    const int64_t i = row / b.L, q = row % b.L;
    const int64_t idx = (i * b.nh + h) * b.L + q;
    b.stats[2 * idx] = -b.lse[idx] * kLog2e;
    b.stats[2 * idx + 1] = acc;
  }
}

// --------------------------------------------------------------------------
// dQ (bf16 MFMA).  Wave w owns queries 32w .. 32w+31 of the item's 256; per
// 64-key tile and 32-key half (lane = query column, registers = keys):
//   S^T  = K Q^T          A = K rows (LDS),  B = Q (registers)
//   dP^T = V dO^T         A = V rows (LDS),  B = dO (registers)
//   dS^T = P^T * (dP^T - rowsum),  P^T = 2^(S^T*scale*log2e - lse*log2e)
//   dQ^T += K^T dS^T      A = K^T (LDS),     B = dS^T (bf16, registers)
// Tiles are double-buffered: the copies of tile t+1 run under the math of t.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDqWaves * 64, 1) void bc_dq_kernel(const BcLaunch b) {
  constexpr int NW = kDqWaves;
  constexpr int KS = D / 16, DB = D / 32;
  using Cfg = TileCfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t kr0[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kr1[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vr0[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vr1[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kt0[Cfg::kVBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kt1[Cfg::kVBytes];

  const int n_qt = (b.L + kBlockM - 1) / kBlockM;
  const int item = xcd_remap(blockIdx.x, gridDim.x, b.n_xcd);     // q-tiles of one (chunk, head) share an XCD
  const int qt = item % n_qt;
  const int h = (item / n_qt) % b.nh;
  const int i = item / (n_qt * b.nh);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int q = qt * kBlockM + w * 32 + l32;
  const bool qok = q < b.L;
  const int64_t row = int64_t(i) * b.L + q;

  bf16x8 qreg[1][KS], greg[1][KS];
  load_b_operand<D>(b.Q, row, b.nh, h, qok, hl, qreg);
  load_b_operand<D>(b.dO, row, b.nh, h, qok, hl, greg);
  const int64_t sidx = (int64_t(i) * b.nh + h) * b.L + (qok ? q : 0);
  const float nl = qok ? b.stats[2 * sidx] : 0.f;
  const float dl = qok ? b.stats[2 * sidx + 1] : 0.f;
  const float c = b.scale * kLog2e;

  LaneConst<D, NW> lc;
  lane_const<D, NW>(lc, w, lane);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // Key sources: anchors a0 .. a0+na-1 (T keys each), then chunks j0 .. j0+nj-1 (L keys each).
  const BcChunk ch = b.chunk[i];
  const int nsrc = ch.na + ch.nj;
  const int ntiles = ch.na * ((b.T + kBlockN - 1) / kBlockN) + ch.nj * ((b.L + kBlockN - 1) / kBlockN);
  int s = 0, n = 0, o = 0;
  const __bf16 *krow = nullptr, *vrow = nullptr, *ktr = nullptr;
  uint32_t toff[Cfg::kVBlocks];
  auto set_source = [&](int s_) {
    s = s_;
    const bool anc = s < ch.na;
    const uint8_t* kv = anc ? b.kv_anchor + int64_t(ch.a0 + s) * b.blk_anchor
                            : b.kv_chunk + int64_t(ch.j0 + s - ch.na) * b.blk_chunk;
    const uint8_t* vk = anc ? b.vk_anchor + int64_t(ch.a0 + s) * b.blk_anchor
                            : b.vk_chunk + int64_t(ch.j0 + s - ch.na) * b.blk_chunk;
    n = anc ? b.T : b.L;
    krow = reinterpret_cast<const __bf16*>(kv) + int64_t(h) * n * D;
    vrow = reinterpret_cast<const __bf16*>(vk) + int64_t(h) * n * D;
    ktr = reinterpret_cast<const __bf16*>(vk) + int64_t(b.nh) * n * D + int64_t(h) * D * n;
    tr_offsets<D, NW>(toff, n, w, lane);
    o = 0;
  };
  // Copies of the cursor's tile into buffer set p; returns its valid keys.
  auto issue = [&](int p) -> int {
    copy_rows<D, NW>(krow, n, o, lc, p ? kr1 : kr0, w);
    copy_rows<D, NW>(vrow, n, o, lc, p ? vr1 : vr0, w);
    copy_tr<D, NW>(ktr, n, o, toff, p ? kt1 : kt0, w);
    const int valid = min(kBlockN, n - o);
    o += kBlockN;
    if (o >= n && s + 1 < nsrc) set_source(s + 1);
    return valid;
  };

  set_source(0);
  int valid = issue(0);
  if (qt * kBlockM + w * 32 >= b.L) {
    // No query row of this wave exists (the last tile of a chunk): it keeps
    // its part of the copies and the barriers and leaves its SIMD to the
    // other wave.
    for (int t = 0; t < ntiles; ++t) {
      wait_dma();
      __syncthreads();
      if (t + 1 < ntiles) issue((t & 1) ^ 1);
    }
    return;
  }
  for (int t = 0; t < ntiles; ++t) {
    const int p = t & 1;
    wait_dma();
    __syncthreads();                      // tile t landed everywhere; tile t-1's buffers are free
    const int valid_next = t + 1 < ntiles ? issue(p ^ 1) : 0;
    const uint8_t* kb = p ? kr1 : kr0;
    const uint8_t* vb = p ? vr1 : vr0;
    const uint8_t* tb = p ? kt1 : kt0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int lim = valid - 32 * half;
      bwd_half<D, NW, true>(
          kb, vb, tb, half, lc, qreg, greg, acc, [] {},
          [&](f32x16& sc, const f32x16& dp, bf16x8 (&dsb)[2]) {
            if (lim < 32) mask_half(sc, lim, hl);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(sc[8 * j + e], c, nl));
                dsb[j][e] = (__bf16)(pv * (dp[8 * j + e] - dl));
              }
          });
    }
    valid = valid_next;
  }
  if (qok) store_rows<D>(b.dQ, row, b.nh, h, hl, b.scale, acc);
}

// --------------------------------------------------------------------------
// dK or dV (bf16 MFMA), key-major.  Wave w owns keys 32w .. 32w+31 of the
// item's 256; per 64-query tile and 32-query half (lane = key column,
// registers = queries):
//   S  = Q K^T            A = Q rows (LDS),   B = K (registers)
//   P  = 2^(S*scale*log2e - lse*log2e)
// dV:  dV^T += dO^T P     A = dO^T (LDS),     B = P (bf16)
// dK:  dP = dO V^T        A = dO rows (LDS),  B = V (registers)
//      dS = P * (dP - rowsum),  dK^T += Q^T dS   A = Q^T (LDS), B = dS (bf16)
// dK and dV run as two kernels: one kernel holding K, V, dK and dV for its
// keys needs more than the 256 registers of a wave that shares its SIMD, and
// with a single wave per SIMD nothing hides the operand reads.  The per-query
// statistics of a tile (512 bytes) are copied with it.
// --------------------------------------------------------------------------
template <int D, bool kDK>
__global__ __launch_bounds__(kKeyWaves * 64, 1) void bc_dkv_kernel(const BcLaunch b) {
  constexpr int NW = kKeyWaves;
  constexpr int KS = D / 16, DB = D / 32;
  using Cfg = TileCfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t qr0[Cfg::kKBytes];   // Q rows
  __shared__ __attribute__((aligned(1024))) uint8_t qr1[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t gr0[kDK ? Cfg::kKBytes : 1024];   // dO rows (dK)
  __shared__ __attribute__((aligned(1024))) uint8_t gr1[kDK ? Cfg::kKBytes : 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t tt0[Cfg::kVBytes];   // Q^T (dK) or dO^T (dV)
  __shared__ __attribute__((aligned(1024))) uint8_t tt1[Cfg::kVBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st0[1024];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[1024];

  // Items: chunk sources first (they have the most readers), then anchors.
  const int nkb_c = (b.L + kKeyBlock - 1) / kKeyBlock;
  const int nkb_a = (b.T + kKeyBlock - 1) / kKeyBlock;
  int item = xcd_remap(blockIdx.x, gridDim.x, b.n_xcd);     // key blocks of one (source, head) share an XCD
  const bool is_chunk = item < b.n_chunk * b.nh * nkb_c;
  int src, n, h, kb;
  if (is_chunk) {
    kb = item % nkb_c;
    h = (item / nkb_c) % b.nh;
    src = item / (nkb_c * b.nh);
    n = b.L;
  } else {
    item -= b.n_chunk * b.nh * nkb_c;
    kb = item % nkb_a;
    h = (item / nkb_a) % b.nh;
    src = item / (nkb_a * b.nh);
    n = b.T;
  }
  const BcReaders rd = b.readers[is_chunk ? kBcMaxAnchors + src : src];
  const int64_t row0 = int64_t(src) * n;          // first token row of the source

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int key = kb * kKeyBlock + w * 32 + l32;
  const bool kok = key < n;

  bf16x8 kreg[1][KS], vreg[1][KS];
  load_b_operand<D>(is_chunk ? b.K : b.Ka, row0 + key, b.nh, h, kok, hl, kreg);
  if (kDK) load_b_operand<D>(is_chunk ? b.V : b.Va, row0 + key, b.nh, h, kok, hl, vreg);
  const float c = b.scale * kLog2e;

  LaneConst<D, NW> lc;
  lane_const<D, NW>(lc, w, lane);
  uint32_t toff[Cfg::kVBlocks];
  tr_offsets<D, NW>(toff, b.L, w, lane);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int nqt = (b.L + kBlockN - 1) / kBlockN;
  const int ntiles = rd.n * nqt;
  auto issue = [&](int t, int p) -> int {
    const int i = rd.i0 + t / nqt;
    const int o = (t % nqt) * kBlockN;
    const __bf16* qq = reinterpret_cast<const __bf16*>(b.qq_chunk + int64_t(i) * b.blk_chunk);
    const __bf16* gg = reinterpret_cast<const __bf16*>(b.gg_chunk + int64_t(i) * b.blk_chunk);
    const int64_t rows = int64_t(h) * b.L * D, tr = int64_t(b.nh) * b.L * D + int64_t(h) * D * b.L;
    copy_rows<D, NW>(qq + rows, b.L, o, lc, p ? qr1 : qr0, w);
    if (kDK) copy_rows<D, NW>(gg + rows, b.L, o, lc, p ? gr1 : gr0, w);
    copy_tr<D, NW>((kDK ? qq : gg) + tr, b.L, o, toff, p ? tt1 : tt0, w);
    if (w == 0) {
      // 64 queries x {-lse*log2e, rowsum}: the first 512 bytes of a 1 KB copy.
      const float* sp = b.stats + 2 * ((int64_t(i) * b.nh + h) * b.L + o);
      dma16(make_rsrc(sp, uint32_t(b.L - o) * 8), uint32_t(lane) * 16, p ? st1 : st0);
    }
    return min(kBlockN, b.L - o);
  };

  int valid = ntiles > 0 ? issue(0, 0) : 0;
  if (kb * kKeyBlock + w * 32 >= n) {
    // No key of this wave exists (the last block of a source): it keeps its
    // part of the copies and the barriers and leaves its SIMD to the other
    // wave.  (Wave 0, which also copies the row statistics, always has keys.)
    for (int t = 0; t < ntiles; ++t) {
      wait_dma();
      __syncthreads();
      if (t + 1 < ntiles) issue(t + 1, (t & 1) ^ 1);
    }
    return;
  }
  for (int t = 0; t < ntiles; ++t) {
    const int p = t & 1;
    wait_dma();
    __syncthreads();                      // tile t landed everywhere; tile t-1's buffers are free
    const int valid_next = t + 1 < ntiles ? issue(t + 1, p ^ 1) : 0;
    const uint8_t* qb = p ? qr1 : qr0;
    const uint8_t* gb = p ? gr1 : gr0;
    const uint8_t* tb = p ? tt1 : tt0;
    const float* stb = reinterpret_cast<const float*>(p ? st1 : st0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int lim = valid - 32 * half;
      // The statistics of the half's queries: registers 8j .. 8j+7 hold
      // queries 32*half + 16j + 8*hl + 0..7.
      float4 stv[2][4];
      bwd_half<D, NW, kDK>(
          qb, gb, tb, half, lc, kreg, vreg, acc,
          [&] {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                stv[j][u] = reinterpret_cast<const float4*>(stb + 2 * (32 * half + 16 * j + 8 * hl))[u];
          },
          [&](f32x16& sc, const f32x16& dp, bf16x8 (&ob)[2]) {
            if (lim < 32) mask_half(sc, lim, hl);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float4 v = stv[j][e >> 1];
                const float nl = (e & 1) ? v.z : v.x, dl = (e & 1) ? v.w : v.y;
                const float pv = __builtin_amdgcn_exp2f(fmaf(sc[8 * j + e], c, nl));
                ob[j][e] = kDK ? (__bf16)(pv * (dp[8 * j + e] - dl)) : (__bf16)pv;
              }
          });
    }
    valid = valid_next;
  }
  if (kok) {
    if (kDK) store_rows<D>(is_chunk ? b.dK : b.dKa, row0 + key, b.nh, h, hl, b.scale, acc);
    else store_rows<D>(is_chunk ? b.dV : b.dVa, row0 + key, b.nh, h, hl, 1.0f, acc);
  }
}

// --------------------------------------------------------------------------
// fp32 paths: one lane per (query row, head) for dQ and per (key row, head)
// for dK/dV, reading the token-major inputs directly.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bc_dq_f32_kernel(const BcLaunch b) {
  const int64_t g = int64_t(blockIdx.x) * 64 + threadIdx.x;
  if (g >= int64_t(b.n_chunk) * b.L * b.nh) return;
  const int nh = b.nh, h = int(g % nh);
  const int64_t row = g / nh;
  const int i = int(row / b.L), q = int(row % b.L);
  const float* qp = static_cast<const float*>(b.Q) + g * D;
  const float* gp = static_cast<const float*>(b.dO) + g * D;
  const int64_t sidx = (int64_t(i) * nh + h) * b.L + q;
  const float nl = b.stats[2 * sidx], dl = b.stats[2 * sidx + 1];
  const float c = b.scale * kLog2e;
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  const BcChunk ch = b.chunk[i];
  for (int s = 0; s < ch.na + ch.nj; ++s) {
    const bool anc = s < ch.na;
    const int n = anc ? b.T : b.L;
    const int64_t r0 = anc ? int64_t(ch.a0 + s) * b.T : int64_t(ch.j0 + s - ch.na) * b.L;
    const float* kb = static_cast<const float*>(anc ? b.Ka : b.K);
    const float* vb = static_cast<const float*>(anc ? b.Va : b.V);
    for (int j = 0; j < n; ++j) {
      const float* kr = kb + ((r0 + j) * nh + h) * D;
      const float* vr = vb + ((r0 + j) * nh + h) * D;
      float sdot = 0.f, gdot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        sdot = fmaf(qp[e], kr[e], sdot);
        gdot = fmaf(gp[e], vr[e], gdot);
      }
      const float ds = __builtin_amdgcn_exp2f(fmaf(sdot, c, nl)) * (gdot - dl);
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, kr[e], acc[e]);
    }
  }
  float* op = static_cast<float*>(b.dQ) + g * D;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * b.scale;
}

template <int D>
__global__ __launch_bounds__(64) void bc_dkv_f32_kernel(const BcLaunch b) {
  const int64_t g = int64_t(blockIdx.x) * 64 + threadIdx.x;
  const int64_t chunk_rows = int64_t(b.n_chunk) * b.L;
  if (g >= (chunk_rows + int64_t(b.n_anchor) * b.T) * b.nh) return;
  const int nh = b.nh, h = int(g % nh);
  int64_t row = g / nh;
  const bool is_chunk = row < chunk_rows;
  if (!is_chunk) row -= chunk_rows;
  const int src = int(is_chunk ? row / b.L : row / b.T);
  const BcReaders rd = b.readers[is_chunk ? kBcMaxAnchors + src : src];
  const float* kr = static_cast<const float*>(is_chunk ? b.K : b.Ka) + (row * nh + h) * D;
  const float* vr = static_cast<const float*>(is_chunk ? b.V : b.Va) + (row * nh + h) * D;
  const float c = b.scale * kLog2e;
  float dk[D], dv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
  for (int i = rd.i0; i < rd.i0 + rd.n; ++i)
    for (int q = 0; q < b.L; ++q) {
      const int64_t qrow = int64_t(i) * b.L + q;
      const float* qp = static_cast<const float*>(b.Q) + (qrow * nh + h) * D;
      const float* gp = static_cast<const float*>(b.dO) + (qrow * nh + h) * D;
      const int64_t sidx = (int64_t(i) * nh + h) * b.L + q;
      float sdot = 0.f, gdot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        sdot = fmaf(qp[e], kr[e], sdot);
        gdot = fmaf(gp[e], vr[e], gdot);
      }
      const float pv = __builtin_amdgcn_exp2f(fmaf(sdot, c, b.stats[2 * sidx]));
      const float ds = pv * (gdot - b.stats[2 * sidx + 1]);
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dv[e] = fmaf(pv, gp[e], dv[e]);
        dk[e] = fmaf(ds, qp[e], dk[e]);
      }
    }
  float* okp = static_cast<float*>(is_chunk ? b.dK : b.dKa) + (row * nh + h) * D;
  float* ovp = static_cast<float*>(is_chunk ? b.dV : b.dVa) + (row * nh + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    okp[e] = dk[e] * b.scale;
    ovp[e] = dv[e];
  }
}

template <int D>
void launch_backward(const BcLaunch& b, hipStream_t s, Profiler* prof) {
  const int64_t rows = int64_t(b.n_chunk) * b.L * b.nh;
  {
    Timed tm(prof, kBwdPre, s);
    if (b.dtype == FF_F32) {
      const int64_t threads = rows * (D / 4);
      hipLaunchKernelGGL((bc_prep_kernel<float, D>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, b);
    } else {
      const int64_t threads = rows * (D / 8);
      hipLaunchKernelGGL((bc_prep_kernel<__bf16, D>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, b);
    }
  }
  if (b.dtype == FF_F32) {
    {
      Timed tm(prof, kBwdDq, s);
      hipLaunchKernelGGL(bc_dq_f32_kernel<D>, dim3(unsigned((rows + 63) / 64)), dim3(64), 0, s, b);
    }
    {
      Timed tm(prof, kBwdDk, s);
      const int64_t keys = (int64_t(b.n_chunk) * b.L + int64_t(b.n_anchor) * b.T) * b.nh;
      hipLaunchKernelGGL(bc_dkv_f32_kernel<D>, dim3(unsigned((keys + 63) / 64)), dim3(64), 0, s, b);
    }
    return;
  }
  {
    Timed tm(prof, kBwdDq, s);
    const int items = b.n_chunk * b.nh * ((b.L + kBlockM - 1) / kBlockM);
    hipLaunchKernelGGL(bc_dq_kernel<D>, dim3(unsigned(items)), dim3(kDqWaves * 64), 0, s, b);
  }
  const int items = (b.n_chunk * ((b.L + kKeyBlock - 1) / kKeyBlock) +
                     b.n_anchor * ((b.T + kKeyBlock - 1) / kKeyBlock)) * b.nh;
  {
    Timed tm(prof, kBwdDk, s);
    hipLaunchKernelGGL((bc_dkv_kernel<D, true>), dim3(unsigned(items)), dim3(kKeyWaves * 64), 0, s, b);
  }
  {
    Timed tm(prof, kBwdDv, s);
    hipLaunchKernelGGL((bc_dkv_kernel<D, false>), dim3(unsigned(items)), dim3(kKeyWaves * 64), 0, s, b);
  }
}

}  // namespace

int dev_launch_bc_backward(const BcLaunch& b0, void* stream, Profiler* prof) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  BcLaunch b = b0;
  int n_cu = 0;
  if (dev_topology(&n_cu, &b.n_xcd) != 0) return FF_E_HIP;
  if (b.d == 64) launch_backward<64>(b, s, prof);
  else launch_backward<128>(b, s, prof);
  return launch_ok();
}

}  // namespace ff
