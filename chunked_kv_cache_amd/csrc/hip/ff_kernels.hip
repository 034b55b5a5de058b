// gfx950 kernels of the renderer hot path.
//
//  attn_bf16<D>   segmented flash attention: bf16 MFMA 32x32x16 for S^T = K Q^T
//                 and O^T = V^T P^T, fp32 online softmax in base 2, K/V tiles
//                 gathered from the anchor bank and the stage ring through the
//                 call's key-source table into LDS (no concatenation copy);
//                 64 query rows per wave at head dim 128, 32 at head dim 64.
//  attn_f32<D>    plain fp32 path (one lane per query row and head).
//  merge_pieces   LSE merge of the items cut in the last scheduling round.
//  publish        token-major K/V -> bank block (K head-major, V transposed).
//  unpack         bank block -> token-major K/V (read-out of B_k).
//
// Pages cited: [S] "In-Flight KV Cache with Clean Anchors for Faster
// Autoregressive Video Diffusion", Korean summary page, section "how it
// works", Eq. (2): the renderer attends its chunk over A_Gamma(i) and B_k^(i)
// and its own K/V, then B_k^(i+1) = Tail_H(B_k^(i) U (i, K, V)).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <vector>

#include "../ff_internal.h"
#include "../ff_schedule.h"
#include "ff_prof.h"
#include "ff_tile.h"

namespace ff {
namespace {

// Overflow guard of the softmax weights.  The reference max m is the exact
// row max of a piece's first 32 keys; later halves use it as long as the
// weights p = 2^(s*c - m) stay small.  A lane's sum of its 16 weights of a
// half bounds each of them: while every sum is <= 2^12 no weight exceeds 2^12
// (ample range for fp32 and bf16); when one is larger (or infinite), that
// half takes the rare exact path -- its row max, a rescale of O and l, and
// the weights again.  The result is exact either way after the division by l.
constexpr float kSumGuard = 4096.0f;


// --------------------------------------------------------------------------
// Segmented attention, bf16 in, fp32 accumulate.
//
// Work item = (pair, head, 256-query tile), possibly cut into two key ranges
// in the last round; one persistent workgroup per CU.  Per 64-key tile:
//   S^T[key][q] = sum_d K[key][d] Q[q][d]     (A = K rows from LDS, B = Q regs)
//   p = 2^(s*scale*log2e - m)                 (per query = per lane column)
//   O^T[d][q] += sum_key V^T[d][key] P^T[key][q]  (A = V^T from LDS, B = P regs)
// MFMA 32x32x16 operand layout: lane l holds A[l%32][8*(l/32)..+7] and
// B[8*(l/32)..+7][l%32]; D[i][l%32] for i = 8*(r/4) + 4*(l/32) + r%4, r < 16.
// The K rows fed to S^T are permuted (bits 2 and 3 of the row swapped) so
// that accumulator registers 8*j..8*j+7 of lane l are keys 16*j + 8*(l/32) +
// 0..7: P leaves the first MFMA already in B-operand order for the second,
// and V^T rows are read as one contiguous 16-byte run per lane.
//
// K/V tiles go global -> LDS directly (buffer_load_dwordx4 ... lds, 1 KB per
// wave instruction, lane i -> LDS bytes 16i..16i+15) into four K and four V^T
// buffers, two tiles ahead of the math.  The LDS layouts are XOR-swizzled for
// conflict-free 16-byte reads; the swizzle is applied by choosing which
// global chunk each lane fetches.
// --------------------------------------------------------------------------
// Waves per work item: eight, two per SIMD.  Head dim 128 runs the 64-row
// form (run_item_r64: wave w owns rows 64w..64w+63 of a 512-row item and
// walks both 32-key halves of every tile, each K or V^T operand read feeds
// two MFMAs); head dim 64 runs the 32-row form (run_item: wave w owns rows
// 32w..32w+31 of a 256-row item, one MFMA per operand read, the S^T of the
// next half beside the softmax of this one).
constexpr int kAttnWaves = 8;







// Key-source cursor of one wave (pointers and counts wave-uniform).
template <int D, int NW>
struct SrcCursor {
  const __bf16* k;      // K rows of this head, key 0 of the source
  const __bf16* v;      // V^T of this head, [D][n]
  int n, t0, t1, s;
  uint32_t vdma[TileCfg<D, NW>::kVBlocks];   // V^T copy j: lane byte offset from the tile's first key
};

template <int D, int NW>
__device__ __forceinline__ void cursor_set(SrcCursor<D, NW>& c, const SegTable& t, int s, int h, int nh, int w,
                                           int lane) {
  using Cfg = TileCfg<D, NW>;
  c.s = s;
  c.n = t.n[s];
  c.t0 = t.tile_start[s];
  c.t1 = t.tile_start[s + 1];
  const __bf16* base = static_cast<const __bf16*>(t.base[s]);
  c.k = base + int64_t(h) * c.n * D;
  c.v = base + int64_t(nh) * c.n * D + int64_t(h) * D * c.n;
#pragma unroll
  for (int j = 0; j < Cfg::kVBlocks; ++j) {
    const int dd = (w * Cfg::kVBlocks + j) * 8 + lane / 8;
    c.vdma[j] = uint32_t(dd * c.n * 2 + (((lane & 7) ^ vrow_swz(dd)) << 4));
  }
}

// Issue the copies of tile t (inside the cursor's source) into kbuf / vbuf.
// Each copy reads through a buffer resource that ends with the head's data:
// K rows past the source's last key read as zeros, and V^T chunks past it
// read the next row's first keys (or zeros after the last row); those keys
// are masked, so their p is exactly 0.  Returns the tile's valid key count.
template <int D, int NW>
__device__ __forceinline__ int issue_tile(const SrcCursor<D, NW>& c, const LaneConst<D, NW>& lc, int t,
                                          uint8_t* kbuf, uint8_t* vbuf, int w) {
  using Cfg = TileCfg<D, NW>;
  const int o = (t - c.t0) * kBlockN;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(c.k + int64_t(o) * D, uint32_t(c.n - o) * D * 2);
#pragma unroll
  for (int j = 0; j < Cfg::kKBlocks; ++j) dma16(rk, lc.kdma[j], kbuf + (w * Cfg::kKBlocks + j) * 1024);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(c.v + o, uint32_t(D * c.n - o) * 2);
#pragma unroll
  for (int j = 0; j < Cfg::kVBlocks; ++j) dma16(rv, c.vdma[j], vbuf + (w * Cfg::kVBlocks + j) * 1024);
  return min(kBlockN, c.n - o);
}

// --------------------------------------------------------------------------
// Per-wave software pipeline over the two 32-key halves of each 64-key tile.
// While the matrix pipe runs the S^T MFMAs of the next half, the VALU does the
// softmax of the current half (the two are independent), then the PV MFMAs of
// the current half follow.  Two score buffers alternate roles across the
// unrolled halves, so nothing is copied.
// --------------------------------------------------------------------------

template <int D>
struct WaveState {
  f32x16 o[D / 32];          // O^T accumulators, one per 32-row block of d
  float m, l;                // reference max (base 2) and per-lane partial sum
};



// Two interleaved chains of 3-input maxima (8 VALU ops for 16 values).
__device__ __forceinline__ float rowmax_half(const f32x16& s) {
  float a = fmaxf(s[0], fmaxf(s[1], s[2]));
  float b = fmaxf(s[3], fmaxf(s[4], s[5]));
  a = fmaxf(a, fmaxf(s[6], s[7]));
  b = fmaxf(b, fmaxf(s[8], s[9]));
  a = fmaxf(a, fmaxf(s[10], s[11]));
  b = fmaxf(b, fmaxf(s[12], s[13]));
  a = fmaxf(a, fmaxf(s[14], s[15]));
  return half_swap_max(fmaxf(a, b));
}

// P = 2^(s*c - m) as bf16 B operands; returns this lane's sum of the 16
// weights (two chains of 8, each starting from its first term).
__device__ __forceinline__ float exp_half(const f32x16& s, float c, float m, bf16x8 (&pb)[2]) {
  const float nm = -m;
  float lsum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(s[8 * j + e], c, nm));
      lsum[j] = e ? lsum[j] + pv : pv;
      pb[j][e] = (__bf16)pv;
    }
  return lsum[0] + lsum[1];
}

// The weights of a half in place: the bf16 pair of registers 8j+2e, 8j+2e+1
// goes to register 8j+e (e < 4), so registers 8j..8j+3 end as the B operand
// of the PV MFMA for keys 16j..16j+15.  Returns this lane's sum of the 16
// weights (fp32, before rounding).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float exp_inplace(f32x16& s, float c, float m) {
  const float nm = -m;
  float lsum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * j + 2 * e], c, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * j + 2 * e + 1], c, nm));
      lsum[j] = (e ? lsum[j] + p0 : p0) + p1;
      const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
      s[8 * j + e] = __builtin_bit_cast(float, pk);
    }
  return lsum[0] + lsum[1];
}
__device__ __forceinline__ bf16x8 p_operand(const f32x16& s, int j) {
  const f32x16 t = s;
  return j ? __builtin_bit_cast(bf16x8, __builtin_shufflevector(t, t, 8, 9, 10, 11))
           : __builtin_bit_cast(bf16x8, __builtin_shufflevector(t, t, 0, 1, 2, 3));
}

// Softmax weights of one half against the reference max, with the overflow
// guard: when some lane's sum exceeds kSumGuard (the branch is wave-uniform),
// raise m to the half's exact row max, rescale O and l, and redo the weights.
template <int D>
__device__ __forceinline__ void softmax_p(const f32x16& s, float c, WaveState<D>& st, bf16x8 (&pb)[2]) {
  float lsum = exp_half(s, c, st.m, pb);
  if (__builtin_expect(__ballot(lsum > kSumGuard) != 0, 0)) {
    const float m_new = fmaxf(st.m, rowmax_half(s) * c);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    st.m = m_new;
    lsum = exp_half(s, c, st.m, pb);
  }
  st.l += lsum;
}

// O^T += V^T P^T for one 32-key half of the V^T tile vbuf; each operand read
// feeds R MFMAs.
template <int D, int NW, int R>
__device__ __forceinline__ void pv_half(const uint8_t* vbuf, int half, const LaneConst<D, NW>& lc,
                                        const bf16x8 (&pb)[R][2], WaveState<D> (&st)[R]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 av = __builtin_bit_cast(
          bf16x8, ld16(vbuf + (int32_t(lc.vread[half][j]) - int32_t(kLdsBias)) + db * 32 * kBlockN * 2));
#pragma unroll
      for (int b = 0; b < R; ++b)
        st[b].o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[b][j], st[b].o[db], 0, 0, 0);
    }
}

// The four K and V^T tile buffers of a workgroup.
struct LdsBufs {
  uint8_t* k[4];
  uint8_t* v[4];
};

// One piece of work: item (head h, query tile qt) over key tiles [t_begin,
// t_end).  A whole item writes O and LSE; a piece writes its unnormalised O,
// running max and sum to `slot` for the merge kernel.  Wave w owns query rows
// 32*R*w .. 32*R*w + 32*R - 1 of the tile, as R blocks of 32.
template <int D, int NW>
__device__ __forceinline__ void run_item(const AttnLaunch& a, const PairLaunch& P, int item, int t_begin, int t_end,
                                         float* slot, const LdsBufs& lb) {
  constexpr int KS = D / 16;       // MFMA k-steps over head_dim
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int R = kBlockM / NW / 32;
  constexpr int kDma = TileCfg<D, NW>::kDmaPerTile;   // per wave
  const int nh = a.nh, lq = a.lq;
  const int qt = item % a.n_qtiles;
  const int h = item / a.n_qtiles;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int row0 = w * 32 * R + l32;             // query row of block 0 within the tile

  // Q^T as the B operand: lane holds Q[q][16*ks + 8*hl .. +7] of its R rows.
  bf16x8 qreg[R][KS];
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const int q = qt * kBlockM + row0 + 32 * b;
    const bool ok = q < lq;
    const __bf16* qp = static_cast<const __bf16*>(P.q) + (int64_t(ok ? q : 0) * nh + h) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = ld16(qp + 16 * ks);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      qreg[b][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const float c = a.scale * kLog2e;
  LaneConst<D, NW> lc;
  lane_const<D, NW>(lc, w, lane);

  WaveState<D> st[R];
#pragma unroll
  for (int b = 0; b < R; ++b) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[b].o[db][r] = 0.f;
    st[b].m = -INFINITY;
    st[b].l = 0.f;
  }

  SrcCursor<D, NW> cur;
  {
    int s = 0;
    while (s + 1 < P.seg.nseg && t_begin >= P.seg.tile_start[s + 1]) ++s;
    cursor_set<D, NW>(cur, P.seg, s, h, nh, w, lane);
  }
  auto issue = [&](int t, int i) -> int {
    if (t >= cur.t1) cursor_set<D, NW>(cur, P.seg, cur.s + 1, h, nh, w, lane);
    return issue_tile<D, NW>(cur, lc, t, lb.k[i], lb.v[i], w);
  };
  // Scores of a half: keys at or past `limit` masked (a rarely taken branch).
  auto mask_scores = [&](f32x16 (&s)[R], int limit) {
    if (limit < 32) {
#pragma unroll
      for (int b = 0; b < R; ++b) mask_half(s[b], limit, hl);
    }
  };
  auto softmax = [&](const f32x16 (&s)[R], bf16x8 (&pb)[R][2]) {
#pragma unroll
    for (int b = 0; b < R; ++b) softmax_p<D>(s[b], c, st[b], pb[b]);
  };

  f32x16 sa[R], sb[R];   // scores of the half awaiting softmax / being computed
  bf16x8 pb[R][2];
  int valid[4];
  __syncthreads();       // the previous piece's reads of the buffers are done
  valid[0] = issue(t_begin, 0);
  if (t_begin + 1 < t_end) valid[1] = issue(t_begin + 1, 1);
  if (t_begin + 2 < t_end) valid[2] = issue(t_begin + 2, 2);
  if (t_begin + 2 < t_end) wait_dma_but<2 * kDma>();
  else if (t_begin + 1 < t_end) wait_dma_but<kDma>();
  else wait_dma();
  __syncthreads();
  qk_half<D, NW, R>(lb.k[0], 0, lc, qreg, sa);
  mask_scores(sa, valid[0]);
  // The reference max: the exact row max of the piece's first half (it holds
  // at least one unmasked key, so m is finite from here on).
#pragma unroll
  for (int b = 0; b < R; ++b) st[b].m = rowmax_half(sa[b]) * c;

  // Tile t is in buffer i (landed); buffer i+1 holds tile t+1 and i+2 tile
  // t+2 (both may still be landing); buffer i+3 is free for tile t+3 (indices
  // mod 4).  Copies run two tiles ahead.
  // Invariant at entry: sa = masked scores of half 0 of tile t.
  auto tile = [&](int t, int i) {
    const int i1 = (i + 1) & 3, i3 = (i + 3) & 3;
    // half 0: S^T(half 1) and softmax(half 0) interleave; then PV(half 0)
    qk_half<D, NW, R>(lb.k[i], 1, lc, qreg, sb);
    softmax(sa, pb);
    pv_half<D, NW, R>(lb.v[i], 0, lc, pb, st);
    mask_scores(sb, valid[i] - 32);
    // half 1: S^T(tile t+1, half 0) and softmax(half 1); then PV(half 1).
    // On the last tile the S^T of buffer i+1 is computed on stale data and dropped.
    const bool more = t + 1 < t_end;
    if (more) {
      if (t + 2 < t_end) wait_dma_but<kDma>();   // tile t+1 landed, t+2 may fly
      else wait_dma();
      __syncthreads();
      if (t + 3 < t_end) valid[i3] = issue(t + 3, i3);
    }
    qk_half<D, NW, R>(lb.k[i1], 0, lc, qreg, sa);
    softmax(sb, pb);
    pv_half<D, NW, R>(lb.v[i], 1, lc, pb, st);
    if (more) mask_scores(sa, valid[i1]);
  };

  for (int t = t_begin; t < t_end; t += 4) {
    tile(t, 0);
    if (t + 1 >= t_end) break;
    tile(t + 1, 1);
    if (t + 2 >= t_end) break;
    tile(t + 2, 2);
    if (t + 3 >= t_end) break;
    tile(t + 3, 3);
  }

  // ---- epilogue
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const float l_tot = half_swap_sum(st[b].l);
    const int row = row0 + 32 * b;
    const int q = qt * kBlockM + row;
    if (q >= lq) continue;
    if (!slot) {
      const float inv = 1.0f / l_tot;
      __bf16* op = static_cast<__bf16*>(P.o) + (int64_t(q) * nh + h) * D + 4 * hl;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(st[b].o[db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g) = ov;
        }
      if (P.lse && hl == 0) P.lse[int64_t(h) * lq + q] = (st[b].m + log2f(l_tot)) * kLn2;
    } else {
      float* op = slot + row * D + 4 * hl;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& o = st[b].o[db];
          *reinterpret_cast<float4*>(op + 32 * db + 8 * g) =
              make_float4(o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]);
        }
      if (hl == 0) {
        slot[kBlockM * D + row] = st[b].m;
        slot[kBlockM * D + kBlockM + row] = l_tot;
      }
    }
  }
}

// --------------------------------------------------------------------------
// 64 query rows per wave (head_dim 128): helpers.
//
// Every K or V^T operand read from LDS feeds two MFMAs (two blocks of 32
// query rows): half the LDS read instructions and bytes per MFMA of the
// 32-row form.  The registers of 64 rows (O^T 128, Q 64, scores 32) leave no
// room for a second score buffer, so the weights are packed in place over the
// scores of one 32-key half, a wave runs S^T, softmax and PV of a half in
// sequence, and the two waves of each SIMD interleave instead (one in its
// softmax while the other runs MFMAs).
// --------------------------------------------------------------------------

// S^T of one key half for the wave's two row blocks.  kread is the lane's
// offset for k-step 0 of that half; with the D = 128 swizzle, k-step ks sits
// at kread ^ (ks << 5) (the swizzle XORs the chunk index, and ks occupies its
// bits 1..3).
__device__ __forceinline__ void qk_w64(const uint8_t* kbuf, uint32_t kread, const bf16x8 (&qreg)[2][8],
                                       f32x16 (&s)[2]) {
  const f32x16 zero = {};
  s[0] = zero;
  s[1] = zero;
  // Each operand read is issued one k-step ahead of its two MFMAs; the
  // scheduling barriers keep that order (left alone, the scheduler waits on
  // every read before its MFMAs).
  bf16x8 cur = __builtin_bit_cast(bf16x8, ld16(kbuf + kread));
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 nxt = cur;
    if (ks < 7) nxt = __builtin_bit_cast(bf16x8, ld16(kbuf + (kread ^ uint32_t((ks + 1) << 5))));
    __builtin_amdgcn_sched_barrier(0);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qreg[0][ks], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qreg[1][ks], s[1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
}

// mask_half on both blocks with per-register bit masks instead of compares
// (no condition registers held across the sixteen selects).
__device__ __forceinline__ void mask_pair(f32x16& a, f32x16& b, int limit, int hl) {
  const int lim = limit - 8 * hl;
  const uint32_t ninf = 0xff800000u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t keep = uint32_t(int32_t(16 * (r >> 3) + (r & 7) - lim) >> 31);
    a[r] = __uint_as_float((__float_as_uint(a[r]) & keep) | (ninf & ~keep));
    b[r] = __uint_as_float((__float_as_uint(b[r]) & keep) | (ninf & ~keep));
  }
}

// The MFMA phase of one tile: PV of this tile (eight V^T operands of vbuf)
// then S^T of the next (eight K operands of kbuf) as one operand stream, each
// read one step ahead of its two MFMAs, so the first K read overlaps the last
// PV MFMAs.  `first` is V^T operand 0, read by the caller beforehand.  The
// scores s hold the weights (packed in place) on entry and the next tile's
// scores on return.
__device__ __forceinline__ void mfma_phase(const uint8_t* vbuf, const uint32_t (&vread)[2], const uint8_t* kbuf,
                                           uint32_t kread, const bf16x8 (&qreg)[2][8], f32x16 (&s)[2],
                                           WaveState<128> (&st)[2], bf16x8 first) {
  auto rd = [&](int k) {
    if (k < 8) {
      const int j = k >> 2, db = k & 3;
      return __builtin_bit_cast(bf16x8,
                                ld16(vbuf + (int32_t(vread[j]) - int32_t(kLdsBias)) + db * 32 * kBlockN * 2));
    }
    return __builtin_bit_cast(bf16x8, ld16(kbuf + (kread ^ uint32_t((k - 8) << 5))));
  };
  const f32x16 zero = {};
  bf16x8 cur = first;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    bf16x8 nxt = cur;
    if (k < 15) nxt = rd(k + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (k < 8) {
      const int j = k >> 2, db = k & 3;
      st[0].o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, j ? p_operand(s[0], 1) : p_operand(s[0], 0),
                                                            st[0].o[db], 0, 0, 0);
      st[1].o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, j ? p_operand(s[1], 1) : p_operand(s[1], 0),
                                                            st[1].o[db], 0, 0, 0);
    } else {
      const int ks = k - 8;
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qreg[0][ks], ks ? s[0] : zero, 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qreg[1][ks], ks ? s[1] : zero, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    cur = nxt;
  }
}

__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The lane's index, read afresh (volatile, so never merged with an earlier
// read): lane-derived offsets are recomputed where they are needed instead of
// holding registers across the key loop.
__device__ __forceinline__ int lane_now() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return int(l);
}

// Operand offsets of key half 0 of a tile for lane `lane`: K operand of
// k-step 0 (k-step ks at ^ (ks << 5)), V^T operands j = 0, 1 (+ kLdsBias).
struct HalfOffsets {
  uint32_t k, v0, v1;
};
__device__ __forceinline__ HalfOffsets half_offsets(int lane) {
  const int l32 = lane & 31, hl = lane >> 5;
  const int prow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
  HalfOffsets o;
  o.k = uint32_t(prow * 128 * 2 + ((hl ^ krow_swz<128>(prow)) << 4));
  const uint32_t v = uint32_t(l32 * kBlockN * 2 + ((hl ^ vrow_swz(l32)) << 4)) + kLdsBias;
  o.v0 = opaque(v);
  o.v1 = opaque(v ^ 32u);
  return o;
}

// --------------------------------------------------------------------------
// 512 query rows per workgroup (head_dim 128): every wave owns 64 rows of its
// own and walks both 32-key halves of each 64-key tile, so one K/V tile in
// LDS serves twice the query rows of the form above and the global -> LDS
// copies per FLOP are halved.  The registers per wave are those of the form
// above (one half's scores at a time, weights packed in place).  A wave runs,
// per tile t: softmax of half 0 (V0), PV of half 0 + S^T of half 1 (M0),
// softmax of half 1 (V1), PV of half 1 + S^T of half 0 of tile t+1 (M1).
// The barrier of a tile that orders the copies (tile t+1 landed, tile t-1's
// buffer free) comes before M1: waves 0..3 reach it after V1 and waves 4..7
// before V1; a second one before M0 (after V0, resp. before it) keeps the
// pairing.  So one wave of each SIMD is in a VALU phase while the other runs
// MFMAs.
// Each wave finishes its own rows: no merge between waves.
// --------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void run_item_r64(const AttnLaunch& a, const PairLaunch& P, int item, int t_begin,
                                             int t_end, float* slot, const LdsBufs& lb) {
  static_assert(D == 128, "the 512-row form is laid out for head_dim 128");
  constexpr int NW = 8;
  constexpr int KS = D / 16;
  constexpr int BM = kBlockMW;
  constexpr int kDma = TileCfg<D, NW>::kDmaPerTile;   // per wave
  static_assert(TileCfg<D, NW>::kKBlocks == 2 && TileCfg<D, NW>::kVBlocks == 2, "two copies of each per wave");
  constexpr uint32_t kHalfK = 32 * D * 2;    // K rows of key half 1: byte offset in a K tile
  constexpr uint32_t kHalfV = 4u << 4;       // V^T chunk of key half 1: XOR on the operand offset
  const int nh = a.nh, lq = a.lq;
  const int qt = item % a.n_qtiles;
  const int h = item / a.n_qtiles;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w >> 2;                    // barrier group

  // Register block b holds rows 64 * w + 32 * b + lane % 32.
  bf16x8 qreg[2][KS];
  {
    const int lane = lane_now();
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int q = qt * BM + w * 64 + 32 * b + (lane & 31);
      const bool ok = q < lq;
      const __bf16* qp = static_cast<const __bf16*>(P.q) + (int64_t(ok ? q : 0) * nh + h) * D + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = ld16(qp + 16 * ks);
        if (!ok) v = u32x4{0u, 0u, 0u, 0u};
        qreg[b][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  const float c = a.scale * kLog2e;
  WaveState<D> st[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[b].o[db][r] = 0.f;
    st[b].l = 0.f;
  }

  // The lane offsets of the tile copies wait in LDS (each lane reads back
  // only what it wrote), not in registers.
  __shared__ u32x2 kdo[NW * 64], vdo[NW * 64];
  {
    const int lane = lane_now();
    LaneConst<D, NW> lc;
    lane_const<D, NW>(lc, w, lane);
    kdo[w * 64 + lane] = u32x2{lc.kdma[0], lc.kdma[1]};
  }
  SrcCursor<D, NW> cur;
  auto set_cursor = [&](int s) {
    const int lane = lane_now();
    cursor_set<D, NW>(cur, P.seg, s, h, nh, w, lane);
    vdo[w * 64 + lane] = u32x2{cur.vdma[0], cur.vdma[1]};
  };
  {
    int s = 0;
    while (s + 1 < P.seg.nseg && t_begin >= P.seg.tile_start[s + 1]) ++s;
    set_cursor(s);
  }
  auto issue = [&](int t, int i) -> int {
    if (t >= cur.t1) set_cursor(cur.s + 1);
    const int lane = lane_now();
    const int o = (t - cur.t0) * kBlockN;
    const u32x2 ko = kdo[w * 64 + lane], vo = vdo[w * 64 + lane];
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(cur.k + int64_t(o) * D, uint32_t(cur.n - o) * D * 2);
    dma16(rk, ko[0], lb.k[i] + (w * 2) * 1024);
    dma16(rk, ko[1], lb.k[i] + (w * 2 + 1) * 1024);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(cur.v + o, uint32_t(D * cur.n - o) * 2);
    dma16(rv, vo[0], lb.v[i] + (w * 2) * 1024);
    dma16(rv, vo[1], lb.v[i] + (w * 2 + 1) * 1024);
    return min(kBlockN, cur.n - o);
  };
  // Operand offsets of key half 0 (half 1: K at + kHalfK, V^T at ^ kHalfV).
  const HalfOffsets ho = half_offsets(lane_now());
  // S^T of key half `hf` of the tile in kbuf, keys at or past `valid` masked
  // (a rarely taken branch).
  auto scores = [&](const uint8_t* kbuf, int valid, int hf, f32x16 (&s)[2]) {
    qk_w64(kbuf + (hf ? kHalfK : 0u), ho.k, qreg, s);
    const int limit = valid - 32 * hf;
    if (limit < 32) mask_pair(s[0], s[1], limit, lane_now() >> 5);
  };
  // Softmax of one half in place over its scores (sa), the lane sums added to
  // l.  Rare exact path: the weights overwrote the scores, so recompute them
  // (the tile is still in buffer i), raise each block's m to the exact row
  // max, rescale O and l, and redo the weights.
  f32x16 sa[2];
  int valid[4];
  auto softmax = [&](int i, int hf) {
    float ls0 = exp_inplace(sa[0], c, st[0].m), ls1 = exp_inplace(sa[1], c, st[1].m);
    if (__builtin_expect(__ballot(ls0 > kSumGuard || ls1 > kSumGuard) != 0, 0)) {
      scores(lb.k[i], valid[i], hf, sa);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float m_new = fmaxf(st[b].m, rowmax_half(sa[b]) * c);
        const float alpha = __builtin_amdgcn_exp2f(st[b].m - m_new);
        st[b].l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[b].o[db][r] *= alpha;
        st[b].m = m_new;
      }
      ls0 = exp_inplace(sa[0], c, st[0].m);
      ls1 = exp_inplace(sa[1], c, st[1].m);
    }
    st[0].l += ls0;
    st[1].l += ls1;
  };

  __syncthreads();       // the previous piece's reads of the buffers are done
  valid[0] = issue(t_begin, 0);
  if (t_begin + 1 < t_end) valid[1] = issue(t_begin + 1, 1);
  if (t_begin + 2 < t_end) valid[2] = issue(t_begin + 2, 2);
  if (t_begin + 2 < t_end) wait_dma_but<2 * kDma>();
  else if (t_begin + 1 < t_end) wait_dma_but<kDma>();
  else wait_dma();
  wg_barrier();
  if (qt * BM + w * 64 >= lq) {
    // No row of this wave exists (the last query tile of a head): it only
    // keeps its part of the copies and the two barriers of every tile, and
    // leaves its SIMD to the partner wave.
    auto idle_tile = [&](int t, int i) {
      wg_barrier();
      if (t + 2 < t_end) wait_dma_but<kDma>();
      else wait_dma();
      wg_barrier();
      if (t + 3 < t_end) issue(t + 3, (i + 3) & 3);
    };
    for (int t = t_begin; t < t_end; t += 4) {   // buffer indices known at compile time
      idle_tile(t, 0);
      if (t + 1 >= t_end) break;
      idle_tile(t + 1, 1);
      if (t + 2 >= t_end) break;
      idle_tile(t + 2, 2);
      if (t + 3 >= t_end) break;
      idle_tile(t + 3, 3);
    }
    return;
  }
  scores(lb.k[0], valid[0], 0, sa);
  // The first half of a piece holds at least one valid key, so m is finite.
#pragma unroll
  for (int b = 0; b < 2; ++b) st[b].m = rowmax_half(sa[b]) * c;

  // Tile t is in buffer i (landed); i+1 holds tile t+1 and i+2 tile t+2 (both
  // may still be landing); i+3 is free for tile t+3 once every wave is past
  // this tile's barrier (indices mod 4).  Invariant at entry: sa = masked
  // scores of half 0 of tile t.
  const uint32_t vr0[2] = {ho.v0, ho.v1};
  const uint32_t vr1[2] = {ho.v0 ^ kHalfV, ho.v1 ^ kHalfV};
  auto tile = [&](int t, int i) {
    const int i1 = (i + 1) & 3, i3 = (i + 3) & 3;
    const bool more = t + 1 < t_end;
    // V0, then M0: PV of half 0, S^T of half 1 (tile t landed before the
    // previous barrier).  A second barrier per tile paces the two groups
    // (waves 0..3 reach it after V0, waves 4..7 before it): with one barrier
    // per tile their phases drift into each other.
    {
      if (grp) wg_barrier();
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, ld16(lb.v[i] + (int32_t(ho.v0) - int32_t(kLdsBias))));
      softmax(i, 0);
      if (!grp) wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_phase(lb.v[i], vr0, lb.k[i] + kHalfK, ho.k, qreg, sa, st, v0);
      const int limit = valid[i] - 32;
      if (limit < 32) mask_pair(sa[0], sa[1], limit, lane_now() >> 5);
    }
    auto sync = [&] {
      if (more && t + 2 < t_end) wait_dma_but<kDma>();   // tile t+1 landed, t+2 may fly
      else wait_dma();
      wg_barrier();
    };
    if (grp) sync();
    // V1, then M1: PV of half 1, S^T of half 0 of tile t+1 (on the last tile
    // computed on stale data and dropped).
    const bf16x8 v0 = __builtin_bit_cast(bf16x8, ld16(lb.v[i] + (int32_t(ho.v0 ^ kHalfV) - int32_t(kLdsBias))));
    softmax(i, 1);
    if (!grp) sync();
    // Both groups are past this tile's barrier here, and both issue the copies
    // of tile t+3 at the start of M1.
    if (t + 3 < t_end) valid[i3] = issue(t + 3, i3);
    __builtin_amdgcn_sched_barrier(0);
    mfma_phase(lb.v[i], vr1, lb.k[i1], ho.k, qreg, sa, st, v0);
    if (more) {
      const int limit = valid[i1];
      if (limit < 32) mask_pair(sa[0], sa[1], limit, lane_now() >> 5);
    }
  };

  for (int t = t_begin; t < t_end; t += 4) {
    tile(t, 0);
    if (t + 1 >= t_end) break;
    tile(t + 1, 1);
    if (t + 2 >= t_end) break;
    tile(t + 2, 2);
    if (t + 3 >= t_end) break;
    tile(t + 3, 3);
  }

  const int lane = lane_now();
  const int hl = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const WaveState<D>& me = st[b];
    const float l_tot = half_swap_sum(me.l);
    const int row = w * 64 + 32 * b + (lane & 31);
    const int q = qt * BM + row;
    if (q < lq) {
      if (!slot) {
        const float inv = 1.0f / l_tot;
        __bf16* op = static_cast<__bf16*>(P.o) + (int64_t(q) * nh + h) * D + 4 * hl;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(me.o[db][4 * g + e] * inv);
            *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * g) = ov;
          }
        if (P.lse && hl == 0) P.lse[int64_t(h) * lq + q] = (me.m + log2f(l_tot)) * kLn2;
      } else {
        float* op = slot + row * D + 4 * hl;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& o = me.o[db];
            *reinterpret_cast<float4*>(op + 32 * db + 8 * g) =
                make_float4(o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]);
          }
        if (hl == 0) {
          slot[BM * D + row] = me.m;
          slot[BM * D + BM + row] = l_tot;
        }
      }
    }
  }
}

template <int D, int NW, bool W64>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(const AttnLaunch a) {
  // One array per tile buffer, so that the compiler sees the copies into one
  // buffer and the operand reads of another as disjoint.
  using Cfg = TileCfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t k0[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k1[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k2[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k3[Cfg::kKBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[Cfg::kVBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v1[Cfg::kVBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v2[Cfg::kVBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v3[Cfg::kVBytes];
  const LdsBufs lb = {{k0, k1, k2, k3}, {v0, v1, v2, v3}};
  // Consecutive workgroup ids sit on one XCD (shared L2).
  const int g = xcd_remap(blockIdx.x, gridDim.x, a.n_xcd);
  for (int p = 0; p < a.n_pairs; ++p) {
    const PairLaunch& P = a.pair[p];
    const LastRound lr = last_round(P.n_items, P.ntiles, a.n_wg);
    // Pieces of this workgroup (one call site, so the item body is inlined
    // once).
    PieceIter it(lr, g);
    int item, t_begin, t_end, si;
    while (it.next(lr, item, t_begin, t_end, si)) {
      float* slot = si < 0 ? nullptr : P.part + int64_t(si) * a.slot_floats;
      if constexpr (W64) run_item_r64<D>(a, P, item, t_begin, t_end, slot, lb);
      else run_item<D, NW>(a, P, item, t_begin, t_end, slot, lb);
    }
  }
}

// --------------------------------------------------------------------------
// Merge of the items of the last round: O = sum_j 2^(m_j - M) O_j /
// sum_j 2^(m_j - M) l_j over the item's pieces j, in workgroup order.  One
// block per 32 query rows of a last-round item and call; D/4 consecutive
// threads share a query row, each taking 4 head-dim values, so partial reads
// and O writes are coalesced.
// --------------------------------------------------------------------------
constexpr int kMergeRows = 32;   // query rows per merge block

template <int D>
__global__ __launch_bounds__(256) void merge_pieces_kernel(const AttnLaunch a) {
  constexpr int TPR = D / 4;                     // threads per row
  constexpr int RPP = 256 / TPR;                 // rows per pass
  constexpr int BM = attn_block_m(D);            // query rows of an item
  const PairLaunch& P = a.pair[blockIdx.y];
  const LastRound lr = last_round(P.n_items, P.ntiles, a.n_wg);
  const int x = blockIdx.x / (BM / kMergeRows);
  if (x >= lr.rem) return;
  const int item = lr.full * a.n_wg + x;
  const int qt = item % a.n_qtiles, h = item / a.n_qtiles;
  // The item's pieces in key order, listed once per block in LDS.
  constexpr int kMaxCand = 2 * kMaxWg;
  __shared__ int32_t cand[kMaxCand];
  const MergeList ml(lr, x);
  const int n_cand = ml.count(lr);             // <= n_wg + left < kMaxCand
  for (int n = threadIdx.x; n < n_cand; n += blockDim.x) cand[n] = ml.slot(lr, n);
  __syncthreads();
  const int c4 = threadIdx.x % TPR;
  const int r0 = (blockIdx.x % (BM / kMergeRows)) * kMergeRows + threadIdx.x / TPR;
  constexpr int NP = kMergeRows / RPP;           // rows per thread
  float M[NP], L[NP];
  float4 acc[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    M[j] = -INFINITY;
    L[j] = 0.f;
    acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Two sweeps over the pieces (the row max, then the weighted sums); the
  // rows past lq read the slots' unwritten rows and are not stored.
  for (int sweep = 0; sweep < 2; ++sweep) {
    for (int n = 0; n < n_cand; ++n) {
      const int32_t slot = cand[n];
      if (slot < 0) continue;
      const float* sp = P.part + int64_t(slot) * a.slot_floats;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int row = r0 + j * RPP;
        const float m = sp[BM * D + row];
        if (sweep == 0) {
          M[j] = fmaxf(M[j], m);
        } else {
          const float wj = __builtin_amdgcn_exp2f(m - M[j]);
          L[j] += wj * sp[BM * D + BM + row];
          const float4 v = reinterpret_cast<const float4*>(sp + row * D)[c4];
          acc[j].x += wj * v.x;
          acc[j].y += wj * v.y;
          acc[j].z += wj * v.z;
          acc[j].w += wj * v.w;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int row = r0 + j * RPP;
    const int q = qt * BM + row;
    if (q >= a.lq) break;
    const float inv = 1.0f / L[j];
    bf16x4 ov;
    ov[0] = (__bf16)(acc[j].x * inv);
    ov[1] = (__bf16)(acc[j].y * inv);
    ov[2] = (__bf16)(acc[j].z * inv);
    ov[3] = (__bf16)(acc[j].w * inv);
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.o) + (int64_t(q) * a.nh + h) * D + 4 * c4) = ov;
    if (P.lse && c4 == 0) P.lse[int64_t(h) * a.lq + q] = (M[j] + log2f(L[j])) * kLn2;
  }
}

// --------------------------------------------------------------------------
// fp32 path: one lane per (pair, query, head); keys streamed in order.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnLaunch a) {
  const int p = blockIdx.y;
  const PairLaunch& P = a.pair[p];
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= int64_t(a.lq) * a.nh) return;
  const int h = int(gid % a.nh), q = int(gid / a.nh);
  const int nh = a.nh;
  const float* qp = static_cast<const float*>(P.q) + gid * D;
  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) { qv[e] = qp[e]; acc[e] = 0.f; }
  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  for (int s = 0; s < P.seg.nseg; ++s) {
    const int n = P.seg.n[s];
    const float* kb = static_cast<const float*>(P.seg.base[s]) + int64_t(h) * n * D;
    const float* vb = static_cast<const float*>(P.seg.base[s]) + int64_t(nh) * n * D + int64_t(h) * D * n;
    for (int j = 0; j < n; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qv[e], kb[int64_t(j) * D + e], dot);
      const float sc = dot * c;
      if (sc > m) {
        const float alpha = __builtin_amdgcn_exp2f(m - sc);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= alpha;
        m = sc;
      }
      const float pv = __builtin_amdgcn_exp2f(sc - m);
      l += pv;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pv, vb[int64_t(e) * n + j], acc[e]);
    }
  }
  float* op = static_cast<float*>(P.o) + gid * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
  if (P.lse) P.lse[int64_t(h) * a.lq + q] = (m + log2f(l)) * kLn2;
}

// --------------------------------------------------------------------------
// Publish (rows -> bank block) and unpack (bank block -> rows).
// Block = 64 tokens x 1 head of one source.  K moves as 16-byte chunks; V goes
// through LDS for the [token][d] <-> [d][token] transpose.
// --------------------------------------------------------------------------
template <typename E, int D, bool kPublish>
__global__ __launch_bounds__(256) void layout_copy_kernel(const CopyLaunch cl) {
  constexpr int EPC = 16 / sizeof(E);             // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                    // chunks per token row
  constexpr int TB = 64;                          // tokens per block
  constexpr int PAD = 1;                          // row padding (elements)
  __shared__ E tile[TB][D + PAD];

  const int job = blockIdx.z, g = blockIdx.y;
  if (job >= cl.n_jobs) return;
  const CopyJob& J = cl.job[job];
  if (g >= J.nseg) return;
  const int nh = cl.nh, L = cl.L;
  const int h = blockIdx.x % nh;
  const int t0 = (blockIdx.x / nh) * TB;
  if (t0 >= L) return;
  const int nt = min(TB, L - t0);                 // multiple of EPC
  const int tid = threadIdx.x;

  uint8_t* blk = static_cast<uint8_t*>(J.block) + int64_t(g) * cl.block_stride;
  E* bk = reinterpret_cast<E*>(blk) + (int64_t(h) * L + t0) * D;               // K [h][t][d]
  E* bv = reinterpret_cast<E*>(blk) + int64_t(nh) * L * D + int64_t(h) * D * L + t0;  // V^T [h][d][t]
  const int64_t row0 = int64_t(g) * L + t0;      // first token row of this block

  if (kPublish) {
    const E* rk = static_cast<const E*>(J.rows_k);
    const E* rv = static_cast<const E*>(J.rows_v);
    for (int i = tid; i < nt * CPR; i += 256) {
      const int t = i / CPR, ch = i % CPR;
      const int64_t src = ((row0 + t) * nh + h) * D + ch * EPC;
      st16(bk + int64_t(t) * D + ch * EPC, ld16(rk + src));
      const u32x4 v = ld16(rv + src);
      const E* ve = reinterpret_cast<const E*>(&v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) tile[t][ch * EPC + e] = ve[e];
    }
    __syncthreads();
    const int tch = nt / EPC;                       // token chunks per d-row
    for (int i = tid; i < D * tch; i += 256) {
      const int dd = i / tch, tc = i % tch;
      u32x4 v;
      E* ve = reinterpret_cast<E*>(&v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) ve[e] = tile[tc * EPC + e][dd];
      st16(bv + int64_t(dd) * L + tc * EPC, v);
    }
  } else {
    E* ok = static_cast<E*>(J.out_k);
    E* ov = static_cast<E*>(J.out_v);
    const int tch = nt / EPC;
    if (ov) {
      for (int i = tid; i < D * tch; i += 256) {
        const int dd = i / tch, tc = i % tch;
        const u32x4 v = ld16(bv + int64_t(dd) * L + tc * EPC);
        const E* ve = reinterpret_cast<const E*>(&v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) tile[tc * EPC + e][dd] = ve[e];
      }
    }
    __syncthreads();
    for (int i = tid; i < nt * CPR; i += 256) {
      const int t = i / CPR, ch = i % CPR;
      const int64_t dst = ((int64_t(t0) + t) * nh + h) * D + ch * EPC;
      if (ok) st16(ok + dst, ld16(bk + int64_t(t) * D + ch * EPC));
      if (ov) {
        u32x4 v;
        E* ve = reinterpret_cast<E*>(&v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) ve[e] = tile[t][ch * EPC + e];
        st16(ov + dst, v);
      }
    }
  }
}

// --------------------------------------------------------------------------
// bf16 publish / unpack with the V transpose done in registers.
// Block = G x 128 tokens x 1 head: G groups of 128 tokens; in each group wave
// w covers tokens 64*(w/2) .. +63 and head-dim 64*(w%2) .. +63.  Lane = tg +
// 8*c: token group tg (8 tokens), 16-byte d-chunk c.  Each lane moves an 8 x 8
// bf16 block per group: 8 token rows of one d-chunk in, 8 d-rows of one token
// group out, transposed with byte permutes.  For a fixed register, the 64
// lanes touch 8 rows x 128 contiguous bytes on both sides.  K moves as plain
// 16-byte chunks (8 per lane and group).  The publish issues all groups'
// loads (G x 16 x 16 bytes per lane) before any store.  G = 2 when the copy
// would otherwise take about two rounds of blocks over the CUs (one 480p
// chunk: 444 blocks of 128 tokens -> 228 of 256), G = 1 for larger copies.
// --------------------------------------------------------------------------
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // in[j] = 8 bf16 of token j (d = 0..7); out[r] = 8 bf16 of d = r (tokens 0..7)
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = in[2 * w][r >> 1], y = in[2 * w + 1][r >> 1];
      out[r][w] = (r & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
    }
}

template <bool kPublish, int G>
__global__ __launch_bounds__(256) void layout_copy_bf16_kernel(const CopyLaunch cl) {
  constexpr int D = 128;
  const int job = blockIdx.z, g = blockIdx.y;
  if (job >= cl.n_jobs) return;
  const CopyJob& J = cl.job[job];
  if (g >= J.nseg) return;
  const int nh = cl.nh, L = cl.L;
  const int h = blockIdx.x % nh;
  const int t0 = (blockIdx.x / nh) * 128 * G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int tg = lane & 7, c = lane >> 3;
  const int d0 = 64 * (w & 1) + 8 * c;               // first d of this lane's chunk
  int tb[G];                                         // first token of this lane's group, per 128-token group
  bool ok[G];                                        // L is a multiple of 8
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    tb[gi] = t0 + 128 * gi + 64 * (w >> 1) + 8 * tg;
    ok[gi] = tb[gi] < L;
  }
  uint8_t* blk = static_cast<uint8_t*>(J.block) + int64_t(g) * cl.block_stride;
  __bf16* bk = reinterpret_cast<__bf16*>(blk) + int64_t(h) * L * D;                          // K [h][t][d]
  __bf16* bv = reinterpret_cast<__bf16*>(blk) + int64_t(nh) * L * D + int64_t(h) * D * L;   // V^T [h][d][t]
  const int64_t row0 = int64_t(g) * L;               // first token row of this source
  if (kPublish) {
    const __bf16* rk = static_cast<const __bf16*>(J.rows_k);
    const __bf16* rv = static_cast<const __bf16*>(J.rows_v);
    u32x4 kin[G][8], vin[G][8], vout[8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      if (!ok[gi]) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t src = ((row0 + tb[gi] + j) * nh + h) * D + d0;
        kin[gi][j] = ld16(rk + src);
        vin[gi][j] = ld16(rv + src);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      if (!ok[gi]) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) st16(bk + int64_t(tb[gi] + j) * D + d0, kin[gi][j]);
      transpose8x8(vin[gi], vout);
#pragma unroll
      for (int r = 0; r < 8; ++r) st16(bv + int64_t(d0 + r) * L + tb[gi], vout[r]);
    }
  } else {
    __bf16* ok_ = static_cast<__bf16*>(J.out_k);
    __bf16* ov_ = static_cast<__bf16*>(J.out_v);
    u32x4 kin[8], vin[8], vout[8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      if (!ok[gi]) continue;
      if (ok_) {
#pragma unroll
        for (int j = 0; j < 8; ++j) kin[j] = ld16(bk + int64_t(tb[gi] + j) * D + d0);
#pragma unroll
        for (int j = 0; j < 8; ++j) st16(ok_ + ((int64_t(tb[gi]) + j) * nh + h) * D + d0, kin[j]);
      }
      if (ov_) {
#pragma unroll
        for (int r = 0; r < 8; ++r) vin[r] = ld16(bv + int64_t(d0 + r) * L + tb[gi]);
        transpose8x8(vin, vout);       // the 8x8 transpose is its own inverse
#pragma unroll
        for (int j = 0; j < 8; ++j) st16(ov_ + ((int64_t(tb[gi]) + j) * nh + h) * D + d0, vout[j]);
      }
    }
  }
}

}  // namespace

// Compute units and XCDs of each device, queried once per device.
int dev_topology(int* n_cu, int* n_xcd) {
  static std::mutex mu;
  static int cu_of[64] = {}, xcd_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FF_E_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!cu_of[dev]) {
    int cu = 0, xcc = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
      return FF_E_HIP;
    if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcc < 1) xcc = 1;
    cu_of[dev] = cu;
    xcd_of[dev] = xcc;
  }
  *n_cu = cu_of[dev];
  *n_xcd = xcd_of[dev];
  return 0;
}

int dev_launch_attention(const AttnLaunch& a0, void* stream, Profiler* prof) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // One persistent workgroup per CU (at most kMaxWg, the partial slots the
  // workspace holds per call), dealt to the XCDs as the device reports them.
  AttnLaunch a = a0;
  int n_cu = 0;
  if (dev_topology(&n_cu, &a.n_xcd) != 0) return FF_E_HIP;
  a.n_wg = n_cu < kMaxWg ? n_cu : kMaxWg;
  if (a.dtype == FF_F32) {
    Timed tm(prof, kAttn, s);
    dim3 grid(unsigned((int64_t(a.lq) * a.nh + 63) / 64), unsigned(a.n_pairs));
    if (a.d == 64) hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, a);
    return launch_ok();
  }
  {
    Timed tm(prof, kAttn, s);
    const dim3 grid(a.n_wg), block(kAttnWaves * 64);
    if (a.d == 64) hipLaunchKernelGGL((attn_bf16_kernel<64, kAttnWaves, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, kAttnWaves, true>), grid, block, 0, s, a);
  }
  if (launch_ok()) return FF_E_HIP;
  {
    Timed tm(prof, kMerge, s);
    int max_rem = 0;
    for (int p = 0; p < a.n_pairs; ++p) {
      const LastRound lr = last_round(a.pair[p].n_items, a.pair[p].ntiles, a.n_wg);
      if (lr.rem > max_rem) max_rem = lr.rem;
    }
    if (max_rem == 0) return 0;
    dim3 grid(unsigned(max_rem * (attn_block_m(a.d) / kMergeRows)), unsigned(a.n_pairs));
    if (a.d == 64) hipLaunchKernelGGL(merge_pieces_kernel<64>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(merge_pieces_kernel<128>, grid, dim3(256), 0, s, a);
  }
  return launch_ok();
}

template <bool kPublish>
static void launch_copy(const CopyLaunch& c, hipStream_t s) {
  if (c.dtype == FF_BF16 && c.d == 128) {
    int n_cu = 0, n_xcd = 0;
    if (dev_topology(&n_cu, &n_xcd) != 0) n_cu = kMaxWg;
    const int64_t blocks128 = int64_t((c.L + 127) / 128) * c.nh * c.max_nseg * c.n_jobs;
    if (blocks128 <= 2 * int64_t(n_cu)) {
      dim3 grid(unsigned(((c.L + 255) / 256) * c.nh), unsigned(c.max_nseg), unsigned(c.n_jobs));
      hipLaunchKernelGGL((layout_copy_bf16_kernel<kPublish, 2>), grid, dim3(256), 0, s, c);
    } else {
      dim3 grid(unsigned(((c.L + 127) / 128) * c.nh), unsigned(c.max_nseg), unsigned(c.n_jobs));
      hipLaunchKernelGGL((layout_copy_bf16_kernel<kPublish, 1>), grid, dim3(256), 0, s, c);
    }
    return;
  }
  dim3 grid(unsigned(((c.L + 63) / 64) * c.nh), unsigned(c.max_nseg), unsigned(c.n_jobs));
  if (c.dtype == FF_F32) {
    if (c.d == 64) hipLaunchKernelGGL((layout_copy_kernel<float, 64, kPublish>), grid, dim3(256), 0, s, c);
    else hipLaunchKernelGGL((layout_copy_kernel<float, 128, kPublish>), grid, dim3(256), 0, s, c);
  } else {
    if (c.d == 64) hipLaunchKernelGGL((layout_copy_kernel<uint16_t, 64, kPublish>), grid, dim3(256), 0, s, c);
    else hipLaunchKernelGGL((layout_copy_kernel<uint16_t, 128, kPublish>), grid, dim3(256), 0, s, c);
  }
}

int dev_launch_publish(const CopyLaunch& c, void* stream, Profiler* prof, bool anchor) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    Timed tm(prof, anchor ? kAnchor : kPublish, s);
    launch_copy<true>(c, s);
  }
  return launch_ok();
}

int dev_launch_layout(const CopyLaunch& c, void* stream, Profiler* prof) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    Timed tm(prof, kLayout, s);
    launch_copy<true>(c, s);
  }
  return launch_ok();
}

int dev_launch_unpack(const CopyLaunch& c, void* stream) {
  launch_copy<false>(c, static_cast<hipStream_t>(stream));
  return launch_ok();
}

Profiler* dev_profiler_create() { return new Profiler(); }

void dev_profiler_destroy(Profiler* p) {
  if (!p) return;
  for (auto& r : p->pending) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
  for (auto e : p->pool) (void)hipEventDestroy(e);
  delete p;
}

void dev_profiler_reset(Profiler* p) {
  if (!p) return;
  for (auto& r : p->pending) {
    (void)hipEventSynchronize(r.b);
    p->pool.push_back(r.a);
    p->pool.push_back(r.b);
  }
  p->pending.clear();
  for (int k = 0; k < kKinds; ++k) { p->count[k] = 0; p->ms[k] = 0; }
}

int dev_profiler_read(Profiler* p, ff_kernel_times* out) {
  int rc = 0;
  for (auto& r : p->pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = FF_E_HIP;
    p->count[r.kind] += 1;
    p->ms[r.kind] += ms;
    p->pool.push_back(r.a);
    p->pool.push_back(r.b);
  }
  p->pending.clear();
  out->attn_launches = p->count[kAttn];     out->attn_ms = p->ms[kAttn];
  out->merge_launches = p->count[kMerge];   out->merge_ms = p->ms[kMerge];
  out->publish_launches = p->count[kPublish]; out->publish_ms = p->ms[kPublish];
  out->anchor_launches = p->count[kAnchor]; out->anchor_ms = p->ms[kAnchor];
  out->layout_launches = p->count[kLayout]; out->layout_ms = p->ms[kLayout];
  out->bwd_pre_launches = p->count[kBwdPre]; out->bwd_pre_ms = p->ms[kBwdPre];
  out->bwd_dq_launches = p->count[kBwdDq];  out->bwd_dq_ms = p->ms[kBwdDq];
  out->bwd_dk_launches = p->count[kBwdDk];  out->bwd_dk_ms = p->ms[kBwdDk];
  out->bwd_dv_launches = p->count[kBwdDv];  out->bwd_dv_ms = p->ms[kBwdDv];
  return rc;
}

}  // namespace ff
