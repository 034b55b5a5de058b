// Device building blocks shared by the gfx950 attention kernels: bf16 MFMA
// 32x32x16 operand layouts, global -> LDS tile copies through buffer
// resources, swizzled LDS tiles and their per-lane offsets.
//
// MFMA 32x32x16 operand layout: lane l holds A[l%32][8*(l/32)..+7] and
// B[8*(l/32)..+7][l%32]; D[i][l%32] for i = 8*(r/4) + 4*(l/32) + r%4, r < 16.
// A "rows" tile holds 64 rows of D values ([row][d], 16-byte chunks XOR
// swizzled per row); a "transposed" tile holds D rows of 64 values ([d][row]).
// The rows of a rows tile are fed to the first MFMA permuted (bits 2 and 3 of
// the row index swapped), so that accumulator registers 8*j..8*j+7 of lane l
// are rows 16*j + 8*(l/32) + 0..7 of the 32-row half: the result, rounded to
// bf16, is already in B-operand order for a second MFMA whose A operand is a
// transposed tile read as one contiguous 16-byte run per lane.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../ff_internal.h"

namespace ff {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

template <int D, int NW>
struct TileCfg {
  static constexpr int kKBytes = kBlockN * D * 2;     // K tile [64][D]
  static constexpr int kVBytes = D * kBlockN * 2;     // V^T tile [D][64]
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kKBlocks = kKBytes / 1024 / NW;   // 1 KB DMA blocks per wave
  static constexpr int kVBlocks = kVBytes / 1024 / NW;
  static constexpr int kDmaPerTile = kKBlocks + kVBlocks;
  static constexpr int kRowsPerKBlock = 1024 / (2 * D);
  static constexpr int kChunksPerRow = D / 8;
};

// XOR swizzles of the 16-byte chunks of an LDS row.  The lanes of one
// ds_read_b128 are served 16 at a time from a 256-byte window (8 at a time
// from 128 bytes on narrower LDS); with these swizzles the rows read together
// land on distinct 16-byte bank groups in both cases.
//   K tile row r (D = 128: 256-byte rows; D = 64: 128-byte rows)
//   V^T tile row dd (128-byte rows)
template <int D>
__device__ __forceinline__ int krow_swz(int r) {
  if (D == 128) return (r & 3) | ((r >> 1) & 4) | ((r << 1) & 8);
  return ((r & 3) | ((r >> 1) & 4)) ^ ((r >> 2) & 1);
}
__device__ __forceinline__ int vrow_swz(int dd) { return (dd & 7) ^ ((dd >> 3) & 1); }

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return zeros.  Word 3 selects the 32-bit data format that untyped gfx9
// buffer loads need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// 16 bytes per lane from buffer offset voff into LDS: a wave writes 1 KB,
// lane i to bytes 16i..16i+15 of dst.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}

// Wait until this wave's outstanding global->LDS copies have landed
// (vmcnt(0)), or all but the newest N (vmcnt(N); the field's low 4 bits sit
// in bits 3:0 of the immediate and its high 2 bits in bits 15:14).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }
template <int N>
__device__ __forceinline__ void wait_dma_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ int xcd_remap(int b, int nb, int nx) {
  // Blocks are dealt to the nx XCDs round-robin; give each XCD a contiguous
  // range of work items so that query tiles sharing a head's K/V share an L2.
  // XCD x receives the blocks b = x (mod nx): per or per + 1 of them, mapped
  // to one run of consecutive items (a bijection on [0, nb)).
  const int x = b % nx, idx = b / nx;
  const int per = nb / nx, rem = nb % nx;
  return x * per + (x < rem ? x : rem) + idx;
}

// The V^T buffers sit past the 64 KB reach of a DS instruction's immediate
// offset.  Their lane offsets carry a +64 KB bias that the optimiser cannot
// see through, so that (buffer base - 64 KB + row block) folds into the
// immediate and a V^T operand read costs no address arithmetic.  The address
// is correct wherever the buffers land; only the folding depends on it.
constexpr uint32_t kLdsBias = 65536;
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Per-lane constants of the tile copies and operand reads (set once).
template <int D, int NW>
struct LaneConst {
  uint32_t kdma[TileCfg<D, NW>::kKBlocks];   // K copy j: byte offset from the tile's first key row
  uint32_t kread[D / 16];                    // K operand of k-step ks, half 0: LDS byte offset
  uint32_t vread[2][2];                      // V^T operand (half, j), rows 0..31: LDS byte offset + kLdsBias
};

template <int D, int NW>
__device__ __forceinline__ void lane_const(LaneConst<D, NW>& lc, int w, int lane) {
  using Cfg = TileCfg<D, NW>;
  constexpr int CPR = Cfg::kChunksPerRow;
#pragma unroll
  for (int j = 0; j < Cfg::kKBlocks; ++j) {
    const int r = (w * Cfg::kKBlocks + j) * Cfg::kRowsPerKBlock + lane / CPR;
    lc.kdma[j] = uint32_t(r * D * 2 + (((lane % CPR) ^ krow_swz<D>(r)) << 4));
  }
  const int l32 = lane & 31, hl = lane >> 5;
  // Row of the K tile this lane feeds as A operand (bits 2 and 3 swapped).
  const int prow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    lc.kread[ks] = uint32_t(prow * D * 2 + (((2 * ks + hl) ^ krow_swz<D>(prow)) << 4));
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      lc.vread[half][j] = opaque(uint32_t(l32 * kBlockN * 2 + (((4 * half + 2 * j + hl) ^ vrow_swz(l32)) << 4)) +
                                 kLdsBias);
}

// Max / sum over the two 32-lane halves (lanes l and l^32 hold the same query).
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// S^T for one 32-key half (keys 32*half .. +31 of the K tile kbuf), for the
// wave's R blocks of 32 queries: each K operand read feeds R MFMAs.
template <int D, int NW, int R>
__device__ __forceinline__ void qk_half(const uint8_t* kbuf, int half, const LaneConst<D, NW>& lc,
                                        const bf16x8 (&qreg)[R][D / 16], f32x16 (&s)[R]) {
  const f32x16 zero = {};
#pragma unroll
  for (int b = 0; b < R; ++b) s[b] = zero;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, ld16(kbuf + lc.kread[ks] + half * 32 * D * 2));
#pragma unroll
    for (int b = 0; b < R; ++b) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[b][ks], s[b], 0, 0, 0);
  }
}

// Register r of this lane holds key 16*(r/8) + 8*hl + r%8 of the half; keys
// at or past `limit` are masked (the per-register offsets are constants, so
// only the lane's threshold lives in a register).
__device__ __forceinline__ void mask_half(f32x16& s, int limit, int hl) {
  const int lim = limit - 8 * hl;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (16 * (r >> 3) + (r & 7) >= lim) s[r] = -INFINITY;
}

}  // namespace
}  // namespace ff
