// Internal interface between the host bookkeeping (plain C++17) and the device
// launchers (HIP).  Only plain pointers and integers cross it, so the host
// side also builds with g++ against a recording stub for CPU-only tests.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/ff.h"

namespace ff {

constexpr int kMaxSeg = 24;        // renderer: <= 3 anchors + 8 history chunks + own chunk;
                                   // planner: one per anchor latent (<= W_ctx)
constexpr int kMaxPairs = 8;       // renderer calls fused into one launch
constexpr int kMaxHistory = 8;
constexpr int kBlockM = 256;       // query rows per work item: attention at head_dim 64 (8 waves x 32)
                                   // and the block-causal backward kernels
constexpr int kBlockMW = 512;      // query rows per attention work item at head_dim 128 (8 waves x 64)
// Query rows per work item of the bf16 attention kernel.
constexpr int attn_block_m(int head_dim) { return head_dim == 128 ? kBlockMW : kBlockM; }
constexpr int kMaxWg = 256;        // persistent attention workgroups at most (one per CU; the
                                   // device's CU count is queried at context creation)
constexpr int kBlockN = 64;        // keys per LDS tile

// One key source as the attention kernel sees it.  `base` points at the
// source's block in the workspace: K head-major [nh][n][d] followed directly by
// V transposed [nh][d][n] (both in the context dtype).
// Every source covers ceil(n/64) whole 64-key tiles of the call's tile index
// space, so no tile straddles two sources; the last tile of a source is
// masked past n.
struct SegTable {
  const void* base[kMaxSeg];
  int32_t n[kMaxSeg];              // tokens of the source (multiple of 8)
  int32_t tile_start[kMaxSeg + 1]; // prefix sums of ceil(n/64); [nseg] = tiles
  int32_t nseg;
};

// Attention work of one call ("pair" = chunk i at stage k).  Work item =
// (head, query tile of attn_block_m(d) rows); each item runs over all of the
// call's key tiles.
// The (item x key tile) units of a call are split evenly and contiguously
// over the persistent workgroups (stream-K); an item cut between workgroups
// leaves partial results in `part` that the merge kernel combines.
struct PairLaunch {
  const void* q;                   // [Lq][nh][d] token-major
  void* o;                         // [Lq][nh][d] token-major
  float* lse;                      // [nh][Lq] or null
  float* part;                     // partial slots of this call: n_wg x 2
  SegTable seg;
  int32_t lk;                      // key tokens
  int32_t ntiles;                  // 64-key tiles (sources padded to whole tiles)
  int32_t n_items;                 // nh x n_qtiles
};

struct AttnLaunch {
  PairLaunch pair[kMaxPairs];
  int32_t n_pairs;
  int32_t nh, d, lq;
  int32_t n_qtiles;
  int32_t n_wg;                    // persistent workgroups: one per CU, <= kMaxWg (set by the launcher)
  int32_t n_xcd;                   // XCDs the workgroups are dealt to round-robin (set by the launcher)
  int32_t dtype;                   // ff_dtype
  float scale;                     // 1/sqrt(d)
  int64_t slot_floats;             // floats per partial slot: O [BM][d], m [BM], l [BM]
};
// Passed by value as the kernel argument block, which is limited to 4 KB.
static_assert(sizeof(AttnLaunch) <= 4096, "attention launch arguments exceed the kernel argument limit");

// Layout copies between token-major rows and bank blocks.  A job moves `nseg`
// consecutive sources of L tokens each: token-major rows [nseg*L][nh][d] on
// one side, bank blocks block + g*block_stride (K [nh][L][d] then V^T
// [nh][d][L]) on the other.  Publish goes rows -> blocks, unpack the reverse.
struct CopyJob {
  const void* rows_k;              // publish: source rows
  const void* rows_v;
  void* out_k;                     // unpack: destination rows
  void* out_v;
  void* block;                     // first bank block of the job
  int32_t nseg;
};

struct CopyLaunch {
  CopyJob job[kMaxPairs];
  int32_t n_jobs;
  int32_t max_nseg;
  int32_t L, nh, d, dtype;
  int64_t block_stride;            // bytes between consecutive bank blocks
};

// Block-causal attention over a clip (training form).  Every source of the
// clip has a fixed place in the workspace, so a chunk's key set is two index
// ranges and the kernels need no per-chunk pointer table.
constexpr int kBcMaxChunks = 96;
constexpr int kBcMaxAnchors = 32;

struct BcChunk {
  int32_t a0, na;                  // anchors a0 .. a0+na-1 (Gamma(i), ascending)
  int32_t j0, nj;                  // chunks j0 .. j0+nj-1; the last one is the chunk itself
};

struct BcReaders {
  int32_t i0, n;                   // query chunks i0 .. i0+n-1 read this source
};

// Arguments of the backward kernels (by value, within the 4 KB limit).
// Workspace blocks have the bank layout: part 0 = rows [nh][n][d], part 1 =
// transposed [nh][d][n] of the pair named (kv = K rows + V^T, vk = V rows +
// K^T, qq = Q rows + Q^T, gg = dO rows + dO^T).
struct BcLaunch {
  int32_t nh, d, T, L;             // heads, head dim, tokens per anchor / per chunk
  int32_t n_anchor, n_chunk, dtype;
  int32_t n_xcd;                   // XCDs the workgroups are dealt to (set by the launcher)
  float scale;
  int64_t blk_anchor, blk_chunk;   // bytes per anchor / chunk block
  const uint8_t* kv_anchor;
  const uint8_t* vk_anchor;
  const uint8_t* kv_chunk;
  const uint8_t* vk_chunk;
  const uint8_t* qq_chunk;
  const uint8_t* gg_chunk;
  const void* Ka;                  // token-major inputs
  const void* Va;
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;                // [N_c][nh][L], natural log
  float* stats;                    // [N_c][nh][L][2]: -lse * log2(e), rowsum(dO * O)
  void* dQ;                        // token-major outputs
  void* dK;
  void* dV;
  void* dKa;
  void* dVa;
  BcChunk chunk[kBcMaxChunks];
  BcReaders readers[kBcMaxAnchors + kBcMaxChunks];   // anchor a at [a], chunk j at [kBcMaxAnchors + j]
};
static_assert(sizeof(BcLaunch) <= 4096, "backward launch arguments exceed the kernel argument limit");

// Fixed device scratch of ff_render_attend_static_scratch: the partial slots
// of one call (two per persistent workgroup, each kBlockMW rows of head_dim
// (<= 128) fp32 values plus the row max and sum), 130 MiB.
constexpr size_t kStaticScratchBytes = size_t(kMaxWg) * 2 * size_t(kBlockMW) * (128 + 2) * 4;
// Device address and size of that scratch on the current device; the
// address is taken once per device.  Returns 0, or FF_E_HIP.
int dev_static_scratch(void** ptr, size_t* bytes);

// Compute units and XCDs of the current device (hipDeviceAttribute*).
// Returns 0, or FF_E_HIP when the device cannot be queried.
int dev_topology(int* n_cu, int* n_xcd);

// Device entry points.  Return 0 on success, FF_E_HIP on a launch error.
// `prof` (nullable) collects start/stop events when profiling is on.
struct Profiler;
int dev_launch_attention(const AttnLaunch& a, void* stream, Profiler* prof);
int dev_launch_publish(const CopyLaunch& c, void* stream, Profiler* prof, bool anchor);
int dev_launch_unpack(const CopyLaunch& c, void* stream);
int dev_launch_layout(const CopyLaunch& c, void* stream, Profiler* prof);    // block-causal operand copies
int dev_launch_bc_backward(const BcLaunch& b, void* stream, Profiler* prof);
Profiler* dev_profiler_create();
void dev_profiler_destroy(Profiler* p);
void dev_profiler_reset(Profiler* p);
void dev_profiler_families(Profiler* p, unsigned families);   // bit f = kernel family f of ff_kernel_times
int dev_profiler_read(Profiler* p, ff_kernel_times* out);

inline int64_t elem_size(int dtype) { return dtype == FF_F32 ? 4 : 2; }

}  // namespace ff
