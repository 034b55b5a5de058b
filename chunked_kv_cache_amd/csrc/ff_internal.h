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
constexpr int kBlockM = 256;       // query rows per attention work item (8 waves x 32)
constexpr int kCUs = 256;          // MI355X compute units (one work item each)
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
// (head, 256-query tile); each item runs over all of the call's key tiles.
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
  int32_t n_wg;                    // persistent workgroups (one per CU)
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

// Device entry points.  Return 0 on success, FF_E_HIP on a launch error.
// `prof` (nullable) collects start/stop events when profiling is on.
struct Profiler;
int dev_launch_attention(const AttnLaunch& a, void* stream, Profiler* prof);
int dev_launch_publish(const CopyLaunch& c, void* stream, Profiler* prof, bool anchor);
int dev_launch_unpack(const CopyLaunch& c, void* stream);
Profiler* dev_profiler_create();
void dev_profiler_destroy(Profiler* p);
void dev_profiler_reset(Profiler* p);
int dev_profiler_read(Profiler* p, ff_kernel_times* out);

inline int64_t elem_size(int dtype) { return dtype == FF_F32 ? 4 : 2; }

}  // namespace ff
