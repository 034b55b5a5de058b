// Recording stand-in for the device launchers, linked only into the host-check
// library (libff_hostcheck.so) that CPU tests load to exercise the C ABI's
// bookkeeping without a GPU.  Nothing is launched: each call records what it
// would have launched, and the tests read the record back.
#include <cstring>

#include "../ff_internal.h"
#include "../ff_schedule.h"

namespace ff {

struct Profiler {};

namespace {
AttnLaunch g_last_attn;
CopyLaunch g_last_copy;
BcLaunch g_last_bc;
int g_n_attn = 0, g_n_publish = 0, g_n_anchor = 0, g_n_unpack = 0, g_n_layout = 0, g_n_bc = 0;
}  // namespace

int dev_launch_attention(const AttnLaunch& a, void*, Profiler*) {
  g_last_attn = a;
  ++g_n_attn;
  return 0;
}

int dev_launch_publish(const CopyLaunch& c, void*, Profiler*, bool anchor) {
  g_last_copy = c;
  ++(anchor ? g_n_anchor : g_n_publish);
  return 0;
}

int dev_launch_unpack(const CopyLaunch& c, void*) {
  g_last_copy = c;
  ++g_n_unpack;
  return 0;
}

int dev_launch_layout(const CopyLaunch& c, void*, Profiler*) {
  g_last_copy = c;
  ++g_n_layout;
  return 0;
}

int dev_launch_bc_backward(const BcLaunch& b, void*, Profiler*) {
  g_last_bc = b;
  ++g_n_bc;
  return 0;
}

// Host stand-in for the fixed device scratch (never dereferenced by the stub).
int dev_static_scratch(void** ptr, size_t* bytes) {
  alignas(256) static uint8_t stand_in[256];
  *ptr = stand_in;
  *bytes = kStaticScratchBytes;
  return 0;
}

Profiler* dev_profiler_create() { return new Profiler(); }
void dev_profiler_destroy(Profiler* p) { delete p; }
void dev_profiler_reset(Profiler*) {}
void dev_profiler_families(Profiler*, unsigned) {}
int dev_profiler_read(Profiler*, ff_kernel_times* out) {
  std::memset(out, 0, sizeof(*out));
  return 0;
}

}  // namespace ff

// Inspection hooks of the host-check build (not part of ff.h).
extern "C" {
void ffstub_counts(int* attn, int* publish, int* anchor, int* unpack) {
  *attn = ff::g_n_attn;
  *publish = ff::g_n_publish;
  *anchor = ff::g_n_anchor;
  *unpack = ff::g_n_unpack;
}
// Key-source table of pair p of the last attention launch, as byte offsets
// from `ws` and token counts; returns the number of sources.
int ffstub_last_segments(int p, const void* ws, long long* offsets, int* n_tokens, int* lk, int* ntiles) {
  const ff::PairLaunch& P = ff::g_last_attn.pair[p];
  for (int s = 0; s < P.seg.nseg; ++s) {
    offsets[s] = static_cast<const char*>(P.seg.base[s]) - static_cast<const char*>(ws);
    n_tokens[s] = P.seg.n[s];
  }
  *lk = P.lk;
  *ntiles = P.ntiles;
  return P.seg.nseg;
}
// Partial-slot region of pair p of the last attention launch, as a byte
// offset from ws.
long long ffstub_last_part(int p, const void* ws) {
  return reinterpret_cast<const char*>(ff::g_last_attn.pair[p].part) - static_cast<const char*>(ws);
}
int ffstub_last_attn_pairs(int* n_wg) {
  *n_wg = ff::g_last_attn.n_wg;
  return ff::g_last_attn.n_pairs;
}
void ffstub_bc_counts(int* layout, int* backward) {
  *layout = ff::g_n_layout;
  *backward = ff::g_n_bc;
}
// Key ranges of chunk i and reader runs of source s (anchor a = s, chunk j =
// s - n_anchor) of the last backward launch.
void ffstub_last_bc_chunk(int i, int* a0, int* na, int* j0, int* nj) {
  const ff::BcChunk& c = ff::g_last_bc.chunk[i];
  *a0 = c.a0; *na = c.na; *j0 = c.j0; *nj = c.nj;
}
void ffstub_last_bc_readers(int s, int* i0, int* n) {
  const int slot = s < ff::g_last_bc.n_anchor ? s : ff::kBcMaxAnchors + (s - ff::g_last_bc.n_anchor);
  *i0 = ff::g_last_bc.readers[slot].i0;
  *n = ff::g_last_bc.readers[slot].n;
}
// Number of jobs of the last copy launch and job j's source rows / block.
int ffstub_last_copy_job(int j, const void** rows_k, const void** rows_v, int* nseg, int* L) {
  *rows_k = ff::g_last_copy.job[j].rows_k;
  *rows_v = ff::g_last_copy.job[j].rows_v;
  *nseg = ff::g_last_copy.job[j].nseg;
  *L = ff::g_last_copy.L;
  return ff::g_last_copy.n_jobs;
}
// Destination block of job j of the last copy launch, as a byte offset from ws.
long long ffstub_last_copy_block(int j, const void* ws) {
  return static_cast<const char*>(ff::g_last_copy.job[j].block) - static_cast<const char*>(ws);
}
// Attention schedule of one call (the kernel's own enumeration): the pieces
// of every workgroup as (g, item, t_begin, t_end, slot) rows; returns the
// row count, or -1 past cap rows.
int ffstub_schedule_pieces(int n_items, int ntiles, int n_wg, int* out, int cap) {
  const ff::LastRound lr = ff::last_round(n_items, ntiles, n_wg);
  int n = 0;
  for (int g = 0; g < n_wg; ++g) {
    ff::PieceIter it(lr, g);
    int item, tb, te, slot;
    while (it.next(lr, item, tb, te, slot)) {
      if (n >= cap) return -1;
      int* r = out + 5 * n++;
      r[0] = g; r[1] = item; r[2] = tb; r[3] = te; r[4] = slot;
    }
  }
  return n;
}
// The merge kernel's slot list of last-round item x (-1 for an empty
// candidate); returns the candidate count, or -1 past cap.
int ffstub_merge_slots(int n_items, int ntiles, int n_wg, int x, int* out, int cap) {
  const ff::LastRound lr = ff::last_round(n_items, ntiles, n_wg);
  const ff::MergeList ml(lr, x);
  const int n = ml.count(lr);
  if (n > cap) return -1;
  for (int i = 0; i < n; ++i) out[i] = ml.slot(lr, i);
  return n;
}
}
