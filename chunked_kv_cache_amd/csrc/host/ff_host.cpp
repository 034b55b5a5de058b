// Host side of the C ABI: shape checks, workspace layout, Gamma(i), the
// stage-bank ring metadata, the key plan of a call, and launch assembly.
// Plain C++17; all device work goes through the dev_* functions.
//
// Pages cited: [S] "In-Flight KV Cache with Clean Anchors for Faster
// Autoregressive Video Diffusion", Korean summary page ("how it works",
// Eq. (2); "how it differs"; "what it is").
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../ff_internal.h"

using namespace ff;

struct ff_ctx {
  ff_shape shape;
  int S = 0, H = 0;
  int n_anchor = 0, n_chunk = 0, n_block = 0;   // anchors, renderer chunks, planner blocks
  int64_t T = 0, Lq = 0;          // tokens per latent, tokens per chunk
  int64_t esz = 2;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  // workspace regions (byte offsets from ws)
  size_t anchor_off = 0, anchor_block = 0;   // anchor a: anchor_off + a*anchor_block
  size_t slot_off = 0, slot_block = 0;       // stage k, slot s: slot_off + (k*(H+1)+s)*slot_block
  size_t part_off = 0, part_slot_bytes = 0;  // stream-K partial slots
  // metadata
  std::vector<uint8_t> anchor_present;
  std::vector<int> next;                     // next chunk per stage
  std::vector<uint8_t> can_rewind;
  Profiler* prof = nullptr;
  bool profiling = false;
  unsigned prof_families = FF_PROF_ALL;
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool shape_ok(const ff_shape* s, int S, int H) {
  if (!s) return false;
  if (s->n_heads < 1 || s->n_heads > 1024) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->tokens_per_latent < 8 || s->tokens_per_latent % 8 || s->tokens_per_latent > (1 << 20)) return false;
  if (s->chunk_latents < 1 || s->anchor_stride < 1) return false;
  // At most 3 anchors per chunk under either rule needs B_R <= Delta.
  if (s->chunk_latents > s->anchor_stride) return false;
  if (s->n_latents < s->chunk_latents || s->n_latents % s->chunk_latents) return false;
  if (s->w_ctx < 1) return false;
  if (s->dtype != FF_BF16 && s->dtype != FF_F32) return false;
  if (s->gamma_rule != FF_GAMMA_BRACKET && s->gamma_rule != FF_GAMMA_CENTER_LR) return false;
  if (S < 1 || S > 64 || H < 1 || H > kMaxHistory) return false;
  if (s->planner_latents < 1 || s->planner_history < 0 || s->planner_history > 1024) return false;
  // A planner call reads one source per anchor latent, at most W_ctx of them
  // (and never more than its window holds).
  const int64_t plan_src = std::min<int64_t>(int64_t(s->planner_history) * s->planner_latents + s->planner_latents,
                                             std::max<int64_t>(s->w_ctx, s->planner_latents));
  if (plan_src > kMaxSeg) return false;
  // query rows per call times heads must index in 32 bits
  const int64_t lq = int64_t(std::max(s->chunk_latents, s->planner_latents)) * s->tokens_per_latent;
  if (lq * s->n_heads * s->head_dim > (int64_t(1) << 31) - 1) return false;
  return true;
}

// Partial slots of one call: two per persistent workgroup.
size_t part_region_bytes(size_t part_slot) { return size_t(kMaxWg) * 2 * part_slot; }

struct Layout {
  size_t anchor_off, anchor_block, slot_off, slot_block, part_off, part_slot, total;
  int n_anchor, n_chunk;
};

Layout layout_of(const ff_shape* s, int S, int H) {
  Layout L{};
  const size_t esz = s->dtype == FF_F32 ? 4 : 2;
  const size_t T = size_t(s->tokens_per_latent), nh = size_t(s->n_heads), d = size_t(s->head_dim);
  const size_t lq = T * size_t(s->chunk_latents);
  L.n_anchor = (s->n_latents + s->anchor_stride - 1) / s->anchor_stride;
  L.n_chunk = s->n_latents / s->chunk_latents;
  L.anchor_block = align_up(2 * nh * T * d * esz);
  L.slot_block = align_up(2 * nh * lq * d * esz);
  L.anchor_off = 0;
  L.slot_off = L.anchor_off + size_t(L.n_anchor) * L.anchor_block;
  // Split-item partial slots (bf16 path): 2 per workgroup, in one region per
  // stage and one for planner calls, so that calls of different stages (or a
  // planner call) may run concurrently on different streams.
  L.part_slot = s->dtype == FF_BF16 ? align_up(size_t(attn_block_m(d)) * (d + 2) * 4) : 0;
  L.part_off = L.slot_off + size_t(S) * size_t(H + 1) * L.slot_block;
  L.total = L.part_off + size_t(S + 1) * part_region_bytes(L.part_slot);
  return L;
}

// Gamma(i): reading of [S] "how it differs" / "how it is used" (see ff.h).
// The anchors come out ascending and consecutive under both rules.
int gamma_ids(const ff_shape& s, int n_anchor, int i, int* ids) {
  const int D = s.anchor_stride, B = s.chunk_latents;
  const int p0 = B * i, p1 = B * i + B - 1;
  int n = 0;
  if (s.gamma_rule == FF_GAMMA_BRACKET) {
    const int lo = (p0 / D) * D, hi = ((p1 + D - 1) / D) * D;
    for (int a = lo / D; a <= hi / D && a < n_anchor; ++a) ids[n++] = a;
  } else {
    const int left = (p0 + B / 2) / D;
    for (int a = left; a <= left + 1 && a < n_anchor; ++a) ids[n++] = a;
  }
  return n;
}
int gamma_of(const ff_ctx* c, int i, int* ids) { return gamma_ids(c->shape, c->n_anchor, i, ids); }

// First history chunk of renderer chunk i when its bank holds chunks
// [next - min(next, H), next): oldest dropped while the key latents exceed
// W_ctx (reading of [S] "how it differs": W_ctx = 21).
int history_first(const ff_shape& s, int H, int n_gamma, int i, int next) {
  int h_first = next - std::min(next, H);
  while (h_first < i && n_gamma + s.chunk_latents * (i - h_first + 1) > s.w_ctx) ++h_first;
  return h_first;
}

// Key sources: n_gamma anchors, history chunks [h_first, i), then chunk i.
void fill_render_plan(const int* ids, int na, int h_first, int i, int64_t T, int64_t Lq, int B,
                      ff_key_sources* p) {
  std::memset(p, 0, sizeof(*p));
  int n = 0;
  for (int j = 0; j < na; ++j) {
    p->kind[n] = FF_SRC_ANCHOR; p->id[n] = ids[j]; p->n_tokens[n] = int32_t(T); ++n;
  }
  for (int ch = h_first; ch < i; ++ch) {
    p->kind[n] = FF_SRC_HISTORY; p->id[n] = ch; p->n_tokens[n] = int32_t(Lq); ++n;
  }
  p->kind[n] = FF_SRC_OWN; p->id[n] = i; p->n_tokens[n] = int32_t(Lq); ++n;
  p->n_sources = n;
  p->key_latents = na + B * (i - h_first + 1);
  int64_t tot = 0;
  for (int j = 0; j < n; ++j) tot += p->n_tokens[j];
  p->key_tokens = int32_t(tot);
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool lse_ok(const float* p) { return !p || (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

uint8_t* anchor_ptr(const ff_ctx* c, int a) { return c->ws + c->anchor_off + size_t(a) * c->anchor_block; }

// Anchors of planner block b: [b*B_P, b*B_P + n).
int block_anchors(const ff_ctx* c, int b, int* first) {
  const int bp = c->shape.planner_latents;
  *first = b * bp;
  return std::min(bp, c->n_anchor - b * bp);
}

uint8_t* slot_ptr(const ff_ctx* c, int stage, int chunk) {
  const int s = chunk % (c->H + 1);
  return c->ws + c->slot_off + (size_t(stage) * size_t(c->H + 1) + size_t(s)) * c->slot_block;
}

// Order contract of one call against the current state (no side effects).
ff_status check_call(const ff_ctx* c, int i, int k) {
  if (k < 0 || k >= c->S || i < 0 || i >= c->n_chunk) return FF_E_RANGE;
  if (c->next[k] != i) return FF_E_ORDER;
  if (k > 0 && c->next[k - 1] <= i) return FF_E_ORDER;
  int ids[8];
  const int n = gamma_of(c, i, ids);
  for (int j = 0; j < n; ++j)
    if (!c->anchor_present[ids[j]]) return FF_E_ANCHOR_MISSING;
  return FF_OK;
}

// Order contract of planner block b (no side effects): every earlier block
// published, the block itself not.
ff_status check_plan(const ff_ctx* c, int b) {
  if (b < 0 || b >= c->n_block) return FF_E_RANGE;
  int first = 0;
  const int n = block_anchors(c, b, &first);
  for (int a = 0; a < first; ++a)
    if (!c->anchor_present[a]) return FF_E_ORDER;
  for (int a = first; a < first + n; ++a)
    if (c->anchor_present[a]) return FF_E_ANCHOR_EXISTS;
  return FF_OK;
}

// Key sources of planner block b: the anchors of the previous min(b, H_P)
// blocks (oldest first, oldest blocks dropped while over W_ctx), then one
// FF_SRC_OWN entry per anchor of the block.
void plan_planner(const ff_ctx* c, int b, ff_key_sources* p) {
  std::memset(p, 0, sizeof(*p));
  const int bp = c->shape.planner_latents;
  int first = 0;
  const int n_own = block_anchors(c, b, &first);
  int h_first = std::max(0, b - c->shape.planner_history);
  while (h_first < b && bp * (b - h_first) + n_own > c->shape.w_ctx) ++h_first;
  int n = 0;
  for (int a = h_first * bp; a < b * bp; ++a) {
    p->kind[n] = FF_SRC_ANCHOR; p->id[n] = a; p->n_tokens[n] = int32_t(c->T); ++n;
  }
  for (int a = first; a < first + n_own; ++a) {
    p->kind[n] = FF_SRC_OWN; p->id[n] = a; p->n_tokens[n] = int32_t(c->T); ++n;
  }
  p->n_sources = n;
  p->key_latents = n;
  p->key_tokens = int32_t(int64_t(n) * c->T);
}

// Key sources of (i, k): Gamma(i) anchors ascending, then B_k^(i) oldest
// first, then the chunk itself; oldest history dropped while over W_ctx.
void plan_of(const ff_ctx* c, int i, int k, ff_key_sources* p) {
  int ids[8];
  const int na = gamma_of(c, i, ids);
  const int h_first = history_first(c->shape, c->H, na, i, c->next[k]);   // B_k^(i) = [h_first, i)
  fill_render_plan(ids, na, h_first, i, c->T, c->Lq, c->shape.chunk_latents, p);
}

// Device addresses of a call's sources.  k < 0 marks a planner call, whose
// own latents are staged in their anchor-bank entries.
void seg_table_of(const ff_ctx* c, int k, const ff_key_sources& p, SegTable* t) {
  std::memset(t, 0, sizeof(*t));
  int32_t tiles = 0;
  for (int j = 0; j < p.n_sources; ++j) {
    const bool in_anchor_bank = p.kind[j] == FF_SRC_ANCHOR || (k < 0 && p.kind[j] == FF_SRC_OWN);
    const uint8_t* base = in_anchor_bank ? anchor_ptr(c, p.id[j]) : slot_ptr(c, k, p.id[j]);
    t->base[j] = base;
    t->n[j] = p.n_tokens[j];
    t->tile_start[j] = tiles;
    tiles += (p.n_tokens[j] + kBlockN - 1) / kBlockN;
  }
  t->tile_start[p.n_sources] = tiles;
  t->nseg = p.n_sources;
}

// Work decomposition: items = heads x 256-query tiles; the (item x key tile)
// units of each call are spread evenly over one persistent workgroup per CU.
// The partition of a call depends only on that call, so it gives the same bits
// alone or inside a grouped launch.
void fill_attention(const ff_ctx* c, int n_pairs, const int* ks, const ff_key_sources* plans, int64_t lq,
                    const void* const* Q, void* const* O, float* const* lse, AttnLaunch* a) {
  std::memset(a, 0, sizeof(*a));
  a->n_pairs = n_pairs;
  a->nh = c->shape.n_heads;
  a->d = c->shape.head_dim;
  a->lq = int32_t(lq);
  a->n_qtiles = int32_t((lq + attn_block_m(a->d) - 1) / attn_block_m(a->d));
  a->dtype = c->shape.dtype;
  a->scale = float(1.0 / std::sqrt(double(c->shape.head_dim)));
  a->slot_floats = int64_t(c->part_slot_bytes / 4);
  for (int p = 0; p < n_pairs; ++p) {
    PairLaunch& pl = a->pair[p];
    pl.q = Q[p];
    pl.o = O[p];
    pl.lse = lse ? lse[p] : nullptr;
    seg_table_of(c, ks[p], plans[p], &pl.seg);
    pl.lk = plans[p].key_tokens;
    pl.ntiles = pl.seg.tile_start[pl.seg.nseg];
    pl.n_items = a->nh * a->n_qtiles;
    const size_t region = ks[p] < 0 ? size_t(c->S) : size_t(ks[p]);     // stage k, or the planner's
    pl.part = c->part_slot_bytes
                  ? reinterpret_cast<float*>(c->ws + c->part_off + region * part_region_bytes(c->part_slot_bytes))
                  : nullptr;
  }
}

}  // namespace

extern "C" {

const char* ff_status_str(ff_status s) {
  switch (s) {
    case FF_OK: return "ok";
    case FF_E_INVAL: return "invalid argument (null/misaligned pointer or unsupported shape)";
    case FF_E_ORDER: return "order contract violated (not the next chunk of this stage, or previous stage not run)";
    case FF_E_ANCHOR_MISSING: return "an anchor of Gamma(i) has not been published";
    case FF_E_ANCHOR_EXISTS: return "anchor already published (anchor bank is append-only)";
    case FF_E_RANGE: return "chunk, stage or anchor id out of range";
    case FF_E_NOSPACE: return "workspace smaller than ff_workspace_bytes()";
    case FF_E_HIP: return "HIP runtime call failed";
    case FF_E_STATE: return "operation not possible in the current state";
  }
  return "unknown status";
}

size_t ff_workspace_bytes(const ff_shape* shape, int n_stages, int history) {
  if (!shape_ok(shape, n_stages, history)) return 0;
  return layout_of(shape, n_stages, history).total;
}

ff_status ff_stage_bank_create(const ff_shape* shape, int n_stages, int history, void* workspace,
                               size_t workspace_bytes, ff_ctx** out) {
  if (!out) return FF_E_INVAL;
  *out = nullptr;
  if (!shape_ok(shape, n_stages, history)) return FF_E_INVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) return FF_E_INVAL;
  const Layout L = layout_of(shape, n_stages, history);
  if (workspace_bytes < L.total) return FF_E_NOSPACE;
  ff_ctx* c = new (std::nothrow) ff_ctx();
  if (!c) return FF_E_INVAL;
  c->shape = *shape;
  c->S = n_stages;
  c->H = history;
  c->n_anchor = L.n_anchor;
  c->n_chunk = L.n_chunk;
  c->n_block = (L.n_anchor + shape->planner_latents - 1) / shape->planner_latents;
  c->T = shape->tokens_per_latent;
  c->Lq = int64_t(shape->tokens_per_latent) * shape->chunk_latents;
  c->esz = elem_size(shape->dtype);
  c->ws = static_cast<uint8_t*>(workspace);
  c->ws_bytes = workspace_bytes;
  c->anchor_off = L.anchor_off;
  c->anchor_block = L.anchor_block;
  c->slot_off = L.slot_off;
  c->slot_block = L.slot_block;
  c->part_off = L.part_off;
  c->part_slot_bytes = L.part_slot;
  c->anchor_present.assign(size_t(L.n_anchor), 0);
  c->next.assign(size_t(n_stages), 0);
  c->can_rewind.assign(size_t(n_stages), 0);
  *out = c;
  return FF_OK;
}

void ff_destroy(ff_ctx* ctx) {
  if (!ctx) return;
  if (ctx->prof) dev_profiler_destroy(ctx->prof);
  delete ctx;
}

ff_status ff_anchor_bank_publish(ff_ctx* c, int first_anchor, int n_anchors, const void* K, const void* V,
                                 void* stream) {
  if (!c || !aligned16(K) || !aligned16(V)) return FF_E_INVAL;
  if (n_anchors < 1 || first_anchor < 0 || first_anchor > c->n_anchor - n_anchors) return FF_E_RANGE;
  for (int a = first_anchor; a < first_anchor + n_anchors; ++a)
    if (c->anchor_present[a]) return FF_E_ANCHOR_EXISTS;
  CopyLaunch cl;
  std::memset(&cl, 0, sizeof(cl));
  cl.n_jobs = 1;
  cl.max_nseg = n_anchors;
  cl.L = int32_t(c->T);
  cl.nh = c->shape.n_heads;
  cl.d = c->shape.head_dim;
  cl.dtype = c->shape.dtype;
  cl.block_stride = int64_t(c->anchor_block);
  cl.job[0].rows_k = K;
  cl.job[0].rows_v = V;
  cl.job[0].block = c->ws + c->anchor_off + size_t(first_anchor) * c->anchor_block;
  cl.job[0].nseg = n_anchors;
  if (dev_launch_publish(cl, stream, c->profiling ? c->prof : nullptr, true) != 0) return FF_E_HIP;
  for (int a = first_anchor; a < first_anchor + n_anchors; ++a) c->anchor_present[a] = 1;
  return FF_OK;
}

}  // extern "C"

namespace {

// The renderer call(s) of ff_render_attend[_grouped]; `part` (nullable)
// replaces the workspace's partial region of the call (one pair only).
ff_status render_attend(ff_ctx* c, int n_pairs, const int* chunks, const int* stages, const void* const* Q,
                        const void* const* K, const void* const* V, void* const* O, float* const* lse, void* stream,
                        float* part) {
  if (!c || !chunks || !stages || !Q || !K || !V || !O) return FF_E_INVAL;
  if (n_pairs < 1 || n_pairs > kMaxPairs) return FF_E_INVAL;
  for (int p = 0; p < n_pairs; ++p) {
    if (!aligned16(Q[p]) || !aligned16(K[p]) || !aligned16(V[p]) || !aligned16(O[p])) return FF_E_INVAL;
    if (lse && !lse_ok(lse[p])) return FF_E_INVAL;
  }
  for (int p = 0; p < n_pairs; ++p) {
    const ff_status st = check_call(c, chunks[p], stages[p]);
    if (st != FF_OK) return st;
    for (int q = 0; q < p; ++q)
      if (stages[q] == stages[p]) return FF_E_ORDER;
  }
  ff_key_sources plans[kMaxPairs];
  for (int p = 0; p < n_pairs; ++p) plan_of(c, chunks[p], stages[p], &plans[p]);

  // 1) Tail_H publish of every pair's in-flight K/V into slot i mod (H+1).
  //    That slot holds chunk i-H-1, which no pair of this call reads.
  CopyLaunch cl;
  std::memset(&cl, 0, sizeof(cl));
  cl.n_jobs = n_pairs;
  cl.max_nseg = 1;
  cl.L = int32_t(c->Lq);
  cl.nh = c->shape.n_heads;
  cl.d = c->shape.head_dim;
  cl.dtype = c->shape.dtype;
  cl.block_stride = int64_t(c->slot_block);
  for (int p = 0; p < n_pairs; ++p) {
    cl.job[p].rows_k = K[p];
    cl.job[p].rows_v = V[p];
    cl.job[p].block = slot_ptr(c, stages[p], chunks[p]);
    cl.job[p].nseg = 1;
  }
  Profiler* prof = c->profiling ? c->prof : nullptr;
  if (dev_launch_publish(cl, stream, prof, false) != 0) return FF_E_HIP;

  // 2) Segmented attention over anchors + history + own (now in the bank).
  AttnLaunch al;
  fill_attention(c, n_pairs, stages, plans, c->Lq, Q, O, lse, &al);
  if (part) al.pair[0].part = part;
  if (dev_launch_attention(al, stream, prof) != 0) return FF_E_HIP;

  for (int p = 0; p < n_pairs; ++p) {
    c->next[stages[p]] = chunks[p] + 1;
    c->can_rewind[stages[p]] = 1;
  }
  return FF_OK;
}

}  // namespace

extern "C" {

ff_status ff_render_attend_grouped(ff_ctx* c, int n_pairs, const int* chunks, const int* stages,
                                   const void* const* Q, const void* const* K, const void* const* V,
                                   void* const* O, float* const* lse, void* stream) {
  return render_attend(c, n_pairs, chunks, stages, Q, K, V, O, lse, stream, nullptr);
}

ff_status ff_render_attend(ff_ctx* c, int chunk, int stage, const void* Q, const void* K, const void* V,
                           void* O, float* lse, void* stream) {
  const void* q[1] = {Q};
  const void* k[1] = {K};
  const void* v[1] = {V};
  void* o[1] = {O};
  float* l[1] = {lse};
  return render_attend(c, 1, &chunk, &stage, q, k, v, o, l, stream, nullptr);
}

ff_status ff_render_attend_static_scratch(ff_ctx* c, int chunk, int stage, const void* Q, const void* K,
                                          const void* V, void* O, float* lse, void* stream) {
  if (!c) return FF_E_INVAL;
  // The call's partial slots: two per persistent workgroup.
  const size_t need = part_region_bytes(c->part_slot_bytes);
  float* part = nullptr;
  if (need) {
    void* ptr = nullptr;
    size_t bytes = 0;
    if (dev_static_scratch(&ptr, &bytes) != 0) return FF_E_HIP;
    if (need > bytes) return FF_E_NOSPACE;
    part = static_cast<float*>(ptr);
  }
  const void* q[1] = {Q};
  const void* k[1] = {K};
  const void* v[1] = {V};
  void* o[1] = {O};
  float* l[1] = {lse};
  return render_attend(c, 1, &chunk, &stage, q, k, v, o, l, stream, part);
}

ff_status ff_plan_attend(ff_ctx* c, int block, const void* Q, const void* K, const void* V, void* O, float* lse,
                         int publish, void* stream) {
  if (!c || !aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !lse_ok(lse)) return FF_E_INVAL;
  const ff_status st = check_plan(c, block);
  if (st != FF_OK) return st;
  ff_key_sources plan;
  plan_planner(c, block, &plan);
  int first = 0;
  const int n_own = block_anchors(c, block, &first);

  // 1) Stage the block's in-flight K/V in its anchor-bank entries.
  CopyLaunch cl;
  std::memset(&cl, 0, sizeof(cl));
  cl.n_jobs = 1;
  cl.max_nseg = n_own;
  cl.L = int32_t(c->T);
  cl.nh = c->shape.n_heads;
  cl.d = c->shape.head_dim;
  cl.dtype = c->shape.dtype;
  cl.block_stride = int64_t(c->anchor_block);
  cl.job[0].rows_k = K;
  cl.job[0].rows_v = V;
  cl.job[0].block = anchor_ptr(c, first);
  cl.job[0].nseg = n_own;
  Profiler* prof = c->profiling ? c->prof : nullptr;
  if (dev_launch_publish(cl, stream, prof, true) != 0) return FF_E_HIP;

  // 2) Segmented attention over the earlier blocks' anchors and its own.
  AttnLaunch al;
  const int stage = -1;
  void* o[1] = {O};
  const void* q[1] = {Q};
  float* l[1] = {lse};
  fill_attention(c, 1, &stage, &plan, int64_t(n_own) * c->T, q, o, l, &al);
  if (dev_launch_attention(al, stream, prof) != 0) return FF_E_HIP;

  if (publish)
    for (int a = first; a < first + n_own; ++a) c->anchor_present[a] = 1;
  return FF_OK;
}

ff_status ff_plan_key_plan(const ff_ctx* c, int block, ff_key_sources* out) {
  if (!c || !out) return FF_E_INVAL;
  const ff_status st = check_plan(c, block);
  if (st != FF_OK) return st;
  plan_planner(c, block, out);
  return FF_OK;
}

ff_status ff_bank_tail(const ff_ctx* c, int stage, int* n_out, int* chunk_ids, void* K_out, void* V_out,
                       void* stream) {
  if (!c || !n_out || !chunk_ids) return FF_E_INVAL;
  if (stage < 0 || stage >= c->S) return FF_E_RANGE;
  if ((K_out && !aligned16(K_out)) || (V_out && !aligned16(V_out))) return FF_E_INVAL;
  const int nx = c->next[stage];
  const int n = std::min(nx, c->H);
  *n_out = n;
  for (int j = 0; j < n; ++j) chunk_ids[j] = nx - n + j;
  if ((!K_out && !V_out) || n == 0) return FF_OK;
  CopyLaunch cl;
  std::memset(&cl, 0, sizeof(cl));
  cl.n_jobs = n;
  cl.max_nseg = 1;
  cl.L = int32_t(c->Lq);
  cl.nh = c->shape.n_heads;
  cl.d = c->shape.head_dim;
  cl.dtype = c->shape.dtype;
  cl.block_stride = int64_t(c->slot_block);
  const size_t chunk_bytes = size_t(c->Lq) * size_t(c->shape.n_heads) * size_t(c->shape.head_dim) * size_t(c->esz);
  for (int j = 0; j < n; ++j) {
    cl.job[j].block = slot_ptr(c, stage, nx - n + j);
    cl.job[j].out_k = K_out ? static_cast<uint8_t*>(K_out) + size_t(j) * chunk_bytes : nullptr;
    cl.job[j].out_v = V_out ? static_cast<uint8_t*>(V_out) + size_t(j) * chunk_bytes : nullptr;
    cl.job[j].nseg = 1;
  }
  if (dev_launch_unpack(cl, stream) != 0) return FF_E_HIP;
  return FF_OK;
}

ff_status ff_gamma(const ff_ctx* c, int chunk, int* n_out, int* anchor_ids) {
  if (!c || !n_out || !anchor_ids) return FF_E_INVAL;
  if (chunk < 0 || chunk >= c->n_chunk) return FF_E_RANGE;
  int ids[8];
  const int n = gamma_of(c, chunk, ids);
  for (int j = 0; j < n; ++j) anchor_ids[j] = ids[j];
  *n_out = n;
  return FF_OK;
}

ff_status ff_key_plan(const ff_ctx* c, int chunk, int stage, ff_key_sources* out) {
  if (!c || !out) return FF_E_INVAL;
  const ff_status st = check_call(c, chunk, stage);
  if (st != FF_OK) return st;
  plan_of(c, chunk, stage, out);
  return FF_OK;
}

ff_status ff_stage_next(const ff_ctx* c, int stage, int* next_chunk) {
  if (!c || !next_chunk) return FF_E_INVAL;
  if (stage < 0 || stage >= c->S) return FF_E_RANGE;
  *next_chunk = c->next[stage];
  return FF_OK;
}

ff_status ff_clip_layout(const ff_shape* shape, int n_stages, ff_clip_counts* out) {
  if (!out || !shape_ok(shape, n_stages, 1)) return FF_E_INVAL;
  const Layout L = layout_of(shape, n_stages, 1);
  out->n_anchors = L.n_anchor;
  out->n_chunks = L.n_chunk;
  out->n_planner_blocks = (L.n_anchor + shape->planner_latents - 1) / shape->planner_latents;
  out->n_diagonals = L.n_chunk + n_stages - 1;
  return FF_OK;
}

ff_status ff_planner_block(const ff_shape* shape, int block, int* first_anchor, int* n_anchors) {
  if (!first_anchor || !n_anchors || !shape_ok(shape, 1, 1)) return FF_E_INVAL;
  const int na = layout_of(shape, 1, 1).n_anchor, bp = shape->planner_latents;
  if (block < 0 || block >= (na + bp - 1) / bp) return FF_E_RANGE;
  *first_anchor = block * bp;
  *n_anchors = std::min(bp, na - block * bp);
  return FF_OK;
}

// The anti-diagonal wavefront: diagonal t runs (t-k, k) for every stage k
// whose chunk t-k exists.
ff_status ff_wavefront(const ff_shape* shape, int n_stages, int t, int* n_pairs, int* chunks, int* stages) {
  if (!n_pairs || !chunks || !stages || !shape_ok(shape, n_stages, 1)) return FF_E_INVAL;
  const int nc = layout_of(shape, n_stages, 1).n_chunk;
  if (t < 0 || t > nc + n_stages - 2) return FF_E_RANGE;
  int n = 0;
  for (int k = 0; k < n_stages; ++k) {
    const int i = t - k;
    if (i < 0 || i >= nc) continue;
    chunks[n] = i;
    stages[n] = k;
    ++n;
  }
  *n_pairs = n;
  return FF_OK;
}

ff_status ff_stage_bank_rewind(ff_ctx* c, int stage) {
  if (!c) return FF_E_INVAL;
  if (stage < 0 || stage >= c->S) return FF_E_RANGE;
  if (!c->can_rewind[stage] || c->next[stage] == 0) return FF_E_STATE;
  const int j = c->next[stage] - 1;
  if (stage + 1 < c->S && c->next[stage + 1] > j) return FF_E_STATE;
  c->next[stage] = j;
  c->can_rewind[stage] = 0;
  return FF_OK;
}

ff_status ff_profile_enable(ff_ctx* c, int on) {
  if (!c) return FF_E_INVAL;
  if (on && !c->prof) {
    c->prof = dev_profiler_create();
    if (!c->prof) return FF_E_HIP;
  }
  if (c->prof) {
    dev_profiler_reset(c->prof);
    dev_profiler_families(c->prof, c->prof_families);
  }
  c->profiling = on != 0;
  return FF_OK;
}

ff_status ff_profile_families(ff_ctx* c, unsigned families) {
  if (!c || (families & ~unsigned(FF_PROF_ALL))) return FF_E_INVAL;
  c->prof_families = families;
  if (c->prof) dev_profiler_families(c->prof, families);
  return FF_OK;
}

ff_status ff_profile_read(ff_ctx* c, ff_kernel_times* out) {
  if (!c || !out) return FF_E_INVAL;
  std::memset(out, 0, sizeof(*out));
  if (!c->prof) return FF_OK;
  return dev_profiler_read(c->prof, out) == 0 ? FF_OK : FF_E_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Block-causal attention over a clip at one stage (training form).
// [S] "how it works", training paragraph; reading: chunk i reads the keys of
// ff_render_attend(i, k) with a full bank (see ff.h).
// ---------------------------------------------------------------------------
struct ff_bc {
  ff_shape shape;
  int H = 0;
  int n_anchor = 0, n_chunk = 0;
  int64_t T = 0, Lq = 0, esz = 2;
  uint8_t* ws = nullptr;
  // workspace regions (byte offsets from ws)
  size_t blk_anchor = 0, blk_chunk = 0;
  size_t kv_anchor = 0, vk_anchor = 0, kv_chunk = 0, vk_chunk = 0, qq_chunk = 0, gg_chunk = 0;
  size_t stats = 0, part = 0, part_slot = 0;
  std::vector<BcChunk> chunk;
  std::vector<BcReaders> readers;      // anchors first, then chunks
  Profiler* prof = nullptr;
  bool profiling = false;
};

namespace {

struct BcLayout {
  size_t blk_anchor, blk_chunk, kv_anchor, vk_anchor, kv_chunk, vk_chunk, qq_chunk, gg_chunk;
  size_t stats, part, part_slot, total;
  int n_anchor, n_chunk;
};

bool bc_shape_ok(const ff_shape* s, int H) {
  if (!shape_ok(s, 1, H)) return false;
  const int n_anchor = (s->n_latents + s->anchor_stride - 1) / s->anchor_stride;
  const int n_chunk = s->n_latents / s->chunk_latents;
  return n_anchor <= kBcMaxAnchors && n_chunk <= kBcMaxChunks;
}

BcLayout bc_layout_of(const ff_shape* s) {
  BcLayout L{};
  const size_t esz = s->dtype == FF_F32 ? 4 : 2;
  const size_t T = size_t(s->tokens_per_latent), nh = size_t(s->n_heads), d = size_t(s->head_dim);
  const size_t lq = T * size_t(s->chunk_latents);
  L.n_anchor = (s->n_latents + s->anchor_stride - 1) / s->anchor_stride;
  L.n_chunk = s->n_latents / s->chunk_latents;
  L.blk_anchor = align_up(2 * nh * T * d * esz);
  L.blk_chunk = align_up(2 * nh * lq * d * esz);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  L.kv_anchor = take(size_t(L.n_anchor) * L.blk_anchor);
  L.vk_anchor = take(size_t(L.n_anchor) * L.blk_anchor);
  L.kv_chunk = take(size_t(L.n_chunk) * L.blk_chunk);
  L.vk_chunk = take(size_t(L.n_chunk) * L.blk_chunk);
  L.qq_chunk = take(size_t(L.n_chunk) * L.blk_chunk);
  L.gg_chunk = take(size_t(L.n_chunk) * L.blk_chunk);
  L.stats = take(size_t(L.n_chunk) * nh * lq * 8);
  L.part_slot = s->dtype == FF_BF16 ? align_up(size_t(attn_block_m(d)) * (d + 2) * 4) : 0;
  L.part = take(size_t(kMaxPairs) * part_region_bytes(L.part_slot));
  L.total = off;
  return L;
}

// Key ranges of every chunk and, transposed, the chunks that read each source.
void bc_plan(ff_bc* b) {
  b->chunk.assign(size_t(b->n_chunk), BcChunk{});
  for (int i = 0; i < b->n_chunk; ++i) {
    int ids[8];
    const int na = gamma_ids(b->shape, b->n_anchor, i, ids);
    const int h_first = history_first(b->shape, b->H, na, i, i);
    b->chunk[size_t(i)] = BcChunk{na ? ids[0] : 0, na, h_first, i - h_first + 1};
  }
  // The readers of a source form one run of consecutive chunks: Gamma's
  // anchors and the history start never move backwards as i grows.
  b->readers.assign(size_t(b->n_anchor + b->n_chunk), BcReaders{0, 0});
  for (int i = 0; i < b->n_chunk; ++i) {
    const BcChunk& c = b->chunk[size_t(i)];
    auto add = [&](int src) {
      BcReaders& r = b->readers[size_t(src)];
      if (r.n == 0) r.i0 = i;
      r.n = i - r.i0 + 1;
    };
    for (int a = c.a0; a < c.a0 + c.na; ++a) add(a);
    for (int j = c.j0; j < c.j0 + c.nj; ++j) add(b->n_anchor + j);
  }
}

bool bc_reads(const ff_bc* b, int i, int src) {
  const BcChunk& c = b->chunk[size_t(i)];
  if (src < b->n_anchor) return src >= c.a0 && src < c.a0 + c.na;
  const int j = src - b->n_anchor;
  return j >= c.j0 && j < c.j0 + c.nj;
}

CopyLaunch bc_copy(const ff_bc* b, int64_t L, int64_t block_stride) {
  CopyLaunch cl;
  std::memset(&cl, 0, sizeof(cl));
  cl.L = int32_t(L);
  cl.nh = b->shape.n_heads;
  cl.d = b->shape.head_dim;
  cl.dtype = b->shape.dtype;
  cl.block_stride = block_stride;
  return cl;
}

void bc_add_job(CopyLaunch* cl, const void* rows_k, const void* rows_v, uint8_t* block, int nseg) {
  CopyJob& j = cl->job[cl->n_jobs++];
  j.rows_k = rows_k;
  j.rows_v = rows_v;
  j.block = block;
  j.nseg = nseg;
  cl->max_nseg = std::max(cl->max_nseg, nseg);
}

}  // namespace

extern "C" {

size_t ff_bc_workspace_bytes(const ff_shape* shape, int history) {
  if (!bc_shape_ok(shape, history)) return 0;
  return bc_layout_of(shape).total;
}

ff_status ff_bc_create(const ff_shape* shape, int history, void* workspace, size_t workspace_bytes, ff_bc** out) {
  if (!out) return FF_E_INVAL;
  *out = nullptr;
  if (!bc_shape_ok(shape, history)) return FF_E_INVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))) return FF_E_INVAL;
  const BcLayout L = bc_layout_of(shape);
  if (workspace_bytes < L.total) return FF_E_NOSPACE;
  ff_bc* b = new (std::nothrow) ff_bc();
  if (!b) return FF_E_INVAL;
  b->shape = *shape;
  b->H = history;
  b->n_anchor = L.n_anchor;
  b->n_chunk = L.n_chunk;
  b->T = shape->tokens_per_latent;
  b->Lq = int64_t(shape->tokens_per_latent) * shape->chunk_latents;
  b->esz = elem_size(shape->dtype);
  b->ws = static_cast<uint8_t*>(workspace);
  b->blk_anchor = L.blk_anchor;
  b->blk_chunk = L.blk_chunk;
  b->kv_anchor = L.kv_anchor;
  b->vk_anchor = L.vk_anchor;
  b->kv_chunk = L.kv_chunk;
  b->vk_chunk = L.vk_chunk;
  b->qq_chunk = L.qq_chunk;
  b->gg_chunk = L.gg_chunk;
  b->stats = L.stats;
  b->part = L.part;
  b->part_slot = L.part_slot;
  bc_plan(b);
  for (int src = 0; src < b->n_anchor + b->n_chunk; ++src)      // one run per source
    for (int i = 0; i < b->n_chunk; ++i) {
      const BcReaders& r = b->readers[size_t(src)];
      if (bc_reads(b, i, src) != (r.n > 0 && i >= r.i0 && i < r.i0 + r.n)) {
        delete b;
        return FF_E_INVAL;
      }
    }
  *out = b;
  return FF_OK;
}

void ff_bc_destroy(ff_bc* b) {
  if (!b) return;
  if (b->prof) dev_profiler_destroy(b->prof);
  delete b;
}

ff_status ff_bc_key_plan(const ff_bc* b, int chunk, ff_key_sources* out) {
  if (!b || !out) return FF_E_INVAL;
  if (chunk < 0 || chunk >= b->n_chunk) return FF_E_RANGE;
  const BcChunk& c = b->chunk[size_t(chunk)];
  int ids[8];
  for (int j = 0; j < c.na; ++j) ids[j] = c.a0 + j;
  fill_render_plan(ids, c.na, c.j0, chunk, b->T, b->Lq, b->shape.chunk_latents, out);
  return FF_OK;
}

ff_status ff_bc_forward(ff_bc* b, const void* Ka, const void* Va, const void* Q, const void* K, const void* V,
                        void* O, float* lse, void* stream) {
  if (!b || !aligned16(Ka) || !aligned16(Va) || !aligned16(Q) || !aligned16(K) || !aligned16(V) ||
      !aligned16(O) || !lse_ok(lse))
    return FF_E_INVAL;
  Profiler* prof = b->profiling ? b->prof : nullptr;
  // 1) Operand copies in bank layout: K rows + V^T of every anchor and chunk.
  CopyLaunch ca = bc_copy(b, b->T, int64_t(b->blk_anchor));
  bc_add_job(&ca, Ka, Va, b->ws + b->kv_anchor, b->n_anchor);
  if (dev_launch_layout(ca, stream, prof) != 0) return FF_E_HIP;
  CopyLaunch cc = bc_copy(b, b->Lq, int64_t(b->blk_chunk));
  bc_add_job(&cc, K, V, b->ws + b->kv_chunk, b->n_chunk);
  if (dev_launch_layout(cc, stream, prof) != 0) return FF_E_HIP;

  // 2) The segmented attention kernel, up to kMaxPairs chunks per launch.
  const int64_t row_bytes = b->Lq * b->shape.n_heads * b->shape.head_dim * b->esz;
  for (int i0 = 0; i0 < b->n_chunk; i0 += kMaxPairs) {
    const int n = std::min(kMaxPairs, b->n_chunk - i0);
    AttnLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.n_pairs = n;
    a.nh = b->shape.n_heads;
    a.d = b->shape.head_dim;
    a.lq = int32_t(b->Lq);
    a.n_qtiles = int32_t((b->Lq + attn_block_m(a.d) - 1) / attn_block_m(a.d));
    a.dtype = b->shape.dtype;
    a.scale = float(1.0 / std::sqrt(double(b->shape.head_dim)));
    a.slot_floats = int64_t(b->part_slot / 4);
    for (int p = 0; p < n; ++p) {
      const int i = i0 + p;
      const BcChunk& c = b->chunk[size_t(i)];
      PairLaunch& pl = a.pair[p];
      pl.q = static_cast<const uint8_t*>(Q) + i * row_bytes;
      pl.o = static_cast<uint8_t*>(O) + i * row_bytes;
      pl.lse = lse ? lse + int64_t(i) * b->shape.n_heads * b->Lq : nullptr;
      SegTable& t = pl.seg;
      int32_t tiles = 0, s = 0;
      auto add = [&](const uint8_t* base, int64_t ntok) {
        t.base[s] = base;
        t.n[s] = int32_t(ntok);
        t.tile_start[s] = tiles;
        tiles += int32_t((ntok + kBlockN - 1) / kBlockN);
        ++s;
      };
      for (int x = c.a0; x < c.a0 + c.na; ++x) add(b->ws + b->kv_anchor + size_t(x) * b->blk_anchor, b->T);
      for (int j = c.j0; j < c.j0 + c.nj; ++j) add(b->ws + b->kv_chunk + size_t(j) * b->blk_chunk, b->Lq);
      t.tile_start[s] = tiles;
      t.nseg = s;
      pl.lk = int32_t(int64_t(c.na) * b->T + int64_t(c.nj) * b->Lq);
      pl.ntiles = tiles;
      pl.n_items = a.nh * a.n_qtiles;
      pl.part = b->part_slot ? reinterpret_cast<float*>(b->ws + b->part + size_t(p) * part_region_bytes(b->part_slot))
                             : nullptr;
    }
    if (dev_launch_attention(a, stream, prof) != 0) return FF_E_HIP;
  }
  return FF_OK;
}

ff_status ff_bc_backward(ff_bc* b, const void* Ka, const void* Va, const void* Q, const void* K, const void* V,
                         const void* O, const float* lse, const void* dO, void* dQ, void* dK, void* dV, void* dKa,
                         void* dVa, void* stream) {
  if (!b || !aligned16(Ka) || !aligned16(Va) || !aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      !lse || !lse_ok(lse) || !aligned16(dO) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) ||
      !aligned16(dKa) || !aligned16(dVa))
    return FF_E_INVAL;
  Profiler* prof = b->profiling ? b->prof : nullptr;
  // 1) Operand copies (bf16 MFMA path only; the f32 path reads rows directly).
  if (b->shape.dtype == FF_BF16) {
    CopyLaunch ca = bc_copy(b, b->T, int64_t(b->blk_anchor));
    bc_add_job(&ca, Ka, Va, b->ws + b->kv_anchor, b->n_anchor);
    bc_add_job(&ca, Va, Ka, b->ws + b->vk_anchor, b->n_anchor);
    if (dev_launch_layout(ca, stream, prof) != 0) return FF_E_HIP;
    CopyLaunch cc = bc_copy(b, b->Lq, int64_t(b->blk_chunk));
    bc_add_job(&cc, K, V, b->ws + b->kv_chunk, b->n_chunk);
    bc_add_job(&cc, V, K, b->ws + b->vk_chunk, b->n_chunk);
    bc_add_job(&cc, Q, Q, b->ws + b->qq_chunk, b->n_chunk);
    bc_add_job(&cc, dO, dO, b->ws + b->gg_chunk, b->n_chunk);
    if (dev_launch_layout(cc, stream, prof) != 0) return FF_E_HIP;
  }
  // 2) rowsum(dO * O), then dQ and dK/dV.
  BcLaunch bl;
  std::memset(&bl, 0, sizeof(bl));
  bl.nh = b->shape.n_heads;
  bl.d = b->shape.head_dim;
  bl.T = int32_t(b->T);
  bl.L = int32_t(b->Lq);
  bl.n_anchor = b->n_anchor;
  bl.n_chunk = b->n_chunk;
  bl.dtype = b->shape.dtype;
  bl.scale = float(1.0 / std::sqrt(double(b->shape.head_dim)));
  bl.blk_anchor = int64_t(b->blk_anchor);
  bl.blk_chunk = int64_t(b->blk_chunk);
  bl.kv_anchor = b->ws + b->kv_anchor;
  bl.vk_anchor = b->ws + b->vk_anchor;
  bl.kv_chunk = b->ws + b->kv_chunk;
  bl.vk_chunk = b->ws + b->vk_chunk;
  bl.qq_chunk = b->ws + b->qq_chunk;
  bl.gg_chunk = b->ws + b->gg_chunk;
  bl.Ka = Ka;
  bl.Va = Va;
  bl.Q = Q;
  bl.K = K;
  bl.V = V;
  bl.O = O;
  bl.dO = dO;
  bl.lse = lse;
  bl.stats = reinterpret_cast<float*>(b->ws + b->stats);
  bl.dQ = dQ;
  bl.dK = dK;
  bl.dV = dV;
  bl.dKa = dKa;
  bl.dVa = dVa;
  for (int i = 0; i < b->n_chunk; ++i) bl.chunk[i] = b->chunk[size_t(i)];
  for (int s = 0; s < b->n_anchor + b->n_chunk; ++s) {
    // anchors at [0, n_anchor), chunks at kBcMaxAnchors + j
    const int slot = s < b->n_anchor ? s : kBcMaxAnchors + (s - b->n_anchor);
    bl.readers[slot] = b->readers[size_t(s)];
  }
  if (dev_launch_bc_backward(bl, stream, prof) != 0) return FF_E_HIP;
  return FF_OK;
}

ff_status ff_bc_profile_enable(ff_bc* b, int on) {
  if (!b) return FF_E_INVAL;
  if (on && !b->prof) {
    b->prof = dev_profiler_create();
    if (!b->prof) return FF_E_HIP;
  }
  if (b->prof) dev_profiler_reset(b->prof);
  b->profiling = on != 0;
  return FF_OK;
}

ff_status ff_bc_profile_read(ff_bc* b, ff_kernel_times* out) {
  if (!b || !out) return FF_E_INVAL;
  std::memset(out, 0, sizeof(*out));
  if (!b->prof) return FF_OK;
  return dev_profiler_read(b->prof, out) == 0 ? FF_OK : FF_E_HIP;
}

}  // extern "C"
