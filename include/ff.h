/*
 * ff.h -- C ABI of the FlashForward renderer hot path on MI355X (gfx950).
 *
 * One renderer call attends a noisy chunk's queries over three key sources at
 * once -- the clean anchor KV chosen by Gamma(i), the same-stage history bank
 * B_k (last H chunks) and the chunk's own in-flight K/V -- and publishes that
 * K/V into B_k by Tail_H, so no cache-update-only forward exists.
 *
 * Pages cited:
 *   [S] "In-Flight KV Cache with Clean Anchors for Faster Autoregressive Video
 *       Diffusion", Korean summary page: sections "what it is" (무엇인가),
 *       "how it works" (어떻게 동작하나, Eq. (2)), "how it differs"
 *       (무엇과 다른가), "how it is used" (어떻게 쓰나).
 *   [A] the same title, abstract page.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are token-major [tokens][n_heads][head_dim], contiguous, in the
 *    context's dtype (bf16 = 2 bytes, f32 = 4 bytes); device pointers are
 *    caller-owned and must be 16-byte aligned.  `lse` is f32 [n_heads][tokens].
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    enqueue kernels on it and return without synchronising; buffers must stay
 *    alive until the stream has passed them.
 *  - Streams and one renderer context: the calls of one stage, and the
 *    planner calls, must be ordered on one stream (or by events), as the
 *    order contract already makes them depend on each other.  Calls of
 *    different stages may run concurrently on different streams: each stage
 *    (and the planner) has its own bank slots and its own split-item partial
 *    region.  The caller orders a call (i, k) after (i, k-1) and after the
 *    publish of every anchor it reads.  A block-causal context's calls share
 *    its whole workspace and must all be ordered on one stream.
 *  - The library allocates no device memory.  All device state (anchor bank,
 *    stage banks, split-item partials) lives in one caller-owned workspace of
 *    ff_workspace_bytes() bytes, 256-byte aligned, which must outlive the ctx.
 *  - The context belongs to the device that is current when its calls are
 *    made; the attention's persistent grid takes that device's CU and XCD
 *    counts (queried once per device).
 *  - Every call validates all arguments and the state contract before it
 *    enqueues anything.  A call that returns an error other than FF_E_HIP has
 *    enqueued nothing and changed no state.  FF_E_HIP means a HIP launch
 *    failed after validation: host metadata is left unchanged, device bank
 *    bytes of the slot being written are undefined.
 *  - One context is used by one host thread at a time (no internal locking).
 *  - The calls enqueue kernel launches only (no allocation, memset, copy or
 *    host wait), so they may be captured into a HIP graph.  A replay repeats
 *    the captured device work; the host bookkeeping (ring slots, next chunk
 *    of each stage) advanced once, at capture.
 */
#ifndef FF_H_
#define FF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FF_OK = 0,
  FF_E_INVAL = -1,           /* null / misaligned pointer, unsupported shape   */
  FF_E_ORDER = -2,           /* (i,k) is not the next call of stage k, chunk i */
                             /* has not run stage k-1 yet, or an earlier      */
                             /* planner block is unpublished                  */
  FF_E_ANCHOR_MISSING = -3,  /* an anchor of Gamma(i) is not published         */
  FF_E_ANCHOR_EXISTS = -4,   /* anchor already published (append-only bank)    */
  FF_E_RANGE = -5,           /* chunk, stage or anchor id out of range         */
  FF_E_NOSPACE = -6,         /* workspace smaller than ff_workspace_bytes()    */
  FF_E_HIP = -7,             /* a HIP runtime call failed                      */
  FF_E_STATE = -8            /* rewind not possible in the current state       */
} ff_status;

typedef enum { FF_BF16 = 0, FF_F32 = 1 } ff_dtype;

/* Gamma(i), the anchor selection of chunk i.  [S] "how it differs" / "how it is
 * used" name it but never write it out; [A] calls the anchors two-sided.
 *  FF_GAMMA_BRACKET  : every anchor at a position in
 *                      [Delta*floor(p0/Delta), Delta*ceil(p1/Delta)], p0..p1 the
 *                      chunk's latent positions (2 anchors, 3 when one lies
 *                      strictly inside the chunk).  Default.
 *  FF_GAMMA_CENTER_LR: the anchor at or left of the chunk's middle latent and
 *                      the next one (always 2 inside the clip).               */
typedef enum { FF_GAMMA_BRACKET = 0, FF_GAMMA_CENTER_LR = 1 } ff_gamma_rule;

/* Static shape of one attention layer.  [S] "how it differs": B_R = 3
 * latents per chunk, B_P = 3 anchors per planner block, Delta = 10,
 * W_ctx = 21, H_P = 6; 81 latents per clip.                                 */
typedef struct {
  int32_t n_heads;            /* >= 1                                         */
  int32_t head_dim;           /* 64 or 128                                    */
  int32_t tokens_per_latent;  /* T >= 8, multiple of 8                        */
  int32_t chunk_latents;      /* B_R (latents per renderer chunk), >= 1       */
  int32_t anchor_stride;      /* Delta: anchors at latent positions 0,D,2D..  */
  int32_t n_latents;          /* clip length, multiple of chunk_latents       */
  int32_t w_ctx;              /* max key latents per call (oldest history is  */
                              /* dropped first beyond it)                     */
  int32_t dtype;              /* ff_dtype                                     */
  int32_t gamma_rule;         /* ff_gamma_rule                                */
  int32_t planner_latents;    /* B_P: anchors per planner block, >= 1         */
  int32_t planner_history;    /* H_P: earlier planner blocks a planner block  */
                              /* attends, >= 0 ([S] "how it differs": 6)      */
} ff_shape;

typedef struct ff_ctx ff_ctx;                    /* opaque host-side state    */

/* Key sources of one call, in the order attention sees them. */
enum { FF_SRC_ANCHOR = 0, FF_SRC_HISTORY = 1, FF_SRC_OWN = 2 };
#define FF_MAX_SOURCES 32
typedef struct {
  int32_t n_sources;
  int32_t kind[FF_MAX_SOURCES];      /* FF_SRC_*                              */
  int32_t id[FF_MAX_SOURCES];        /* anchor id or chunk id                 */
  int32_t n_tokens[FF_MAX_SOURCES];
  int32_t key_tokens;                /* sum of n_tokens (L_k)                 */
  int32_t key_latents;
} ff_key_sources;

/* Accumulated device time per kernel family while profiling is enabled. */
typedef struct {
  int64_t attn_launches;    double attn_ms;      /* segmented attention        */
  int64_t merge_launches;   double merge_ms;     /* merge of split items        */
  int64_t publish_launches; double publish_ms;   /* Tail_H stage-bank publish  */
  int64_t anchor_launches;  double anchor_ms;    /* anchor-bank publish        */
  int64_t layout_launches;  double layout_ms;    /* block-causal operand copies */
  int64_t bwd_pre_launches; double bwd_pre_ms;   /* rowsum(dO*O), -lse*log2(e)  */
  int64_t bwd_dq_launches;  double bwd_dq_ms;    /* dQ (query-major)           */
  int64_t bwd_dk_launches;  double bwd_dk_ms;    /* dK (key-major; fp32: dK+dV) */
  int64_t bwd_dv_launches;  double bwd_dv_ms;    /* dV (key-major)             */
} ff_kernel_times;

/* Bytes of device workspace for a context with n_stages banks of history H.
 * 0 if the shape is unsupported.  Layout: anchor bank (every anchor of the
 * clip), S*(H+1) stage-bank slots, split-item partials (one region per stage
 * and one for planner calls).                                               */
size_t ff_workspace_bytes(const ff_shape* shape, int n_stages, int history);

/* ff_stage_bank_create -- [S] "how it works", Eq. (2): one history bank B_k
 * per denoising stage k (S of them) of capacity H, plus the anchor bank A.
 * Each bank is a ring of H+1 slots so that the publish of chunk i never
 * overwrites chunk i-H, which the same call still reads.  history <= 8.
 * On success *out owns only host memory; the workspace stays the caller's.   */
ff_status ff_stage_bank_create(const ff_shape* shape, int n_stages, int history,
                               void* workspace, size_t workspace_bytes, ff_ctx** out);

/* Frees the host-side context (not the workspace).  NULL is accepted. */
void ff_destroy(ff_ctx* ctx);

/* ff_anchor_bank_publish -- [S] "how it differs": after each completed
 * planner block one cache-extraction forward publishes the block's clean
 * anchor KV.  K, V: [n_anchors*T][n_heads][head_dim] of anchors
 * first_anchor .. first_anchor+n_anchors-1 (anchor a sits at latent a*Delta).
 * Append-only: republishing an anchor is FF_E_ANCHOR_EXISTS.                 */
ff_status ff_anchor_bank_publish(ff_ctx* ctx, int first_anchor, int n_anchors,
                                 const void* K, const void* V, void* stream);

/* ff_render_attend -- [S] "how it works", Eq. (2):
 *   (v_hat, K, V) = F_R(x, c, tau_k; A_Gamma(i), B_k^(i)),
 *   B_k^(i+1)     = Tail_H(B_k^(i) U (i, K, V)).
 * Q, K, V: the chunk's in-flight projections, [B_R*T][n_heads][head_dim].
 * O: same shape, O = softmax(Q K_all^T / sqrt(d)) V_all over the keys of
 * Gamma(i)'s anchors, B_k^(i) (oldest first) and the chunk itself, no mask.
 * lse: natural-log row log-sum-exp [n_heads][B_R*T] f32, or NULL.
 * Then K, V become the newest entry of B_k (the stage-k bank keeps the last H
 * chunks).  Order contract: chunk i must be the next chunk of stage k (0 for
 * an empty bank), chunk i must already have run stage k-1 (k > 0), and every
 * anchor of Gamma(i) must be published; else FF_E_ORDER / FF_E_ANCHOR_MISSING
 * with no state change.  There is deliberately no publish-only call: the
 * renderer has no cache-update-only forward ([S] "what it is").               */
ff_status ff_render_attend(ff_ctx* ctx, int chunk, int stage,
                           const void* Q, const void* K, const void* V,
                           void* O, float* lse, void* stream);

/* ff_render_attend_grouped -- n_pairs independent renderer calls in one
 * launch of each kernel, e.g. the anti-diagonal {(t-k, k)} of the wavefront
 * schedule ([S] "how it works": same-stage dependency; [A] abstract: a
 * chunk's stage cache is ready for the next chunk as soon as it finishes that
 * stage).  Each pair is validated against the state before the call, so the
 * pairs must not depend on one another (at most one pair per stage).
 * Results and bank contents equal n_pairs ff_render_attend calls.
 * 1 <= n_pairs <= 8; arrays are host arrays of length n_pairs; lse[p] may be
 * NULL and lse itself may be NULL.                                           */
ff_status ff_render_attend_grouped(ff_ctx* ctx, int n_pairs, const int* chunks, const int* stages,
                                   const void* const* Q, const void* const* K, const void* const* V,
                                   void* const* O, float* const* lse, void* stream);

/* ff_render_attend_static_scratch -- ff_render_attend for callers that
 * cannot allocate device memory or have the workspace grow: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, validation, results and bank update as ff_render_attend;
 * the only difference is where the call's split-item partials live: in a
 * fixed device array of the library (130 MiB, one per device, held until
 * the process ends) instead of the workspace's partial region.  The call
 * itself allocates nothing.  Its first call on a device takes that array's
 * address (host metadata only).  Every call on one device shares the array
 * and leaves its contents behind: calls that overlap on one device (other
 * streams, other contexts, other host threads) race on it and must be
 * ordered by the caller.  FF_E_NOSPACE if the call's partials would exceed
 * the array (head_dim <= 128 always fits); FF_E_HIP if its address cannot
 * be taken.                                                                  */
ff_status ff_render_attend_static_scratch(ff_ctx* ctx, int chunk, int stage,
                                          const void* Q, const void* K, const void* V,
                                          void* O, float* lse, void* stream);

/* ff_bank_tail -- contents of B_k: *n_out chunk ids, oldest first, written to
 * chunk_ids[0..H-1] (host) immediately; if K_out / V_out are non-NULL their
 * bytes ([n*B_R*T][n_heads][head_dim], the published K/V in the same order)
 * are enqueued on the stream.  [S] "how it works", Eq. (2), Tail_H.          */
ff_status ff_bank_tail(const ff_ctx* ctx, int stage, int* n_out, int* chunk_ids,
                       void* K_out, void* V_out, void* stream);

/* ff_gamma -- Gamma(chunk) under the context's rule: *n_out (<= 3) anchor ids,
 * ascending, into anchor_ids[0..2].  Host only.                               */
ff_status ff_gamma(const ff_ctx* ctx, int chunk, int* n_out, int* anchor_ids);

/* ff_key_plan -- the key sources ff_render_attend(chunk, stage) would read in
 * the current state (after the W_ctx cap).  Host only; validates the order
 * contract exactly like ff_render_attend.                                     */
ff_status ff_key_plan(const ff_ctx* ctx, int chunk, int stage, ff_key_sources* out);

/* Next chunk id stage k expects (== number of chunks it has published). */
ff_status ff_stage_next(const ff_ctx* ctx, int stage, int* next_chunk);

/* Counts that follow from a shape.  [S] "how it differs": 81 latents give 9
 * anchors at 0, 10, .., 80 (3 planner blocks of B_P = 3) and 27 renderer
 * chunks of B_R = 3 latents; [S] "how it works": with one denoising stage
 * per pipeline step the renderer runs as an anti-diagonal wavefront, whose
 * N_c + S - 1 diagonals hold every (chunk, stage) call once.               */
typedef struct {
  int32_t n_anchors;         /* ceil(n_latents / Delta)                      */
  int32_t n_chunks;          /* N_c = n_latents / B_R                        */
  int32_t n_planner_blocks;  /* ceil(n_anchors / B_P)                        */
  int32_t n_diagonals;       /* N_c + n_stages - 1                           */
} ff_clip_counts;

/* ff_clip_layout -- the counts above for `shape` with n_stages stages.
 * Host only; FF_E_INVAL for an unsupported shape or n_stages outside 1..64. */
ff_status ff_clip_layout(const ff_shape* shape, int n_stages, ff_clip_counts* out);

/* ff_planner_block -- anchors of planner block `block`: first_anchor ..
 * first_anchor + n_anchors - 1 ([S] "how it differs": anchors are generated
 * B_P at a time, in order; the last block may be shorter).  Host only;
 * FF_E_RANGE for a block outside the clip.                                  */
ff_status ff_planner_block(const ff_shape* shape, int block, int* first_anchor, int* n_anchors);

/* ff_wavefront -- the renderer calls of anti-diagonal t of the wavefront
 * schedule: the pairs (chunk t-k, stage k) for 0 <= k < n_stages with
 * 0 <= t-k < N_c, in ascending stage order, written to chunks[] and
 * stages[] (host arrays of at least n_stages entries), *n_pairs of them.
 * [S] "how it works": the renderer's same-stage dependency lets the chunks
 * sit at different stages at once, one stage per pipeline step; [A]
 * abstract: once chunk i finishes stage k, its stage-k cache is ready for
 * chunk i+1.  Every dependency of a call on diagonal t -- (i-1, k) and
 * (i, k-1) -- lies on diagonal t-1, so the calls of one diagonal are
 * independent (one per stage: one ff_render_attend_grouped launch, or
 * several when a diagonal holds more than its 8 pairs -- any split is legal),
 * and t = 0 .. N_c+n_stages-2 in order runs every call of the clip legally.
 * Host only; FF_E_RANGE for t outside that range.                          */
ff_status ff_wavefront(const ff_shape* shape, int n_stages, int t, int* n_pairs, int* chunks, int* stages);

/* ff_stage_bank_rewind -- undo the newest publish of stage k (retry of that
 * chunk, or a steady-state replay).  Exact because the ring keeps H+1 slots:
 * the chunk the undone publish evicted is still intact.  Allowed once per
 * publish, and only if stage k+1 has not consumed that chunk; else
 * FF_E_STATE.  Host metadata only; enqueues nothing.  Not in the pages.       */
ff_status ff_stage_bank_rewind(ff_ctx* ctx, int stage);

/* ff_plan_attend -- one planner-role attention call of planner block `block`
 * (anchors block*B_P .. block*B_P + n_b - 1, n_b = B_P except a shorter last
 * block).  [S] "how it differs": anchors are generated B_P at a time and one
 * cache-extraction forward per completed block publishes the block's clean
 * anchor KV; [S] training paragraph: a planner block attends causally to the
 * clean KV of earlier blocks.  Reading taken (not printed on the pages): the
 * block attends the published anchors of the previous min(block, H_P) blocks
 * (oldest first; oldest blocks dropped while the key latents exceed W_ctx)
 * plus its own in-flight K/V, no mask.
 * Q, K, V, O: [n_b*T][n_heads][head_dim]; lse as for ff_render_attend.
 * The block's K/V are staged in its own anchor-bank entries; with publish != 0
 * the call is the cache-extraction forward and those anchors become published
 * (usable by renderer calls), else they stay unpublished and the next call
 * of the block overwrites them.  Order contract: every earlier block
 * published (else FF_E_ORDER) and the block itself not (FF_E_ANCHOR_EXISTS).
 * ff_anchor_bank_publish remains the way to publish anchors computed
 * elsewhere.                                                                  */
ff_status ff_plan_attend(ff_ctx* ctx, int block, const void* Q, const void* K, const void* V,
                         void* O, float* lse, int publish, void* stream);
/* ff_plan_key_plan -- the key sources ff_plan_attend(block) would read in the
 * current state: FF_SRC_ANCHOR entries for earlier blocks' anchors, then one
 * FF_SRC_OWN entry per anchor of the block (id = anchor id).  Host only;
 * validates the order contract exactly like ff_plan_attend.                   */
ff_status ff_plan_key_plan(const ff_ctx* ctx, int block, ff_key_sources* out);
/* Per-kernel device timing: while enabled, each launch is bracketed by HIP
 * events on its stream; ff_profile_read synchronises those events and returns
 * the accumulated totals since enabling (enable also resets them).            */
ff_status ff_profile_enable(ff_ctx* ctx, int on);
ff_status ff_profile_read(ff_ctx* ctx, ff_kernel_times* out);
/* ff_profile_families -- restrict the event pairs to the kernel families set
 * in `families` (bit f = the f-th family of ff_kernel_times: FF_PROF_ATTN,
 * FF_PROF_MERGE, ...; default FF_PROF_ALL).  Each event pair costs a few
 * microseconds of stream time, so a caller timing a whole step can bracket
 * only the kernel it needs.  Holds until changed, across enable/disable.
 * Host only; FF_E_INVAL for a null ctx or bits outside FF_PROF_ALL.          */
enum {
  FF_PROF_ATTN = 1 << 0, FF_PROF_MERGE = 1 << 1, FF_PROF_PUBLISH = 1 << 2, FF_PROF_ANCHOR = 1 << 3,
  FF_PROF_LAYOUT = 1 << 4, FF_PROF_BWD_PRE = 1 << 5, FF_PROF_BWD_DQ = 1 << 6, FF_PROF_BWD_DK = 1 << 7,
  FF_PROF_BWD_DV = 1 << 8, FF_PROF_ALL = (1 << 9) - 1
};
ff_status ff_profile_families(ff_ctx* ctx, unsigned families);

/* ---------------------------------------------------------------------------
 * Block-causal renderer attention over a whole clip at one stage: the
 * training form of the renderer attention, forward and backward.
 * [S] "how it works", training paragraph: a renderer target attends the clean
 * anchor KV that Gamma(i) allows and the previous H chunks at its own noise
 * level; in self-rollout distillation the renderer runs as one block-causal
 * forward over the clip instead of per-chunk cache updates, so that gradients
 * reach earlier chunks from later ones and the planner (through the anchors)
 * from the renderer.
 * Reading taken (not printed on the pages): chunk i's queries attend exactly
 * the keys ff_render_attend(i, k) reads once its bank is full -- the anchors
 * of Gamma(i), chunks max(0, i-H) .. i-1 (oldest dropped first while the key
 * latents exceed W_ctx) and chunk i itself, no mask inside a source -- so
 * chunk i's output equals that call's output on the same K/V.
 *
 * Tensors (token-major, context dtype, 16-byte aligned, caller-owned):
 *   Ka, Va, dKa, dVa   [N_a*T][n_heads][head_dim], anchor a at rows a*T ..
 *   Q, K, V, O, dO,
 *   dQ, dK, dV         [N_c*B_R*T][n_heads][head_dim], chunk i at rows i*B_R*T ..
 *   lse                f32 [N_c][n_heads][B_R*T], natural log
 * with N_a = ceil(n_latents / Delta) and N_c = n_latents / B_R.  The
 * workspace holds the operand copies in bank layout; it is scratch between
 * calls (no state is kept in it from one call to the next).  Limits:
 * N_c <= 96, N_a <= 32.  Same validation / stream / error conventions as the
 * calls above; the gradients are written, not accumulated.                   */
typedef struct ff_bc ff_bc;

/* Workspace bytes of a block-causal context (0 if the shape is unsupported). */
size_t ff_bc_workspace_bytes(const ff_shape* shape, int history);
ff_status ff_bc_create(const ff_shape* shape, int history, void* workspace, size_t workspace_bytes,
                       ff_bc** out);
void ff_bc_destroy(ff_bc* bc);

/* ff_bc_forward -- O and lse of every chunk (lse may be NULL). */
ff_status ff_bc_forward(ff_bc* bc, const void* Ka, const void* Va, const void* Q, const void* K,
                        const void* V, void* O, float* lse, void* stream);

/* ff_bc_backward -- gradients of sum(dO * O) with respect to Q, K, V and the
 * anchors' K, V, given the inputs, the forward's O and lse, and dO.  Every
 * pointer is required.  dK/dV of a chunk sum the contributions of the (up to
 * H+1) chunks that read it; dKa/dVa of an anchor those of the chunks whose
 * Gamma holds it.                                                            */
ff_status ff_bc_backward(ff_bc* bc, const void* Ka, const void* Va, const void* Q, const void* K,
                         const void* V, const void* O, const float* lse, const void* dO,
                         void* dQ, void* dK, void* dV, void* dKa, void* dVa, void* stream);

/* ff_bc_key_plan -- chunk i's key sources (FF_SRC_ANCHOR, FF_SRC_HISTORY,
 * FF_SRC_OWN) as ff_bc_forward reads them.  Host only.                       */
ff_status ff_bc_key_plan(const ff_bc* bc, int chunk, ff_key_sources* out);

/* Per-kernel device timing of a block-causal context (as ff_profile_*). */
ff_status ff_bc_profile_enable(ff_bc* bc, int on);
ff_status ff_bc_profile_read(ff_bc* bc, ff_kernel_times* out);

/* Static description of a status code. */
const char* ff_status_str(ff_status s);

#ifdef __cplusplus
}
#endif

#endif  /* FF_H_ */
