/*
 * gca.h - C ABI of the MI355X (gfx950) Geometric Context Attention library.
 *
 * One GCA layer step, as the LingBot-Map pages describe it: the current
 * frame's M image tokens plus S summary tokens (1 camera, 1 anchor, 4
 * register; gitcode technical summary of lingbot-map, §2.3 summary-token
 * table) attend to every token of the n anchor frames, every token of the k
 * pose-reference window frames before it, and only the S summary tokens of
 * every older frame (technical summary §2.2 frame-type table, §2.5 mask
 * table; "LingBot-Map 论文精读" (lshu.cn) §二 2.1-2.3).  The frame is then
 * appended to a paged KV cache, and a frame leaving the window keeps only its
 * summary rows ("compressing eviction", same page §二 2.3; paged layout:
 * "LingBot-Map 深度解析" (e.mffb.com.cn) §3.4).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Device pointers are HIP device addresses; `stream` is a hipStream_t
 *   passed as void* (NULL = the default stream).  All work is enqueued
 *   asynchronously on `stream`; nothing synchronises the host except
 *   gca_export_state and gca_profile_read.
 * - Token tensors are dense row-major [rows, H, D] (the [tokens, heads,
 *   head_dim] view of a q/k/v projection) in the configured dtype: bf16
 *   (GCA_BF16) or fp32 (GCA_FP32).  Within a frame, rows 0..S-1 are the
 *   summary rows and rows S..S+M-1 the image rows.
 * - The caller owns every buffer (inputs, outputs, workspace) and keeps it
 *   alive until `stream` has passed the call.  The library never allocates
 *   device memory; it copies K and V rows into pages inside the workspace.
 * - Return value: GCA_OK (0) or a negative GCA_E_* code; gca_last_error()
 *   then describes the failure (thread-local).  No exception crosses the ABI.
 *   Errors detected on the host (arguments, call order, pool exhaustion) are
 *   reported before anything is enqueued, so device state is unchanged.
 * - A context is not thread-safe, and its calls must all use one stream:
 *   they share scratch memory in the workspace.
 */
#ifndef GCA_H
#define GCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GCA_BF16 = 0, GCA_FP32 = 1 };

enum {
  GCA_OK = 0,
  GCA_E_INVALID_ARG = -1,  /* bad config, null pointer, layer out of range */
  GCA_E_BAD_STATE = -2,    /* call out of order (step before anchor init, ...) */
  GCA_E_OUT_OF_PAGES = -3, /* the page pool (or max_frames) would be exceeded */
  GCA_E_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  GCA_E_UNSUPPORTED = -5   /* valid but unsupported shape (head_dim, page size) */
};

/* Stream configuration; field names follow the pages' cache-manager fields
 * (deep dive §3.4: number of blocks, max frames, tokens per frame, heads,
 * head dim, special tokens, scale frames, sliding window). */
typedef struct {
  int32_t num_layers;     /* independent GCA layers sharing the context (>= 1) */
  int32_t num_heads;      /* H >= 1 */
  int32_t head_dim;       /* D; must be 64 */
  int32_t image_tokens;   /* M >= 1 */
  int32_t summary_tokens; /* S, 1..64 (6 on the pages; 1 = camera token only) */
  int32_t n_anchor;       /* n >= 1 anchor frames */
  int32_t k_window;       /* k >= 0 window frames; k >= max_frames = full causal */
  int32_t max_frames;     /* frames per stream between resets; sizes the pool */
  int32_t page_tokens;    /* P token slots per page; must be 64 */
  int32_t dtype;          /* GCA_BF16 or GCA_FP32 (accumulation is always fp32) */
  float scale;            /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t pool_pages;     /* 0: the exact peak a max_frames stream needs; else pool size */
  int32_t max_splits;     /* 0: automatic key-split count; else an upper bound (>= 1) */
  int32_t keyframe_interval; /* m (deep dive §3.2): frame t >= n_anchor enters the cache only
                                when (t - n_anchor) % m == 0; other frames are attended (they
                                see the cache and themselves) but not appended.  The window
                                counts cached keyframes.  0 or 1: every frame is cached. */
} gca_config;

typedef struct gca_ctx gca_ctx;

/* Bytes of device workspace the configuration needs (page pools, page tables,
 * split-K scratch).  Returns 0 if the configuration is invalid.  Host only. */
size_t gca_workspace_bytes(const gca_config* cfg);

/* Create a context on the current HIP device over a caller-owned workspace of
 * `bytes` bytes (>= gca_workspace_bytes, 256-byte aligned).  Enqueues one
 * kernel that clears the page tables.  On success *out receives the context. */
int gca_create(const gca_config* cfg, void* dev_workspace, size_t bytes, void* stream,
               gca_ctx** out);

/* Anchor initialisation of `layer` (paper-to-code map §二 2.1; deep dive §3.2):
 * full, unmasked softmax attention among the n*(M+S) tokens of frames 0..n-1,
 * which are then appended to the cache as the anchor frames.
 *   q, k, v: [n*(M+S), H, D] input (device);  out: [n*(M+S), H, D] (device);
 *   lse: [H, n*(M+S)] fp32 log-sum-exp of the scaled scores, or NULL.
 * Requires the layer to be empty (fresh or reset): else GCA_E_BAD_STATE. */
int gca_anchor_init(gca_ctx* ctx, int32_t layer, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* stream);

/* One GCA step of `layer` for its next frame t (t = n, n+1, ...): attend over
 * anchors + trajectory summaries + the window (the k most recent cached
 * keyframes; frames t-k..t-1 when every frame is a keyframe) + frame t itself
 * (technical summary §2.2, §2.5).  If frame t is a keyframe (the config's
 * keyframe_interval schedule, deep dive §3.2) it is appended; then, if more
 * than k keyframes follow the anchors, the oldest one's S summary rows move
 * into the trajectory memory and its pages are freed (paper-to-code map
 * §二 2.3).  A frame that is not a keyframe leaves the cache unchanged.
 *   q, k, v: [M+S, H, D] (device);  out: [M+S, H, D] (device);
 *   lse: [H, M+S] fp32 or NULL.
 * GCA_E_BAD_STATE before anchor init; GCA_E_OUT_OF_PAGES when frame t would
 * exceed max_frames or the pool (checked on the host before any launch). */
int gca_step(gca_ctx* ctx, int32_t layer, const void* q, const void* k, const void* v,
             void* out, float* lse, void* stream);

/* gca_step with the keyframe decision made by the caller (technical summary
 * §5.1 selects keyframes by an optical-flow threshold computed from the
 * model's own predictions): append != 0 caches frame t, append == 0 only
 * attends.  The pool is sized for the config's keyframe_interval schedule;
 * caching more frames than that schedule can end in GCA_E_OUT_OF_PAGES
 * (an interval of 0 or 1 sizes it for every frame).  gca_plan describes the
 * schedule, not the caller's choices. */
int gca_step_keyframe(gca_ctx* ctx, int32_t layer, const void* q, const void* k, const void* v,
                      void* out, float* lse, int32_t append, void* stream);

/* gca_step for callers that cannot allocate device memory at step time (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step, with the same kernels and results, except that
 * the key splits' partial results go to a static device array inside the
 * library (32 MiB, one per GPU, held until the process ends) instead of the
 * context's workspace.  The caller still passes the inputs, the outputs and a
 * context; nothing is allocated and no library allocating routine is called.
 * Every call on one GPU shares that array, so calls that overlap on one GPU
 * (other streams, other contexts, other threads) race.  A step whose
 * partials would need more than the array holds (possible for fp32 frames of
 * at most 256 rows with many visible pages) returns GCA_E_INVALID_ARG before
 * anything is enqueued or changed; gca_step serves such a step. */
int gca_step_noalloc(gca_ctx* ctx, int32_t layer, const void* q, const void* k, const void* v,
                     void* out, float* lse, void* stream);

/* Rotary position embedding for the calls that follow (technical summary
 * §2.7 and the deep dive's 3D-RoPE switch: the model encodes frame time, and
 * optionally patch position, into Q and K; the frequency schedule is not on
 * the pages, so the caller supplies the angles).  cos_sin: device fp32 table
 * [rows][D/2][2] holding (cos, sin) of the angle by which channels (2i, 2i+1)
 * of each row turn (RoFormer rotation, each product rounded separately);
 * rows are the rows of the call: M+S for gca_step / gca_step_keyframe, n*(M+S)
 * for gca_anchor_init, frames*(M+S) for gca_frame_attention.  Queries are
 * rotated before attention and keys before they enter the cache (cached keys
 * stay rotated; V is never rotated).  The table is read when the kernels run,
 * so it must stay valid until then.  NULL switches rotation off (the default). */
int gca_set_rotary(gca_ctx* ctx, const float* cos_sin);

/* Intra-frame attention (the frame-attention layers that alternate with the
 * GCA layers: technical summary §2.1; news article, pipeline figure): full,
 * unmasked softmax attention of each frame's M+S tokens among themselves,
 * for `frames` frames.  Uses the context's shape, dtype and scale; no
 * layer's cache is read or changed.  Frames go in batches, one launch each.
 * bf16 frames of at most 8 pages: a call of up to 4 frames runs one page per
 * wave of a workgroup (32 query rows per workgroup, the waves' partial
 * softmax results combined in LDS: no scratch, no merge launch); larger calls,
 * up to 64 frames per launch, run the GCA step's page loop over the frames'
 * own rows (with rotary angles: each frame held whole in LDS).  Longer frames and the
 * fp32 mode go through scratch pages inside the workspace
 * (ceil(256 / (H * query blocks)) frames per launch, capped at 64; a lone
 * such frame splits its keys, then the merge).
 *   q, k, v: [frames, M+S, H, D] (device);  out: [frames, M+S, H, D] (device);
 *   lse: [frames, H, M+S] fp32 or NULL. */
int gca_frame_attention(gca_ctx* ctx, const void* q, const void* k, const void* v, void* out,
                        float* lse, int32_t frames, void* stream);

/* Free every page of every layer and return all layers to the empty state
 * (window reset of the windowed mode: paper-to-code map §五). */
int gca_reset(gca_ctx* ctx, void* stream);

/* Destroy the host-side context (the workspace stays the caller's). */
void gca_destroy(gca_ctx* ctx);

/* Description of the last error on this thread ("" if none). */
const char* gca_last_error(void);

/* ---- host-only planning: the counts a configuration implies at step t ---- */
typedef struct {
  int64_t keys;            /* keys visible to frame t's queries */
  int64_t cached_after;    /* cached tokens after step t */
  int32_t pages_visible;   /* length of the page list attention walks at step t */
  int32_t used_pages_after;/* pages in use after step t */
  int32_t pool_pages;      /* pool size of the configuration */
  int32_t pages_per_frame; /* ceil((M+S)/P) */
  int32_t splits;          /* key splits of the attention launch at step t */
  int32_t qblocks;         /* 512-row query blocks of the attention launch */
  double flop;             /* 4 * (M+S) * keys * D * H (algorithmic) */
} gca_plan_info;

/* Fill *out for step t of a stream (t < n describes the anchor block, with
 * keys = n*(M+S)).  Host only, no device needed. */
int gca_plan(const gca_config* cfg, int32_t t, gca_plan_info* out);

/* ---- inspection (tests) and profiling ---- */

/* Bits of gca_state_host.device_error. */
enum {
  /* a kernel met a page id outside the pool in the frame table or the
     summary list (it read nothing there and masked every slot of that page);
     set on the device, kept until gca_reset */
  GCA_ERR_PAGE_OUT_OF_POOL = 1,
  /* gca_export_state found the device's frame table, summary list, bitmap or
     counters different from the host's record of every decision it made */
  GCA_ERR_TABLE_MISMATCH = 2
};

typedef struct {
  int32_t frames_appended; /* frames in the cache's frame table so far (anchors, then
                              keyframes); equals the next frame index when every frame
                              is a keyframe */
  int32_t n_traj;          /* frames in the trajectory memory */
  int32_t n_summary_pages;
  int32_t used_pages;
  int32_t pool_pages;
  int32_t pages_per_frame;
  int32_t max_frames;
  int32_t max_summary_pages;
  int32_t device_error;    /* GCA_ERR_* bits; 0 when the device tables are consistent */
  uint32_t* used_bitmap;   /* host buffer [ceil(pool_pages/32)] or NULL */
  int32_t* frame_table;    /* host buffer [max_frames * pages_per_frame] or NULL; -1 = none */
  int32_t* summary_pages;  /* host buffer [max_summary_pages] or NULL */
} gca_state_host;

/* Copy `layer`'s page-table state (counters from device memory, plus the
 * arrays whose pointers are non-NULL) to the host, and check it: the frame
 * table, summary list, bitmap and counters the kernels wrote are compared
 * with the host's own record of every page decision (a difference sets
 * GCA_ERR_TABLE_MISMATCH), and the kernels' error bits are added.
 * Synchronises `stream`. */
int gca_export_state(gca_ctx* ctx, int32_t layer, gca_state_host* dst, void* stream);

/* Failure injection for tests (the consistency check above must catch a
 * corrupted table): write `value` into entry `index` of `layer`'s device frame
 * table (table 0, [max_frames * pages_per_frame] entries) or summary list
 * (table 1, [max_summary_pages] entries), ordered on `stream`, leaving the
 * host's record alone.  An index out of range is GCA_E_INVALID_ARG.  A value
 * outside [0, pool_pages) is never dereferenced: attention masks that page and
 * sets GCA_ERR_PAGE_OUT_OF_POOL.  gca_reset clears the tables and the bits. */
int gca_debug_set_table_entry(gca_ctx* ctx, int32_t layer, int32_t table, int64_t index,
                              int32_t value, void* stream);

/* Device addresses of `layer`'s K and V page pools and the byte size of one
 * page.  Page p of K holds [H][P][D] (slot s of head h at row s); page p of V
 * holds [H][D][P] transposed, slot s at column s with bits 2 and 3 of s
 * swapped.  For tests that compare cached bytes with the inputs. */
int gca_pool_views(gca_ctx* ctx, int32_t layer, void** k_pool, void** v_pool,
                   size_t* page_bytes);

typedef struct {
  double attn_ms;        /* summed duration of the attention kernel launches */
  int64_t attn_launches;
  double attn_flop;      /* summed algorithmic flop of those launches */
  double attn_kv_bytes;  /* summed algorithmic K/V bytes read by those launches */
  double attn_clock_ghz; /* shader clock during the bf16 attention launches, from
                            the cycle and 100 MHz reference counters that one
                            workgroup per launch samples; 0 if none ran */
  double phase_cycles[16]; /* builds with GCA_PHASE_TIMING=1 only (else 0): summed
                              shader cycles of the bf16 attention's phases in
                              workgroup 0 of the sampled launches, waves 0 and 4
                              ([8g + i]: i = 0 arguments and split arithmetic, 1 page
                              list, 2 first pages, 3 MFMA phases, 4 softmax phases,
                              5 barrier and copy waits, 6 epilogue, 7 pages) */
} gca_profile;

/* HIP-event timing of the context's attention launches: on = N > 0 times
 * every N-th launch (1: every launch; a larger N keeps the event records from
 * slowing the stream), 0 disables.  The launches are counted from this call,
 * the first one is timed; enabling clears the accumulators (and waits for the
 * device).  The clock counters are sampled on the same launches.  Returns
 * GCA_E_INVALID_ARG for on < 0. */
int gca_profile_enable(gca_ctx* ctx, int32_t on);

/* Wait for the timed launches to finish and return the accumulators (sums
 * over the sampled launches only). */
int gca_profile_read(gca_ctx* ctx, gca_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* GCA_H */
