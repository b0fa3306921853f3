// Host runtime of the GCA library: configuration checks, workspace layout,
// call-order state, page-count prediction and kernel sequencing.
//
// Every cache decision is a deterministic function of the frame counter, so
// the host predicts page use (and refuses a step that would exhaust the pool)
// without reading anything back from the device.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gca.h"
#include "gca_internal.h"

using namespace gca;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GCA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr size_t kClockBytes = 256;  // profiling counters at the end of the workspace
constexpr int kClockSlots = 18;      // shader cycles, reference ticks, 16 phase counters
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Derived sizes and workspace layout of a configuration.
struct Geometry {
  int F = 0, ppf = 0, pool = 0, words = 0, max_sum_pages = 0, f_last_valid = 0;
  int64_t ftab_entries = 0;
  size_t eb = 0;          // element bytes
  size_t pool_bytes = 0;  // one pool (K or V) of one layer
  size_t meta_bytes = 0;  // bitmap + ftab + slist + ctr of one layer
  size_t part_o_bytes = 0, part_ml_bytes = 0;
  size_t scratch_bytes = 0;  // one pool (K or V) of fa_batch * ppf pages for frame attention
  int fa_batch = 1;          // frames per batched intra-frame attention launch
  size_t layer_stride = 0;
  size_t total = 0;
  float scale = 0.f;
};

int query_rows(const gca_config& c) { return c.dtype == GCA_FP32 ? 256 : kQBlock; }

// Key splits per (head, query block): enough workgroups to fill the chip,
// at most max_splits if set, never more than there are pages, and never so
// few that a split can hold more than kListCap pages (that bound wins over
// max_splits).  The kernels weight the appended frame's pages (at most
// kMaxFramePages) by 3/2 when cutting splits, so a split may get up to
// (npg + fresh / 2) / s + 1 pages.
int choose_splits(const gca_config& c, int qblocks, int64_t npg) {
  const int64_t base = (int64_t)c.num_heads * qblocks;
  int64_t s = cdiv(kTargetWgs, base);
  if (c.max_splits > 0 && s > c.max_splits) s = c.max_splits;
  if (s > npg) s = npg;
  s = std::max<int64_t>(s, cdiv(npg + kMaxFramePages, kListCap - 1));
  if (s < 1) s = 1;
  return (int)s;
}

int validate(const gca_config* c, std::string& why) {
  if (c == nullptr) { why = "config is NULL"; return GCA_E_INVALID_ARG; }
  if (c->num_layers < 1) { why = "num_layers must be >= 1"; return GCA_E_INVALID_ARG; }
  if (c->num_heads < 1 || c->num_heads > 4096) { why = "num_heads must be in [1, 4096]"; return GCA_E_INVALID_ARG; }
  if (c->head_dim < 1) { why = "head_dim must be >= 1"; return GCA_E_INVALID_ARG; }
  if (c->head_dim != kHeadDim) { why = "only head_dim 64 is supported"; return GCA_E_UNSUPPORTED; }
  if (c->image_tokens < 1) { why = "image_tokens must be >= 1"; return GCA_E_INVALID_ARG; }
  if (c->summary_tokens < 1 || c->summary_tokens > kPage) {
    why = "summary_tokens must be in [1, 64]"; return GCA_E_INVALID_ARG;
  }
  if (c->image_tokens > (1 << 20)) { why = "image_tokens too large"; return GCA_E_INVALID_ARG; }
  if (c->n_anchor < 1) { why = "n_anchor must be >= 1"; return GCA_E_INVALID_ARG; }
  if (c->k_window < 0) { why = "k_window must be >= 0"; return GCA_E_INVALID_ARG; }
  if (c->max_frames < c->n_anchor) { why = "max_frames must be >= n_anchor"; return GCA_E_INVALID_ARG; }
  if (c->page_tokens != kPage) { why = "only page_tokens 64 is supported"; return GCA_E_UNSUPPORTED; }
  if (c->dtype != GCA_BF16 && c->dtype != GCA_FP32) { why = "dtype must be GCA_BF16 or GCA_FP32"; return GCA_E_INVALID_ARG; }
  if (!(std::isfinite(c->scale) && c->scale >= 0.f)) { why = "scale must be finite and >= 0"; return GCA_E_INVALID_ARG; }
  if (c->pool_pages < 0) { why = "pool_pages must be >= 0"; return GCA_E_INVALID_ARG; }
  if (c->max_splits < 0) { why = "max_splits must be >= 0"; return GCA_E_INVALID_ARG; }
  if (c->keyframe_interval < 0) { why = "keyframe_interval must be >= 0"; return GCA_E_INVALID_ARG; }
  const int64_t F = (int64_t)c->image_tokens + c->summary_tokens;
  if ((int64_t)c->n_anchor * F > (1 << 24)) { why = "anchor block too large"; return GCA_E_INVALID_ARG; }
  const int64_t ppf = cdiv(F, kPage);
  if (ppf > kMaxFramePages) { why = "frames of more than 2048 tokens are not supported"; return GCA_E_UNSUPPORTED; }
  if (c->pool_pages != 0 && c->pool_pages < (int64_t)c->n_anchor * ppf) {
    why = "pool_pages is smaller than the anchor block";
    return GCA_E_INVALID_ARG;
  }
  if ((int64_t)c->max_frames * ppf > (1LL << 30)) { why = "max_frames too large"; return GCA_E_INVALID_ARG; }
  return GCA_OK;
}

// Peak pages of a max_frames stream: anchors + window + current frame +
// summary pages at the last eviction (the tail page is taken before the
// evicted frame's pages are freed).
int64_t interval(const gca_config& c) { return c.keyframe_interval > 1 ? c.keyframe_interval : 1; }

// Keyframes among frames n .. t-1 (frame n + j*m is one).
int64_t keyframes_before(const gca_config& c, int64_t t) {
  return t <= c.n_anchor ? 0 : cdiv(t - c.n_anchor, interval(c));
}

bool is_keyframe(const gca_config& c, int64_t t) {
  return t < c.n_anchor || (t - c.n_anchor) % interval(c) == 0;
}

int64_t peak_pages(const gca_config& c, int ppf) {
  // Window and trajectory memory only grow, so the last step needs the most
  // pages: its own frame's pages, the window it sees, and the summary pages
  // including the one a final eviction takes before freeing.
  const int64_t n = c.n_anchor, k = c.k_window, T = c.max_frames;
  const int64_t wmax = T > n ? std::min<int64_t>(k, keyframes_before(c, T - 1)) : -1;
  const int64_t full = (n + wmax + 1) * ppf;
  const int64_t traj = std::max<int64_t>(0, keyframes_before(c, T) - k);
  return full + cdiv(traj * c.summary_tokens, kPage);
}

void make_geometry(const gca_config& c, Geometry& g) {
  g.F = c.image_tokens + c.summary_tokens;
  g.ppf = (int)cdiv(g.F, kPage);
  g.f_last_valid = g.F - (g.ppf - 1) * kPage;
  const int64_t peak = peak_pages(c, g.ppf);
  g.pool = c.pool_pages > 0 ? c.pool_pages : (int)peak;
  g.words = (int)cdiv(g.pool, 32);
  // The summary list is sized for every frame being cached (gca_step_keyframe
  // lets the caller cache more frames than the keyframe schedule); only the
  // pool is sized for the schedule.
  const int64_t traj_max = std::max<int64_t>(0, (int64_t)c.max_frames - c.n_anchor - c.k_window);
  g.max_sum_pages = (int)std::max<int64_t>(1, cdiv(traj_max * c.summary_tokens, kPage));
  g.ftab_entries = (int64_t)c.max_frames * g.ppf;
  g.eb = c.dtype == GCA_FP32 ? 4 : 2;
  const size_t page_bytes = (size_t)c.num_heads * kPage * kHeadDim * g.eb;
  g.pool_bytes = align256((size_t)g.pool * page_bytes);
  g.meta_bytes = align256((size_t)g.words * 4) + align256((size_t)g.ftab_entries * 4) +
                 align256((size_t)g.max_sum_pages * 4) + align256(kCtrCount * 4);
  g.layer_stride = 2 * g.pool_bytes + g.meta_bytes;
  // split-K scratch, sized for the larger of the anchor block and a step
  const int qr = query_rows(c);
  size_t po = 0, pml = 0;
  const int64_t lq[2] = {(int64_t)c.n_anchor * g.F, g.F};
  for (int64_t L : lq) {
    const int qb = (int)cdiv(L, qr);
    const int64_t lq_pad = cdiv(L, kQBlock) * kQBlock;
    // no step sees more pages than the pool holds, and the pool holds the
    // anchor block (validate), so also a lone frame of intra-frame attention
    const int s = choose_splits(c, qb, std::max<int64_t>(g.pool, (int64_t)c.n_anchor * g.ppf));
    if (s > 1) {
      po = std::max(po, (size_t)c.num_heads * s * lq_pad * kHeadDim * (c.dtype == GCA_FP32 ? 4 : 2));
      pml = std::max(pml, (size_t)c.num_heads * s * lq_pad * 8);
    }
  }
  g.part_o_bytes = align256(po);
  g.part_ml_bytes = align256(pml);
  // a batched intra-frame launch fills the CUs with head x query-block x frame
  // workgroups; each frame of it needs its own ppf scratch pages
  g.fa_batch = (int)std::min<int64_t>(64, std::max<int64_t>(1, cdiv(kTargetWgs, (int64_t)c.num_heads *
                                                                                   cdiv(g.F, query_rows(c)))));
  g.scratch_bytes = align256((size_t)g.fa_batch * g.ppf * page_bytes);
  g.total = g.layer_stride * c.num_layers + g.part_o_bytes + g.part_ml_bytes + kClockBytes +
            2 * g.scratch_bytes;
  g.scale = c.scale > 0.f ? c.scale : 1.0f / std::sqrt((float)c.head_dim);
}

// Host mirror of one layer's page table.  The host takes every allocation
// decision (lowest free page first) and passes the page ids to the kernels,
// which write the device copy of the table; both copies evolve identically.
struct LayerHost {
  bool streaming = false;
  int next = 0;    // next frame index of the stream
  int frames = 0;  // frames appended to the cache (frame-table slots used)
  int traj = 0;    // frames in trajectory memory
  int used = 0;    // pages in use
  int hint = 0;    // no page below this index is free
  std::vector<uint32_t> bits;
  std::vector<int32_t> ftab;
  std::vector<int32_t> slist;

  void init(const Geometry& g) {
    streaming = false;
    next = frames = traj = used = hint = 0;
    bits.assign((size_t)g.words, 0u);
    ftab.assign((size_t)g.ftab_entries, -1);
    slist.assign((size_t)g.max_sum_pages, -1);
  }
  int alloc(int pool) {
    int p = hint;
    while (p < pool && (bits[p >> 5] >> (p & 31) & 1u)) ++p;
    if (p >= pool) return -1;
    bits[p >> 5] |= 1u << (p & 31);
    hint = p + 1;
    ++used;
    return p;
  }
  void release(int p) {
    bits[p >> 5] &= ~(1u << (p & 31));
    if (p < hint) hint = p;
    --used;
  }
  // Pages for frame f, lowest free first, in ascending order.
  bool alloc_frame(int f, int ppf, int pool, FramePages& out) {
    for (int j = 0; j < ppf; ++j) {
      const int p = alloc(pool);
      if (p < 0) return false;
      out.p[j] = p;
      ftab[(size_t)f * ppf + j] = p;
    }
    return true;
  }
};

struct EventPair {
  hipEvent_t a = nullptr, b = nullptr;
  double flop = 0, bytes = 0;
  bool pending = false;
};

}  // namespace

struct gca_ctx {
  gca_config cfg;
  Geometry g;
  char* ws = nullptr;
  std::vector<LayerDev> dev;
  std::vector<LayerHost> host;
  void* part_o = nullptr;
  float2* part_ml = nullptr;
  void* static_scratch = nullptr;       // this device's static split-K scratch (gca_step_noalloc)
  unsigned long long* clock = nullptr;  // [2] device: shader cycles, reference ticks
  LayerDev scratch{};                   // ppf K/V pages for frame attention (pools only)
  const float2* rope = nullptr;         // rotary table of the next calls (gca_set_rotary)
  unsigned long long clock_base[kClockSlots] = {};
  bool f32 = false;
  // profiling
  bool prof = false;
  int64_t prof_every = 1;  // time every prof_every-th attention launch
  int64_t prof_count = 0;
  std::vector<EventPair> ev;
  size_t ev_next = 0;
  double attn_ms = 0, attn_flop = 0, attn_bytes = 0;
  int64_t attn_launches = 0;
};

namespace {

int harvest(gca_ctx* c, EventPair& e) {
  if (!e.pending) return GCA_OK;
  hipError_t r = hipEventSynchronize(e.b);
  if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
  float ms = 0.f;
  r = hipEventElapsedTime(&ms, e.a, e.b);
  if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
  c->attn_ms += ms;
  c->attn_flop += e.flop;
  c->attn_bytes += e.bytes;
  c->attn_launches += 1;
  e.pending = false;
  return GCA_OK;
}

// Bytes of split-K partials (O, then the (m, l) pairs at the next 256-byte
// boundary) of an attention launch with `nsplit` splits over Lq query rows.
size_t partial_bytes(const gca_ctx* c, int Lq, int nsplit, size_t* ml_offset) {
  const size_t lq_pad = (size_t)cdiv(Lq, kQBlock) * kQBlock;
  const size_t o = align256((size_t)c->cfg.num_heads * nsplit * lq_pad * kHeadDim * c->g.eb);
  if (ml_offset) *ml_offset = o;
  return nsplit > 1 ? o + (size_t)c->cfg.num_heads * nsplit * lq_pad * sizeof(float2) : 0;
}

// Attention over the page list `pl` for `Lq` query rows (appending the frame
// `fresh_frame` from k/v when pl.fresh_cnt > 0), then the merge of the key
// splits and the eviction `ev` (if any) in a second launch.  With
// static_partials the split partials go to the static scratch array (the
// caller has checked that they fit) instead of the workspace.
int run_step_kernels(gca_ctx* c, int layer, const void* q, const void* k, const void* v,
                     void* out, float* lse, int Lq, const PageList& pl, const FramePages& fresh,
                     int fresh_frame, const EvictPlan* ev, int64_t keys, hipStream_t st,
                     bool use_scratch = false, int batch = 1, bool static_partials = false) {
  const gca_config& cfg = c->cfg;
  AttnArgs a{};
  a.q = q;
  a.kpool = use_scratch ? c->scratch.kpool : c->dev[layer].kpool;
  a.vpool = use_scratch ? c->scratch.vpool : c->dev[layer].vpool;
  a.ftab = c->dev[layer].ftab;
  a.slist = c->dev[layer].slist;
  a.pl = pl;
  a.fresh = fresh;
  a.k_in = k;
  a.v_in = v;
  a.fresh_frame = fresh_frame;
  a.L = c->dev[layer];
  a.Lq = Lq;
  a.H = cfg.num_heads;
  a.F = c->g.F;
  a.qblocks = (int)cdiv(Lq, query_rows(cfg));
  const int64_t npg = (int64_t)pl.a_cnt + pl.s_cnt + pl.w_cnt + pl.fresh_cnt;
  // intra-frame attention of a few bf16 frames that fit the LDS tiles: one
  // page per wave, no key splits
  const bool wsplit = use_scratch && !c->f32 && c->g.ppf <= kFrameTiles && batch <= kWsplitBatchMax;
  // a batched launch (intra-frame attention) runs one split per frame
  a.nsplit = batch > 1 || wsplit ? 1 : choose_splits(cfg, a.qblocks, npg);
  a.batch = batch;
  a.scale = c->g.scale;
  a.scale_log2 = (float)(c->g.scale * 1.4426950408889634);
  a.out = out;
  a.lse = lse;
  a.part_o = c->part_o;
  a.part_ml = c->part_ml;
  if (static_partials) {
    size_t ml_off = 0;
    if (partial_bytes(c, Lq, a.nsplit, &ml_off) > kStaticScratchBytes)
      return fail(GCA_E_INVALID_ARG, "split partials exceed the static scratch");  // checked by the caller
    a.part_o = c->static_scratch;
    a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(c->static_scratch) + ml_off);
  }
  a.Lq_pad = (int)(cdiv(Lq, kQBlock) * kQBlock);
  a.pool = use_scratch ? c->g.ppf : c->g.pool;
  a.rope = c->rope;
  // profiling samples every prof_every-th attention launch
  const bool sample = c->prof && (c->prof_count++ % c->prof_every) == 0;
  a.clock = sample ? c->clock : nullptr;
  EventPair* ep = nullptr;
  if (sample) {
    ep = &c->ev[c->ev_next];
    c->ev_next = (c->ev_next + 1) % c->ev.size();
    int rc = harvest(c, *ep);
    if (rc != GCA_OK) return rc;
    hipError_t r = hipEventRecord(ep->a, st);
    if (r != hipSuccess) return hip_fail(r, "hipEventRecord");
  }
  hipError_t e = wsplit ? launch_frame_wsplit(a, st) : launch_attention(a, c->f32, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (ep != nullptr) {
    hipError_t r = hipEventRecord(ep->b, st);
    if (r != hipSuccess) return hip_fail(r, "hipEventRecord");
    ep->flop = 4.0 * Lq * (double)keys * cfg.head_dim * cfg.num_heads * batch;
    ep->bytes = 2.0 * (double)keys * cfg.num_heads * cfg.head_dim * c->g.eb * batch;
    ep->pending = true;
  }
  e = launch_merge_evict(a, ev, c->f32, st);
  if (e != hipSuccess) return hip_fail(e, "merge/evict launch");
  return GCA_OK;
}

int check_ctx_layer(gca_ctx* c, int layer) {
  if (c == nullptr) return fail(GCA_E_INVALID_ARG, "context is NULL");
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(GCA_E_INVALID_ARG, "layer out of range");
  return GCA_OK;
}

}  // namespace

extern "C" {

size_t gca_workspace_bytes(const gca_config* cfg) {
  std::string why;
  if (validate(cfg, why) != GCA_OK) {
    g_err = why;
    return 0;
  }
  Geometry g;
  make_geometry(*cfg, g);
  return g.total;
}

int gca_create(const gca_config* cfg, void* dev_workspace, size_t bytes, void* stream,
               gca_ctx** out) {
  std::string why;
  int rc = validate(cfg, why);
  if (rc != GCA_OK) return fail(rc, why);
  if (out == nullptr) return fail(GCA_E_INVALID_ARG, "out is NULL");
  if (dev_workspace == nullptr) return fail(GCA_E_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)dev_workspace & 255) != 0) return fail(GCA_E_INVALID_ARG, "workspace must be 256-byte aligned");
  Geometry g;
  make_geometry(*cfg, g);
  if (bytes < g.total) return fail(GCA_E_INVALID_ARG, "workspace too small: need " + std::to_string(g.total) + " bytes");
  gca_ctx* c = new gca_ctx();
  c->cfg = *cfg;
  c->g = g;
  c->ws = (char*)dev_workspace;
  c->f32 = cfg->dtype == GCA_FP32;
  c->dev.resize(cfg->num_layers);
  c->host.resize(cfg->num_layers);
  for (int l = 0; l < cfg->num_layers; ++l) {
    char* base = c->ws + g.layer_stride * l;
    LayerDev& d = c->dev[l];
    d.kpool = base;
    d.vpool = base + g.pool_bytes;
    char* m = base + 2 * g.pool_bytes;
    d.bitmap = (uint32_t*)m;
    m += align256((size_t)g.words * 4);
    d.ftab = (int32_t*)m;
    m += align256((size_t)g.ftab_entries * 4);
    d.slist = (int32_t*)m;
    m += align256((size_t)g.max_sum_pages * 4);
    d.ctr = (int32_t*)m;
  }
  char* tail = c->ws + g.layer_stride * cfg->num_layers;
  c->part_o = g.part_o_bytes ? (void*)tail : nullptr;
  c->part_ml = g.part_ml_bytes ? (float2*)(tail + g.part_o_bytes) : nullptr;
  c->clock = (unsigned long long*)(tail + g.part_o_bytes + g.part_ml_bytes);
  c->scratch.kpool = tail + g.part_o_bytes + g.part_ml_bytes + kClockBytes;
  c->scratch.vpool = (char*)c->scratch.kpool + g.scratch_bytes;
  hipError_t se = static_scratch_address(&c->static_scratch);  // once per device, cached
  if (se != hipSuccess) {
    delete c;
    return hip_fail(se, "looking up the static scratch");
  }
  rc = gca_reset(c, stream);
  if (rc != GCA_OK) {
    delete c;
    return rc;
  }
  *out = c;
  return GCA_OK;
}

int gca_reset(gca_ctx* c, void* stream) {
  if (c == nullptr) return fail(GCA_E_INVALID_ARG, "context is NULL");
  hipStream_t st = (hipStream_t)stream;
  for (int l = 0; l < c->cfg.num_layers; ++l) {
    hipError_t e = launch_reset(c->dev[l], c->g.words, (int)c->g.ftab_entries, c->g.max_sum_pages, st);
    if (e != hipSuccess) return hip_fail(e, "reset launch");
    c->host[l].init(c->g);
  }
  return GCA_OK;
}

int gca_anchor_init(gca_ctx* c, int32_t layer, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* stream) {
  int rc = check_ctx_layer(c, layer);
  if (rc != GCA_OK) return rc;
  if (!q || !k || !v || !out) return fail(GCA_E_INVALID_ARG, "q, k, v and out must be non-NULL");
  LayerHost& hs = c->host[layer];
  if (hs.streaming || hs.frames != 0) return fail(GCA_E_BAD_STATE, "anchor_init on a layer that is not empty");
  const gca_config& cfg = c->cfg;
  const Geometry& g = c->g;
  const int need = cfg.n_anchor * g.ppf;
  if (need > g.pool - hs.used) return fail(GCA_E_OUT_OF_PAGES, "pool cannot hold the anchor frames");
  hipStream_t st = (hipStream_t)stream;
  const size_t frame_bytes = (size_t)g.F * cfg.num_heads * cfg.head_dim * g.eb;
  for (int f = 0; f < cfg.n_anchor; ++f) {
    FramePages pages{};
    hs.alloc_frame(f, g.ppf, g.pool, pages);
    hipError_t e = launch_append(c->dev[layer], (const char*)k + f * frame_bytes,
                                 (const char*)v + f * frame_bytes, f, pages, g.ppf, g.F,
                                 cfg.num_heads, c->f32,
                                 c->rope ? c->rope + (size_t)f * g.F * (kHeadDim / 2) : nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  PageList pl{};
  pl.a_cnt = need;
  pl.s_last_valid = kPage;
  pl.ppf = g.ppf;
  pl.f_last_valid = g.f_last_valid;
  const int Lq = cfg.n_anchor * g.F;
  FramePages none{};
  rc = run_step_kernels(c, layer, q, k, v, out, lse, Lq, pl, none, -1, nullptr, (int64_t)Lq, st);
  if (rc != GCA_OK) return rc;
  hs.streaming = true;
  hs.frames = cfg.n_anchor;
  hs.next = cfg.n_anchor;
  hs.traj = 0;
  return GCA_OK;
}

namespace {
// append: 1 cache frame t, 0 attend only, -1 follow the keyframe schedule;
// noalloc: split partials in the static scratch array
int step_impl(gca_ctx* c, int32_t layer, const void* q, const void* k, const void* v, void* out,
              float* lse, int append, void* stream, bool noalloc = false) {
  int rc = check_ctx_layer(c, layer);
  if (rc != GCA_OK) return rc;
  if (!q || !k || !v || !out) return fail(GCA_E_INVALID_ARG, "q, k, v and out must be non-NULL");
  LayerHost& hs = c->host[layer];
  if (!hs.streaming) return fail(GCA_E_BAD_STATE, "step before anchor_init");
  const gca_config& cfg = c->cfg;
  const Geometry& g = c->g;
  const int n = cfg.n_anchor, kw = cfg.k_window, S = cfg.summary_tokens;
  const int t = hs.next;
  if (t >= cfg.max_frames) return fail(GCA_E_OUT_OF_PAGES, "stream reached max_frames; reset first");
  // Frame t is appended to frame-table slot hs.frames if it is a keyframe;
  // the window is the last w cached keyframes (slots hs.frames-w .. hs.frames-1).
  const bool key = append < 0 ? is_keyframe(cfg, t) : append != 0;
  const int w = std::min(kw, hs.frames - n);
  const bool evict = key && hs.frames + 1 - n > kw;
  const int nsp = (int)cdiv((int64_t)S * hs.traj, kPage);
  const int new_sum = evict ? (int)(cdiv((int64_t)S * (hs.traj + 1), kPage) - nsp) : 0;
  if ((int64_t)hs.used + g.ppf + new_sum > g.pool)
    return fail(GCA_E_OUT_OF_PAGES, "page pool exhausted at frame " + std::to_string(t));
  if (nsp + new_sum > g.max_sum_pages)  // cannot happen with the list sized for every frame
    return fail(GCA_E_OUT_OF_PAGES, "summary page list full at frame " + std::to_string(t));
  if (noalloc) {
    const int npg = n * g.ppf + nsp + w * g.ppf + g.ppf;
    const int ns = choose_splits(cfg, (int)cdiv(g.F, query_rows(cfg)), npg);
    const size_t need = partial_bytes(c, g.F, ns, nullptr);
    if (need > kStaticScratchBytes)
      return fail(GCA_E_INVALID_ARG, "step " + std::to_string(t) + " needs " + std::to_string(need) +
                                         " bytes of split partials, more than the " +
                                         std::to_string(kStaticScratchBytes) + " of the static scratch");
  }
  hipStream_t st = (hipStream_t)stream;
  // pages of frame t (lowest free first; a non-keyframe gives them back at
  // the end of the step); then, if a keyframe leaves the window, a new
  // summary page (before its pages are freed)
  const int slot = hs.frames;
  FramePages fresh{};
  hs.alloc_frame(slot, g.ppf, g.pool, fresh);
  if (!key)
    for (int j = 0; j < g.ppf; ++j) hs.ftab[(size_t)slot * g.ppf + j] = -1;
  EvictPlan ev{};
  if (evict) {
    const int fe = slot - kw;  // the oldest window keyframe once frame t is in
    ev.frame = fe;
    ev.ppf = g.ppf;
    ev.S = S;
    ev.g0 = S * hs.traj;
    for (int j = 0; j < g.ppf; ++j) ev.src.p[j] = hs.ftab[(size_t)fe * g.ppf + j];
    ev.tail_index = nsp - 1;
    ev.tail_page = nsp > 0 ? hs.slist[nsp - 1] : -1;
    ev.new_page = -1;
    ev.new_index = nsp;
    if (new_sum > 0) {
      ev.new_page = hs.alloc(g.pool);
      hs.slist[nsp] = ev.new_page;
    }
  }
  PageList pl{};
  pl.a_cnt = n * g.ppf;
  pl.s_cnt = nsp;
  pl.s_last_valid = nsp > 0 ? (int)((int64_t)S * hs.traj - (int64_t)(nsp - 1) * kPage) : kPage;
  pl.w_first = (hs.frames - w) * g.ppf;
  pl.w_cnt = w * g.ppf;
  pl.fresh_cnt = g.ppf;
  pl.ppf = g.ppf;
  pl.f_last_valid = g.f_last_valid;
  const int64_t keys = (int64_t)(n + w + 1) * g.F + (int64_t)S * hs.traj;
  rc = run_step_kernels(c, layer, q, k, v, out, lse, g.F, pl, fresh, key ? slot : -1,
                        evict ? &ev : nullptr, keys, st, false, 1, noalloc);
  if (rc != GCA_OK) return rc;
  hs.next = t + 1;
  if (!key) {
    for (int j = 0; j < g.ppf; ++j) hs.release(fresh.p[j]);
    return GCA_OK;
  }
  hs.frames = slot + 1;
  if (evict) {
    for (int j = 0; j < g.ppf; ++j) {
      hs.release(ev.src.p[j]);
      hs.ftab[(size_t)ev.frame * g.ppf + j] = -1;
    }
    hs.traj += 1;
  }
  return GCA_OK;
}

}  // namespace

int gca_step(gca_ctx* c, int32_t layer, const void* q, const void* k, const void* v, void* out,
             float* lse, void* stream) {
  return step_impl(c, layer, q, k, v, out, lse, -1, stream);
}

int gca_step_noalloc(gca_ctx* c, int32_t layer, const void* q, const void* k, const void* v,
                     void* out, float* lse, void* stream) {
  return step_impl(c, layer, q, k, v, out, lse, -1, stream, true);
}

int gca_set_rotary(gca_ctx* c, const float* cos_sin) {
  if (c == nullptr) return fail(GCA_E_INVALID_ARG, "context is NULL");
  c->rope = reinterpret_cast<const float2*>(cos_sin);
  return GCA_OK;
}

int gca_frame_attention(gca_ctx* c, const void* q, const void* k, const void* v, void* out,
                        float* lse, int32_t frames, void* stream) {
  if (c == nullptr) return fail(GCA_E_INVALID_ARG, "context is NULL");
  if (!q || !k || !v || !out) return fail(GCA_E_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (frames < 0) return fail(GCA_E_INVALID_ARG, "frames must be >= 0");
  const Geometry& g = c->g;
  hipStream_t st = (hipStream_t)stream;
  // every frame is a lone "appended frame" over the scratch pages 0..ppf-1
  PageList pl{};
  pl.s_last_valid = kPage;
  pl.fresh_cnt = g.ppf;
  pl.ppf = g.ppf;
  pl.f_last_valid = g.f_last_valid;
  FramePages pages{};
  for (int j = 0; j < g.ppf; ++j) pages.p[j] = j;
  const size_t rows = (size_t)g.F * c->cfg.num_heads * c->cfg.head_dim;
  const float2* table = c->rope;
  int rc = GCA_OK;
  // several frames: batches of up to fa_batch frames, one launch each (frame f
  // of a batch on grid row f, over its own scratch pages); a lone frame: the
  // split-K path over ppf pages.
  // bf16 frames of at most kFrameTiles pages need no scratch pages (their
  // kernels read the input rows): batches of up to kFrameBatchMax
  const int batch_max = g.ppf <= kFrameTiles && c->cfg.dtype == GCA_BF16 ? kFrameBatchMax : g.fa_batch;
  for (int f = 0; f < frames && rc == GCA_OK;) {
    const int nb = std::min(batch_max, frames - f);
    const size_t off = (size_t)f * rows * g.eb;
    if (table != nullptr) c->rope = table + (size_t)f * g.F * (kHeadDim / 2);
    rc = run_step_kernels(c, 0, (const char*)q + off, (const char*)k + off, (const char*)v + off,
                          (char*)out + off, lse ? lse + (size_t)f * c->cfg.num_heads * g.F : nullptr,
                          g.F, pl, pages, -1, nullptr, g.F, st, true, nb);
    f += nb;
  }
  c->rope = table;
  return rc;
}

int gca_step_keyframe(gca_ctx* c, int32_t layer, const void* q, const void* k, const void* v,
                      void* out, float* lse, int32_t append, void* stream) {
  return step_impl(c, layer, q, k, v, out, lse, append != 0 ? 1 : 0, stream);
}

void gca_destroy(gca_ctx* c) {
  if (c == nullptr) return;
  for (EventPair& e : c->ev) {
    if (e.a) (void)hipEventDestroy(e.a);
    if (e.b) (void)hipEventDestroy(e.b);
  }
  delete c;
}

const char* gca_last_error(void) { return g_err.c_str(); }

int gca_plan(const gca_config* cfg, int32_t t, gca_plan_info* out) {
  std::string why;
  int rc = validate(cfg, why);
  if (rc != GCA_OK) return fail(rc, why);
  if (out == nullptr) return fail(GCA_E_INVALID_ARG, "out is NULL");
  if (t < 0 || t >= cfg->max_frames) return fail(GCA_E_INVALID_ARG, "t out of range");
  Geometry g;
  make_geometry(*cfg, g);
  const int64_t n = cfg->n_anchor, k = cfg->k_window, S = cfg->summary_tokens, F = g.F;
  gca_plan_info p{};
  int64_t Lq, npg;
  if (t < n) {
    Lq = n * F;
    p.keys = n * F;
    p.cached_after = n * F;
    npg = n * g.ppf;
    p.used_pages_after = (int32_t)(n * g.ppf);
  } else {
    Lq = F;
    const int64_t kb = keyframes_before(*cfg, t);
    const int64_t w = std::min<int64_t>(k, kb);
    const int64_t traj = std::max<int64_t>(0, kb - k);
    p.keys = (n + w + 1) * F + S * traj;
    npg = n * g.ppf + cdiv(S * traj, kPage) + (w + 1) * g.ppf;
    const int64_t ka = kb + (is_keyframe(*cfg, t) ? 1 : 0);
    const int64_t wa = std::min<int64_t>(k, ka);
    const int64_t traj_after = ka - wa;
    p.cached_after = (n + wa) * F + S * traj_after;
    p.used_pages_after = (int32_t)((n + wa) * g.ppf + cdiv(S * traj_after, kPage));
  }
  p.pages_visible = (int32_t)npg;
  p.pool_pages = g.pool;
  p.pages_per_frame = g.ppf;
  p.qblocks = (int32_t)cdiv(Lq, query_rows(*cfg));
  p.splits = choose_splits(*cfg, p.qblocks, npg);
  p.flop = 4.0 * (double)Lq * (double)p.keys * cfg->head_dim * cfg->num_heads;
  *out = p;
  return GCA_OK;
}

int gca_export_state(gca_ctx* c, int32_t layer, gca_state_host* dst, void* stream) {
  int rc = check_ctx_layer(c, layer);
  if (rc != GCA_OK) return rc;
  if (dst == nullptr) return fail(GCA_E_INVALID_ARG, "dst is NULL");
  hipStream_t st = (hipStream_t)stream;
  const LayerDev& d = c->dev[layer];
  int32_t ctr[kCtrCount];
  hipError_t e = hipMemcpyAsync(ctr, d.ctr, sizeof(ctr), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && dst->used_bitmap)
    e = hipMemcpyAsync(dst->used_bitmap, d.bitmap, (size_t)c->g.words * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && dst->frame_table)
    e = hipMemcpyAsync(dst->frame_table, d.ftab, (size_t)c->g.ftab_entries * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && dst->summary_pages)
    e = hipMemcpyAsync(dst->summary_pages, d.slist, (size_t)c->g.max_sum_pages * 4, hipMemcpyDeviceToHost, st);
  // the device tables, for the comparison with the host's record
  const LayerHost& hs = c->host[layer];
  std::vector<uint32_t> bits(hs.bits.size());
  std::vector<int32_t> ftab(hs.ftab.size()), slist(hs.slist.size());
  if (e == hipSuccess)
    e = hipMemcpyAsync(bits.data(), d.bitmap, bits.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(ftab.data(), d.ftab, ftab.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(slist.data(), d.slist, slist.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "export_state copy");
  const int64_t sum_pages = cdiv((int64_t)c->cfg.summary_tokens * hs.traj, kPage);
  const bool same = bits == hs.bits && ftab == hs.ftab && slist == hs.slist &&
                    ctr[kCtrFrames] == hs.frames && ctr[kCtrTraj] == hs.traj &&
                    ctr[kCtrSumPages] == sum_pages && ctr[kCtrUsed] == hs.used;
  dst->frames_appended = ctr[kCtrFrames];
  dst->n_traj = ctr[kCtrTraj];
  dst->n_summary_pages = ctr[kCtrSumPages];
  dst->used_pages = ctr[kCtrUsed];
  dst->device_error = ctr[kCtrError] | (same ? 0 : GCA_ERR_TABLE_MISMATCH);
  dst->pool_pages = c->g.pool;
  dst->pages_per_frame = c->g.ppf;
  dst->max_frames = c->cfg.max_frames;
  dst->max_summary_pages = c->g.max_sum_pages;
  return GCA_OK;
}

int gca_debug_set_table_entry(gca_ctx* c, int32_t layer, int32_t table, int64_t index,
                              int32_t value, void* stream) {
  int rc = check_ctx_layer(c, layer);
  if (rc != GCA_OK) return rc;
  const int64_t n = table == 0 ? c->g.ftab_entries : table == 1 ? c->g.max_sum_pages : -1;
  if (n < 0) return fail(GCA_E_INVALID_ARG, "table must be 0 (frame table) or 1 (summary list)");
  if (index < 0 || index >= n) return fail(GCA_E_INVALID_ARG, "table index out of range");
  int32_t* dst = (table == 0 ? c->dev[layer].ftab : c->dev[layer].slist) + index;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(dst, &value, 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // `value` lives on this stack frame
  if (e != hipSuccess) return hip_fail(e, "debug table write");
  return GCA_OK;
}

int gca_pool_views(gca_ctx* c, int32_t layer, void** k_pool, void** v_pool, size_t* page_bytes) {
  int rc = check_ctx_layer(c, layer);
  if (rc != GCA_OK) return rc;
  if (k_pool) *k_pool = c->dev[layer].kpool;
  if (v_pool) *v_pool = c->dev[layer].vpool;
  if (page_bytes) *page_bytes = (size_t)c->cfg.num_heads * kPage * kHeadDim * c->g.eb;
  return GCA_OK;
}

int gca_profile_enable(gca_ctx* c, int32_t on) {
  if (c == nullptr) return fail(GCA_E_INVALID_ARG, "context is NULL");
  if (on < 0) return fail(GCA_E_INVALID_ARG, "profile sampling interval is negative");
  if (on) {
    if (c->ev.empty()) {
      c->ev.resize(2048);
      for (EventPair& e : c->ev) {
        hipError_t r = hipEventCreate(&e.a);
        if (r == hipSuccess) r = hipEventCreate(&e.b);
        if (r != hipSuccess) return hip_fail(r, "hipEventCreate");
      }
    }
    for (EventPair& e : c->ev) e.pending = false;
    c->attn_ms = c->attn_flop = c->attn_bytes = 0;
    c->attn_launches = 0;
    // the clock counters only ever grow: remember where they stand
    hipError_t r = hipDeviceSynchronize();
    if (r == hipSuccess) r = hipMemcpy(c->clock_base, c->clock, sizeof(c->clock_base), hipMemcpyDeviceToHost);
    if (r != hipSuccess) return hip_fail(r, "reading the clock counters");
  }
  c->prof = on > 0;
  c->prof_every = on > 0 ? on : 1;
  c->prof_count = 0;
  return GCA_OK;
}

int gca_profile_read(gca_ctx* c, gca_profile* out) {
  if (c == nullptr || out == nullptr) return fail(GCA_E_INVALID_ARG, "NULL argument");
  for (EventPair& e : c->ev) {
    int rc = harvest(c, e);
    if (rc != GCA_OK) return rc;
  }
  out->attn_ms = c->attn_ms;
  out->attn_launches = c->attn_launches;
  out->attn_flop = c->attn_flop;
  out->attn_kv_bytes = c->attn_bytes;
  out->attn_clock_ghz = 0.0;
  unsigned long long now[kClockSlots];
  hipError_t r = hipMemcpy(now, c->clock, sizeof(now), hipMemcpyDeviceToHost);
  if (r != hipSuccess) return hip_fail(r, "reading the clock counters");
  const unsigned long long cyc = now[0] - c->clock_base[0], ticks = now[1] - c->clock_base[1];
  if (ticks > 0) out->attn_clock_ghz = 0.1 * (double)cyc / (double)ticks;
  for (int i = 0; i < 16; ++i) out->phase_cycles[i] = (double)(now[2 + i] - c->clock_base[2 + i]);
  return GCA_OK;
}

}  // extern "C"
