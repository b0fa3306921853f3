// Internal declarations shared by the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gca.h"

namespace gca {

constexpr int kPage = 64;        // token slots per page
constexpr int kHeadDim = 64;     // head dimension the kernels are written for
constexpr int kQBlock = 512;     // query rows per bf16 attention workgroup (8 waves x 64)
constexpr int kF32Rows = 256;    // query rows per fp32 attention workgroup
constexpr int kTargetWgs = 256;  // one workgroup per MI355X compute unit
// Logical pages one key split of the bf16 attention may hold: each workgroup
// resolves its split's page ids into an LDS list of this many entries.
constexpr int kListCap = 4096;
constexpr int kMaxFramePages = 32;  // pages of one frame passed by value (F <= 2048)
// Intra-frame attention of bf16 frames of at most kFrameTiles pages reads the
// input rows directly (the frame mode of the page loop; with rotary angles a
// kernel that holds the whole frame's K and V^T tiles in LDS), up to
// kFrameBatchMax frames per launch.
constexpr int kFrameTiles = 8;
constexpr int kFrameBatchMax = 64;
// Up to kWsplitBatchMax such frames per call run in a kernel that splits each
// frame's pages over the waves of a workgroup (no key splits, no merge); the
// larger calls go to the frame mode of the page loop.  (-DGCA_WS_BATCH_MAX=n
// moves the boundary; the default is where the frame mode became faster.)
#ifndef GCA_WS_BATCH_MAX
#define GCA_WS_BATCH_MAX 4
#endif
static_assert(GCA_WS_BATCH_MAX >= 1 && GCA_WS_BATCH_MAX <= 64, "a batch of the wave-split kernel fits its grid rows");
constexpr int kWsplitBatchMax = GCA_WS_BATCH_MAX;

// Device-side state of one layer's cache, carved from the workspace.
struct LayerDev {
  void* kpool;       // [pool][H][P][D]
  void* vpool;       // [pool][H][D][P], slot s stored at column swap23(s)
  uint32_t* bitmap;  // [ceil(pool/32)], bit set = page in use
  int32_t* ftab;     // [max_frames][ppf], -1 = not resident
  int32_t* slist;    // [max_summary_pages] summary pages in order
  int32_t* ctr;      // counters, see Ctr
};

enum Ctr : int {
  kCtrFrames = 0,    // frames appended
  kCtrTraj = 1,      // frames in trajectory memory
  kCtrSumPages = 2,  // summary pages
  kCtrUsed = 3,      // pages in use
  kCtrError = 4,     // error bits (GCA_ERR_*), sticky until the next reset
  kCtrCount = 8
};

// Page ids of one frame, passed by value.
struct FramePages {
  int32_t p[kMaxFramePages];
};

// The page list attention walks, in logical order:
//   ftab[0 .. a_cnt)                       anchor frame pages
//   slist[0 .. s_cnt)                      summary pages (trajectory memory)
//   ftab[w_first .. w_first + w_cnt)       window frame pages
//   fresh.p[0 .. fresh_cnt)                pages of the frame being appended,
//                                          filled from k_in / v_in on the way
struct PageList {
  int32_t a_cnt;
  int32_t s_cnt;
  int32_t s_last_valid;  // valid slots of the last summary page
  int32_t w_first;
  int32_t w_cnt;
  int32_t fresh_cnt;     // 0 or ppf
  int32_t ppf;           // pages per frame
  int32_t f_last_valid;  // valid slots of a frame's last page
};

struct AttnArgs {
  const void* q;        // [Lq][H][D]
  void* kpool;
  void* vpool;
  const int32_t* ftab;
  const int32_t* slist;
  PageList pl;
  FramePages fresh;     // page ids of the appended frame
  const void* k_in;     // [F][H][D] rows of the appended frame (fresh_cnt > 0)
  const void* v_in;
  int32_t fresh_frame;  // its frame-table slot; -1: not a keyframe (attended, not cached)
  LayerDev L;           // for the bookkeeping of the append (workgroup 0)
  int32_t Lq;
  int32_t H;
  int32_t F;            // rows per frame
  int32_t qblocks;      // query blocks of the kernel's block size
  int32_t nsplit;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
  // nsplit == 1: final outputs; else partials
  void* out;            // [Lq][H][D] in the stream dtype
  float* lse;           // [H][Lq] or null
  void* part_o;         // [H][nsplit][Lq_pad][D]: fp32 O_s (fp32 path) or bf16 O_s / l_s (bf16 path)
  float2* part_ml;      // [H][nsplit][Lq_pad] (max of raw scores, sum of exp)
  int32_t Lq_pad;       // round_up(Lq, 512)
  int32_t pool;         // pages in the pool (entries outside [0, pool) are masked)
  // rotary position embedding: (cos, sin) of channel pair i of row r at
  // rope[r * D/2 + i] for the query rows and, with the same row index, the
  // appended frame's key rows (null: no rotation)
  const float2* rope;
  // profiling: workgroup 0 adds its duration in shader cycles to clock[0] and
  // in 100 MHz reference ticks to clock[1] (null: not sampled)
  unsigned long long* clock;
  // frames of a batched intra-frame launch (grid y; 1 otherwise): frame f
  // reads and writes the rows, outputs and rotary angles after those of
  // frame f-1 and uses the ppf scratch pages after its pages (nsplit == 1)
  int32_t batch;
};

// Moving frame `frame` (pages `src`) into the trajectory memory: its S
// summary rows go to summary slots g0 .. g0+S-1; slot g lives in page
// `tail_page` when g / 64 == tail_index, else in `new_page` (a page that
// starts zero-filled and is appended to the summary list at index
// new_index).  Then the frame's pages are freed.
struct EvictPlan {
  FramePages src;
  int32_t frame;
  int32_t ppf;
  int32_t S;
  int32_t g0;
  int32_t tail_page;   // -1 if the summary list is empty
  int32_t tail_index;  // index of tail_page in the summary list
  int32_t new_page;    // -1 if no page is needed
  int32_t new_index;
};

// Split-K scratch of gca_step_noalloc: a static device array of this many
// bytes (one per GPU, held until the process ends), shared by every call on
// that GPU.  static_scratch_address gives its device address on the current
// device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch_address(void** out);

// Launch wrappers (gca_kernels.hip).  All return hipGetLastError() after launch.
hipError_t launch_reset(const LayerDev& L, int pool_words, int ftab_entries, int slist_entries,
                        hipStream_t st);
hipError_t launch_append(const LayerDev& L, const void* k, const void* v, int frame,
                         const FramePages& pages, int ppf, int F, int H, bool f32,
                         const float2* rope, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, bool f32, hipStream_t st);
// Intra-frame attention of bf16 frames of at most kFrameTiles pages, one page
// per wave (a.nsplit must be 1; batch frames on grid rows).
hipError_t launch_frame_wsplit(const AttnArgs& a, hipStream_t st);
// Merge of the key splits (when a.nsplit > 1) and the eviction (when ev != null),
// in one launch.
hipError_t launch_merge_evict(const AttnArgs& a, const EvictPlan* ev, bool f32, hipStream_t st);

}  // namespace gca
