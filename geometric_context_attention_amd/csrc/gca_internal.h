// Internal declarations shared by the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gca {

constexpr int kPage = 64;        // token slots per page
constexpr int kHeadDim = 64;     // head dimension the kernels are written for
constexpr int kQBlock = 512;     // query rows per attention workgroup (8 waves x 64)
constexpr int kTargetWgs = 256;  // one workgroup per MI355X compute unit

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
  kCtrError = 4,     // nonzero: a cache kernel found an inconsistency
  kCtrCount = 8
};

// The page list attention walks: ftab[0..a_cnt) ++ slist[0..s_cnt) ++
// ftab[w_first .. w_first + w_cnt), entries of ftab being per frame-page.
struct PageList {
  int32_t a_cnt;        // anchor page entries (n * ppf)
  int32_t s_cnt;        // summary pages
  int32_t s_last_valid; // valid slots of the last summary page
  int32_t w_first;      // first ftab entry of the window + current frames
  int32_t w_cnt;        // window + current page entries
  int32_t ppf;          // pages per frame
  int32_t f_last_valid; // valid slots of a frame's last page
};

struct AttnArgs {
  const void* q;        // [Lq][H][D]
  const void* kpool;
  const void* vpool;
  const int32_t* ftab;
  const int32_t* slist;
  PageList pl;
  int32_t Lq;
  int32_t H;
  int32_t qblocks;      // ceil(Lq / 512)
  int32_t nsplit;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
  // nsplit == 1: final outputs; else partials
  void* out;            // [Lq][H][D] in the stream dtype
  float* lse;           // [H][Lq] or null
  float* part_o;        // [H][nsplit][Lq_pad][D]
  float2* part_ml;      // [H][nsplit][Lq_pad] (max of raw scores, sum of exp)
  int32_t Lq_pad;       // round_up(Lq, 512)
  int32_t pool;         // pages in the pool (entries outside [0, pool) are masked)
};

// Launch wrappers (gca_kernels.hip).  All return hipGetLastError() after launch.
hipError_t launch_reset(const LayerDev& L, int pool_words, int ftab_entries, int slist_entries,
                        hipStream_t st);
hipError_t launch_alloc_frames(const LayerDev& L, int pool_pages, int ppf, int first_frame,
                               int nframes, hipStream_t st);
hipError_t launch_append(const LayerDev& L, const void* k, const void* v, int first_frame,
                         int nframes, int ppf, int F, int H, bool f32, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, bool f32, hipStream_t st);
hipError_t launch_merge(const AttnArgs& a, bool f32, hipStream_t st);
hipError_t launch_evict(const LayerDev& L, int pool_pages, int frame, int ppf, int S, int H,
                        bool f32, hipStream_t st);

}  // namespace gca
