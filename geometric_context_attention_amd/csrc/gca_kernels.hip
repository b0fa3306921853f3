// gfx950 kernels of the GCA step: paged-cache maintenance and attention.
//
// Cache format (one layer): a pool of pages of 64 token slots.  K page p holds
// [H][64][D] (slot s of head h at row s).  V page p holds [H][D][64]
// transposed, with slot s stored at column swap23(s) (bits 2 and 3 of s
// exchanged).  That column order is what makes the P^T operand that the
// QK^T accumulator already holds line up with 16-byte V^T fragments in the
// PV product (see k_attn_bf16).
//
// Allocation policy (the oracle models it exactly): the lowest-numbered free
// page first; a frame takes ceil((M+S)/64) pages in ascending order; a frame
// that leaves the window copies its S summary rows to the trajectory memory
// (a packed list of summary pages, a new page taken only when the tail page
// is full) and only then frees its own pages.  The pages describe the
// three-part context (gitcode technical summary of lingbot-map, §2.2 and §2.5)
// and the compressing eviction ("LingBot-Map 论文精读", lshu.cn, §二 2.3); the
// page policy itself is this library's.

#include <math.h>
#include <stddef.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "gca_exp2_poly.h"
#include "gca_internal.h"

namespace gca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swap23(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

// ---------------------------------------------------------------------------
// Cache maintenance
// ---------------------------------------------------------------------------

__global__ void k_reset(LayerDev L, int pool_words, int ftab_entries, int slist_entries) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int stride = gridDim.x * blockDim.x;
  for (int j = i; j < pool_words; j += stride) L.bitmap[j] = 0u;
  for (int j = i; j < ftab_entries; j += stride) L.ftab[j] = -1;
  for (int j = i; j < slist_entries; j += stride) L.slist[j] = -1;
  if (i < kCtrCount) L.ctr[i] = 0;
}

// Rotary position embedding (RoFormer): channels (2i, 2i+1) of a row turn by
// the angle whose cosine and sine are given.  Each product and the sum are
// rounded separately (no fused multiply-add), so the rotated values are the
// ones an unfused fp32 evaluation of the same formula gives.
__device__ __forceinline__ void rope_rotate(float& x0, float& x1, float2 cs) {
#pragma clang fp contract(off)
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Stream elements: bf16 bits (uint16_t) or fp32; bf16 rounding is RNE.
__device__ __forceinline__ float elem_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ __forceinline__ float elem_to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T f32_to_elem(float x);
template <>
__device__ __forceinline__ uint16_t f32_to_elem<uint16_t>(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
template <>
__device__ __forceinline__ float f32_to_elem<float>(float x) { return x; }

// Rotate a 16-byte chunk of 8 bf16 channels d0 .. d0+7 (pairs d0/2 ..) of one
// row; with a factor `s` the rotated values are also multiplied by it, in
// fp32, before the one rounding to bf16.
__device__ __forceinline__ uint4 rope_bf16x8(uint4 v, const float2* cs, float s = 1.f) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
    rope_rotate(x0, x1, cs[e]);
    w[e] = pack_bf16(x0 * s, x1 * s);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 8 bf16 values times `s` (fp32 product, rounded to bf16)
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16(bf16_lo(w[e]) * s, bf16_hi(w[e]) * s);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Grid (ppf, H): copy one head's 64 slots of one page of frame `frame` into
// the page the host chose for it.  K rows are copied as they are; V rows are
// transposed through LDS.  Slots past the frame's last row are zero-filled.
// Workgroup (0, 0) records the pages in the frame table and the bitmap.
// T = uint16_t (bf16 bits) or float.
template <typename T>
__global__ __launch_bounds__(256) void k_append(LayerDev L, const T* __restrict__ kin,
                                                const T* __restrict__ vin, int frame,
                                                FramePages pages, int ppf, int F, int H,
                                                const float2* __restrict__ rope) {
  constexpr int D = kHeadDim, P = kPage;
  const int j = blockIdx.x, h = blockIdx.y;
  const int page = pages.p[j];
  T* kdst = reinterpret_cast<T*>(L.kpool) + ((size_t)page * H + h) * P * D;
  T* vdst = reinterpret_cast<T*>(L.vpool) + ((size_t)page * H + h) * D * P;
  __shared__ T tile[P][D + 1];
  const int row0 = j * P;
  const int nvalid = min(P, F - j * P);
  for (int e = threadIdx.x; e < P * D; e += 256) {
    const int s = e / D, d = e % D;
    T kv = T(0), vv = T(0);
    if (s < nvalid) {
      const size_t src = ((size_t)(row0 + s) * H + h) * D + d;
      kv = kin[src];
      vv = vin[src];
    }
    kdst[e] = kv;
    tile[s][d] = vv;
  }
  if (rope != nullptr) {  // K rows rotated (the frame's rows of the table)
    __syncthreads();
    for (int e = threadIdx.x; e < P * D / 2; e += 256) {
      const int s = e / (D / 2), i = e % (D / 2);
      if (s < nvalid) {
        const size_t src = ((size_t)(row0 + s) * H + h) * D + 2 * i;
        float x0 = elem_to_f32(kin[src]), x1 = elem_to_f32(kin[src + 1]);
        rope_rotate(x0, x1, rope[(size_t)(row0 + s) * (D / 2) + i]);
        kdst[s * D + 2 * i] = f32_to_elem<T>(x0);
        kdst[s * D + 2 * i + 1] = f32_to_elem<T>(x1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < P * D; e += 256) {
    const int d = e / P, c = e % P;
    vdst[e] = tile[swap23(c)][d];
  }
  if (j == 0 && h == 0) {
    if ((int)threadIdx.x < ppf) {
      const int p = pages.p[threadIdx.x];
      L.ftab[frame * ppf + threadIdx.x] = p;
      atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
    }
    if (threadIdx.x == 0) {
      L.ctr[kCtrFrames] = frame + 1;
      atomicAdd(&L.ctr[kCtrUsed], ppf);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention over the page list
// ---------------------------------------------------------------------------

// Logical page i -> physical page and its valid slot count.  Fresh pages
// (the frame being appended) report their index within the frame in `fj`
// (else fj = -1).  A page index outside the pool (only possible if the page
// table is corrupt) reads page 0 with every slot masked.
// The frame table and summary list are read through the constant address
// space (scalar loads): the entries read here are never written during the
// launch (the appended frame's pages come in the arguments), and scalar loads
// do not count against the vector-memory counter the LDS copies are waited on.
typedef const int32_t __attribute__((address_space(4)))* const_i32p;

// Page ids of the appended frame, read in place from the kernel's argument
// block (the kernels below take one AttnArgs by value, which sits at the
// start of that block).  A per-lane index into the by-value copy would make
// the compiler move the whole argument block to scratch memory.
__device__ __forceinline__ const_i32p fresh_page_ids() {
  typedef const char __attribute__((address_space(4)))* const_bytep;
  const const_bytep kargs = (const_bytep)__builtin_amdgcn_kernarg_segment_ptr();
  return (const_i32p)(kargs + offsetof(AttnArgs, fresh) + offsetof(FramePages, p));
}

__device__ __forceinline__ int map_page(const AttnArgs& a, int i, int& valid, int& fj) {
  const PageList& pl = a.pl;
  fj = -1;
  int pg;
  if (i < pl.a_cnt) {
    valid = (i % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = ((const_i32p)a.ftab)[i];
  } else if ((i -= pl.a_cnt) < pl.s_cnt) {
    valid = (i == pl.s_cnt - 1) ? pl.s_last_valid : kPage;
    pg = ((const_i32p)a.slist)[i];
  } else if ((i -= pl.s_cnt) < pl.w_cnt) {
    const int e = pl.w_first + i;
    valid = (e % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = ((const_i32p)a.ftab)[e];
  } else {
    i -= pl.w_cnt;
    fj = i;
    valid = (i == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = fresh_page_ids()[i];
  }
  if ((unsigned)pg >= (unsigned)a.pool) {  // corrupt table: flag it, read nothing
    atomicOr(&a.L.ctr[kCtrError], GCA_ERR_PAGE_OUT_OF_POOL);
    valid = 0;
    fj = -1;
    pg = 0;
  }
  return pg;
}


// Where logical page i's physical id comes from, for one lane (i may differ
// across lanes): the table entry to load (always a valid address) and the
// page's valid slots.
__device__ __forceinline__ const_i32p page_source(const AttnArgs& a, int i, int& valid) {
  const PageList& pl = a.pl;
  if (i < pl.a_cnt) {
    valid = (i % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    return (const_i32p)a.ftab + i;
  }
  if ((i -= pl.a_cnt) < pl.s_cnt) {
    valid = (i == pl.s_cnt - 1) ? pl.s_last_valid : kPage;
    return (const_i32p)a.slist + i;
  }
  if ((i -= pl.s_cnt) < pl.w_cnt) {
    const int e = pl.w_first + i;
    valid = (e % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    return (const_i32p)a.ftab + e;
  }
  i -= pl.w_cnt;
  valid = (i == pl.ppf - 1) ? pl.f_last_valid : kPage;
  return fresh_page_ids() + i;
}

// List entry: physical page << 7 | valid slots; an id outside the pool (only
// possible if the tables are corrupt) becomes page 0 with every slot masked,
// and the layer's error counter records it.
__device__ __forceinline__ uint32_t page_entry(const AttnArgs& a, int pg, int valid) {
  if ((unsigned)pg >= (unsigned)a.pool) {
    atomicOr(&a.L.ctr[kCtrError], GCA_ERR_PAGE_OUT_OF_POOL);
    return 0u;
  }
  return ((uint32_t)pg << 7) | (uint32_t)valid;
}

// First logical page of key split s (s = nsplit gives npg).  Splits take
// equal cost, a page of the appended frame counting 3/2 of another: the
// workgroup holding those pages also writes them to the pool first.  Every
// split keeps at least one page (nsplit <= npg).
__host__ __device__ __forceinline__ int split_begin(const AttnArgs& a, int s) {
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt + a.pl.fresh_cnt;
  const int old_pages = npg - a.pl.fresh_cnt;
  const long long cost = 2LL * old_pages + 3LL * a.pl.fresh_cnt;  // in half pages
  const long long x = cost * s / a.nsplit;
  int b = x <= 2LL * old_pages ? (int)(x / 2) : old_pages + (int)((x - 2LL * old_pages) / 3);
  b = b > s ? b : s;
  const int last = npg - (a.nsplit - s);
  return b < last ? b : last;
}

// Workgroup index -> (head, query block, split).  Workgroups are dealt to the
// 8 XCDs round-robin; when the grid divides evenly, consecutive logical
// indices (the splits and query blocks of one head) land on one XCD and share
// its L2.
__device__ __forceinline__ void decode_wg(const AttnArgs& a, int& h, int& qb, int& s) {
  const int G = gridDim.x, bid = blockIdx.x;
  const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  s = logical % a.nsplit;
  qb = (logical / a.nsplit) % a.qblocks;
  h = logical / (a.nsplit * a.qblocks);
}

// Bookkeeping of the appended frame, done once per launch.
__device__ __forceinline__ void record_fresh_frame(const AttnArgs& a) {
  const int ppf = a.pl.ppf;
  if ((int)threadIdx.x < ppf) {
    const int p = fresh_page_ids()[threadIdx.x];
    a.L.ftab[a.fresh_frame * ppf + threadIdx.x] = p;
    atomicOr(&a.L.bitmap[p >> 5], 1u << (p & 31));
  }
  if (threadIdx.x == 0) {
    a.L.ctr[kCtrFrames] = a.fresh_frame + 1;
    atomicAdd(&a.L.ctr[kCtrUsed], ppf);
  }
}

// bf16 attention, one workgroup = (head, 512 query rows, one key split).
// 8 waves; wave w owns query rows [64w, 64w+64) of the block as two 32-row
// tiles j.  Per 64-slot page:
//   S^T[key][q] = K Q^T   v_mfma_f32_32x32x16_bf16, A = K (LDS), B = Q^T (regs)
//   online softmax per query column, p = exp2((s - m) * scale * log2 e)
//   O^T[d][q] += V^T P^T  A = V^T (LDS), B = P^T straight from the S^T
//                         accumulator: lane half h holds keys {4h..4h+3,
//                         8+4h..8+4h+3} of each 16-key chunk, which is the
//                         order the V page stores them in (swap23).
// Operand layout of the 32x32x16 MFMA: A lane l holds row l%32, k 8(l/32)..+7;
// B lane l holds column l%32, same k; accumulator register r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l%32.
//
// Staging: pages go from HBM straight into a ring of four LDS slots with
// global_load_lds_dwordx4 (no registers), three pages ahead of the one being
// computed, which hides the HBM latency.  Each 8 KB tile (K [64][64] or V^T
// [64][64]) is stored unpadded with an XOR swizzle: 16-byte chunk c of row r
// sits at chunk c ^ ((r >> 1) & 7), so the fragment reads are bank-conflict free.
// The loop is unrolled over the ring so every slot index is a constant (the
// compiler can then tell the slots apart and only waits where this code asks
// it to: vmcnt for the copies, one barrier per page).
// The running max is only raised (and O rescaled) when a page's probabilities
// against the current max grow too large (see valu_phase).
// Pages of the frame being appended are first written to their pool pages by
// the workgroups whose split holds them (V transposed through LDS), then read
// back through the ring like any other page.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#ifndef GCA_PINGPONG
#define GCA_PINGPONG 1
#endif
#ifndef GCA_RING
#define GCA_RING 6
#endif
#ifndef GCA_AHEAD
#define GCA_AHEAD 4
#endif
// Exponentials of a page computed on the FMA path instead of v_exp_f32: this
// many of every 16 (0, 4 or 8); see exp2_poly.
#ifndef GCA_SOFT_EXP
#define GCA_SOFT_EXP 0
#endif
static_assert(GCA_SOFT_EXP == 0 || GCA_SOFT_EXP == 4 || GCA_SOFT_EXP == 8, "a quarter or a half");
// 1: the older wave group (A, favoured by the issue arbiter) computes its
// exponent arguments in its softmax phase, the younger one beside its MFMAs.
#ifndef GCA_ASYM_ARGS
#define GCA_ASYM_ARGS 0
#endif
constexpr bool kAsymArgs = GCA_ASYM_ARGS != 0;
// 1: the stream kernel multiplies Q by scale * log2 e before the QK^T
// product (Q rounded to bf16 once more), so that the scores come out of the
// matrix core in log2 units, and it subtracts a running max only once some
// row of the wave needs one (see valu_phase_qs): the softmax then runs no
// per-score arithmetic before the exponential.  0: every score is turned
// into s * scale * log2 e - m by a multiply-add.
#ifndef GCA_QSCALE
#define GCA_QSCALE 0
#endif
// 1: the QK^T products of a page run d-chunk by d-chunk with the next
// chunk's K fragments read one chunk ahead; 0: key tile by key tile, each
// fragment read just before its two products.
#ifndef GCA_KPREFETCH
#define GCA_KPREFETCH 0
#endif
// Independent accumulator chains of a lane's row sum over a page (1, 2 or 4)
#ifndef GCA_SUM_CHAINS
#define GCA_SUM_CHAINS 1
#endif
constexpr int kSumChains = GCA_SUM_CHAINS;
static_assert(kSumChains == 1 || kSumChains == 2 || kSumChains == 4, "1, 2 or 4 chains");
// Intra-frame attention without rotary angles through the pipelined page
// loop (frame mode of k_attn_bf16) instead of k_frame_attn_bf16.
#ifndef GCA_FRAME_RING
#define GCA_FRAME_RING 1
#endif
// ... with persistent workgroups when the items outnumber the CUs
#ifndef GCA_FRAME_PERSIST
#define GCA_FRAME_PERSIST 1
#endif
// 1: the stream loop also issues page j+kAhead's copy in page j's MFMA phase,
// after its V reads (as the frame mode must), instead of in its softmax phase
#ifndef GCA_STAGE_MFMA
#define GCA_STAGE_MFMA 0
#endif
// k_frame_wsplit_bf16: V copied slot-major and read transposed (1) or
// transposed through registers (0)
#ifndef GCA_WS_VROW
#define GCA_WS_VROW 1
#endif

// Phase timing (diagnostic builds, GCA_PHASE_TIMING=1): in workgroup 0 of a
// sampled launch (AttnArgs::clock set), wave 0 (group A) and wave 4 (group B)
// add the shader cycles (s_memtime) of each phase of k_attn_bf16 to
// clock[2 + 8g + i], g = 0 for wave 0 and 1 for wave 4:
//   i = 0  kernel start to the Q loads issued (arguments, split arithmetic)
//       1  to the split's page list in LDS
//       2  to the first pages landed (the loop starts)
//       3  MFMA phases            4  softmax (VALU) phases
//       5  waits at the barriers and on the copies
//       6  the last PV, the epilogue and the output stores
//       7  pages walked
// Reading the timer waits on the wave's scalar/LDS counter, so these builds
// run a little slower; the default build has none of it.
#ifndef GCA_PHASE_TIMING
#define GCA_PHASE_TIMING 0
#endif
constexpr bool kPhaseTiming = GCA_PHASE_TIMING != 0;

struct PhaseClock {
  unsigned long long t, acc[8];
  bool on;
  __device__ __forceinline__ void start(bool enabled) {
    on = kPhaseTiming && enabled;
    if (on) {
      t = __builtin_amdgcn_s_memtime();
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0;
    }
  }
  __device__ __forceinline__ void lap(int i) {
    if (kPhaseTiming && on) {
      const unsigned long long n = __builtin_amdgcn_s_memtime();
      acc[i] += n - t;
      t = n;
    }
  }
  __device__ __forceinline__ void flush(unsigned long long* clock, int g, int pages, bool lane0) {
    if (kPhaseTiming && on && lane0) {
      acc[7] = (unsigned long long)pages;
#pragma unroll
      for (int i = 0; i < 8; ++i) atomicAdd(&clock[2 + 8 * g + i], acc[i]);
    }
  }
};
constexpr int kRing = GCA_RING;    // LDS page slots
constexpr int kAhead = GCA_AHEAD;  // a wave stages page j + kAhead while it computes page j
static_assert(kRing >= kAhead + 2, "a slot is refilled only after both wave groups have read it");
constexpr int kTileElems = 4096;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kAttnWaves = 8;  // 512 threads, 2 waves per SIMD

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max / sum of a lane's value and the value of the lane 32 apart (the two
// halves of a wave hold the two key halves of the same query column)
__device__ __forceinline__ float half_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float half_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// element offset of 16-byte chunk c of row r in a swizzled 64x64 tile: the
// chunk index is XORed with (r >> 1) & 7, so the 16 rows one ds_read_b128
// pass touches (two 128-byte rows per 256 bytes of banks) hit 16 different
// 16-byte bank groups
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// V tiles of the frame mode are slot-major (row r = slot, 64 d); 16-byte
// chunk c of slot r sits at chunk position c ^ vswz(r), so that the rows one
// transposing read takes (see vrow_offsets) fall on different banks
__device__ __forceinline__ int vswz(int r) { return (r & 3) << 1; }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane 4a+b gets
// element b of the 8-byte chunks addressed by lanes a, a+4, a+8 and a+12 of
// its group, in that order
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) uint16_t* lds_u16;
  typedef __attribute__((address_space(3))) bf16x4* lds_v4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_v4>((lds_u16)(const_cast<uint16_t*>(p))));
}

// Per-lane element offsets into a slot-major V tile for the PV operand of
// d-tile dt (v_mfma_f32_32x32x16_bf16 A operand: lane (l32, hf) holds d =
// 32dt + l32 against the keys of chunk kc that the V^T column order gives:
// slots swap23(16kc + 8hf + e), e = 0..7).  Two transposing reads, at
// offset + 1024kc and + 1024kc + 512, give e = 0..3 and 4..7: address lane
// 4e' + a of a 16-lane group points at slot 16kc + 8r + 4hf + e' (the
// swap23 image of 16kc + 8hf + 4r + e'), d = 32dt + 16(l32 >> 4) + 4a.
__device__ __forceinline__ int vrow_offset(int dt, int lane) {
  const int hf = lane >> 5, g = (lane >> 4) & 1, jl = lane & 15;
  const int e = jl >> 2, a = jl & 3;
  const int d0 = dt * 32 + 16 * g + 4 * a;
  const int slot = hf * 4 + e;  // plus 16kc + 8r, which keep slot & 3
  return slot * 64 + (((d0 >> 3) ^ vswz(slot)) << 3) + ((d0 >> 2) & 1) * 4;
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding; expcnt and
// lgkmcnt left at their maxima)
#define GCA_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(0x0F70 | ((N) & 15) | (((N) >> 4) << 14))

// Workgroup barrier without a memory fence: the copies into LDS are made
// visible by the explicit vmcnt wait before it, and the compiler is kept from
// moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Scores of the empty slots (key >= valid) of a page become -inf.  Keys of
// register r of tile kt are 32kt + 8(r/4) + 4h + r%4 for lane half h, so the
// slots form a suffix; a group of four registers is only looked at when the
// (uniform) key range it covers reaches valid.
// Score of an empty slot: -inf, or, when some exponentials run on the FMA
// path, a finite value far below any real score (its exponential is still 0,
// and the range reduction of exp2_poly stays finite).
constexpr float kMaskedScore = GCA_SOFT_EXP ? -1e30f : -INFINITY;

template <int NJ>
__device__ __forceinline__ void mask_page(f32x16 (&sc)[2][NJ], int valid, int hf) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (kt * 32 + 8 * g + 7 >= valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool dead = kt * 32 + 8 * g + 4 * hf + q >= valid;
#pragma unroll
          for (int j = 0; j < NJ; ++j) sc[kt][j][4 * g + q] = dead ? kMaskedScore : sc[kt][j][4 * g + q];
        }
      }
    }
}

// The running max m of a row is kept in log2 units of the scaled scores
// (s * scale * log2 e).  The MFMA phase turns the scores of a page in place
// into x = s * scale * log2 e - m, beside the PV product (see mfma_phase);
// the VALU phase then only exponentiates.
//
// 2^x on the FMA path (Cody-Waite range reduction: 2^x = 2^floor(x) * 2^f
// with f = x - floor(x) in [0, 1); 2^f from a minimax polynomial by Horner's
// rule, then an exact ldexp).  The coefficients and the error bound, 7.5e-5
// relative over the arguments the softmax produces, come from fit_exp2.py.
// x = -inf is never passed (masked slots are finite when this is used).
__device__ __forceinline__ float exp2_poly(float x) {
  const float f = __builtin_amdgcn_fractf(x);
  const int n = (int)floorf(x);
  float p = __builtin_fmaf(GCA_EXP2_C3, f, GCA_EXP2_C2);
  p = __builtin_fmaf(p, f, GCA_EXP2_C1);
  p = __builtin_fmaf(p, f, GCA_EXP2_C0);
  return __builtin_amdgcn_ldexpf(p, n);
}
static_assert(GCA_EXP2_POLY_DEGREE == 3, "exp2_poly evaluates a cubic");

// Register r of a 16-register score group takes its exponential from
// exp2_poly when it is one of the GCA_SOFT_EXP of 16 spread evenly.
__device__ __forceinline__ constexpr bool soft_exp_slot(int r) {
  return GCA_SOFT_EXP > 0 && r % (16 / (GCA_SOFT_EXP > 0 ? GCA_SOFT_EXP : 16)) ==
                                 16 / (GCA_SOFT_EXP > 0 ? GCA_SOFT_EXP : 16) - 1;
}

// p = exp2(x - shift) as packed bf16 P^T fragments (pf[j][kc]: 16-key chunk
// kc of the page); psum[j] is the sum of the same rounded values over this
// lane's 32 keys (v_dot2 with (1, 1), in kSumChains independent
// accumulator chains added pairwise at the end).
template <int NJ, bool kShift>
__device__ __forceinline__ void page_exp(const f32x16 (&sc)[2][NJ], const float (&shift)[NJ],
                                         bf16x8 (&pf)[NJ][4], float (&psum)[NJ]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = kShift ? sc[kt][j][r] - shift[j] : sc[kt][j][r];
        pf[j][kt * 2 + (r >> 3)][r & 7] = (__bf16)(soft_exp_slot(r) ? exp2_poly(x) : __builtin_amdgcn_exp2f(x));
      }
    float acc[kSumChains];
#pragma unroll
    for (int t = 0; t < kSumChains; ++t) acc[t] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pf[j][kc][e], pf[j][kc][e + 1]};
        const int t = (kc * 4 + e / 2) % kSumChains;
        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc[t], false);
      }
#pragma unroll
    for (int w = 1; w < kSumChains; w *= 2)
#pragma unroll
      for (int t = 0; t < kSumChains; t += 2 * w) acc[t] += acc[t + w];
    psum[j] = acc[0];
  }
}

// Move the running max up to the page's row max (on a split's first page:
// set it, nothing has been summed yet) and rescale l and O by the rise;
// shift[j] receives the rise, by which the page's x must still come down.
template <int NJ>
__device__ __forceinline__ void raise_max(const f32x16 (&sc)[2][NJ], float (&m)[NJ], float (&l)[NJ],
                                          f32x16 (&o)[2][NJ], float (&shift)[NJ], bool first) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const f32x16& u = sc[0][j];
    const f32x16& v = sc[1][j];
    const float a = max3f(u[0], u[1], u[2]), b = max3f(u[3], u[4], u[5]);
    const float c = max3f(u[6], u[7], u[8]), d = max3f(u[9], u[10], u[11]);
    const float e = max3f(u[12], u[13], u[14]), f = max3f(u[15], v[0], v[1]);
    const float g = max3f(v[2], v[3], v[4]), h = max3f(v[5], v[6], v[7]);
    const float i = max3f(v[8], v[9], v[10]), k = max3f(v[11], v[12], v[13]);
    const float x = max3f(max3f(a, b, c), max3f(d, e, f), max3f(g, h, i));
    // finite: every page holds a visible key for every row
    const float mx = half_pair_max(max3f(x, k, fmaxf(v[14], v[15])));
    shift[j] = first ? mx : fmaxf(mx, 0.f);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-shift[j]);
      l[j] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][j][r] *= alpha;
        o[1][j][r] *= alpha;
      }
    }
    m[j] += shift[j];
  }
}

// VALU phase of page j: turn x into P (bf16) and add the row sums.  The max
// is not looked at unless some lane's sum over its 32 keys exceeds
// 2^kSumLimitLog2 (or is inf), or on a split's first page, where it starts
// from that page's row max; only then is it raised to the page max, O and l
// rescaled and P recomputed.  Every p is therefore at most 2^kSumLimitLog2,
// far from fp32 overflow in O and l, and since the max only grows from
// values that occurred, P keeps bf16's relative precision.
constexpr uint32_t kSumLimitBits = 0x47800000u;  // 2^16 as fp32 bits; inf and NaN compare above

// kSkipFirst: skip the pass at the old max on a first page, whose P would
// be discarded (the frame kernels, whose every item of a few pages starts
// with a first page; a split of the stream has one among dozens).
template <int NJ, bool kArgs = false, bool kSkipFirst = false>
__device__ __forceinline__ void valu_phase(f32x16 (&sc)[2][NJ], float (&m)[NJ], float (&l)[NJ],
                                           f32x16 (&o)[2][NJ], bf16x8 (&pf)[NJ][4], bool first, float c2 = 0.f) {
  if constexpr (kArgs) {  // the exponent arguments, when the MFMA phase left them
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][j][r] = __builtin_fmaf(sc[kt][j][r], c2, -m[j]);
  }
  float psum[NJ], shift[NJ];
  bool big = first;
  if (!kSkipFirst || !first) {
    page_exp<NJ, false>(sc, shift, pf, psum);
#pragma unroll
    for (int j = 0; j < NJ; ++j) big |= __builtin_bit_cast(uint32_t, psum[j]) > kSumLimitBits;
  }
  if (__any(big)) {
    raise_max<NJ>(sc, m, l, o, shift, first);
    page_exp<NJ, true>(sc, shift, pf, psum);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) l[j] += psum[j];
}

// VALU phase of the stream kernel when Q was multiplied by scale * log2 e
// before the QK^T product: a score is already in log2 units.  Every row's
// max starts at 0 and is left there while the split's first page gives each
// lane a sum (over its 32 keys) in [2^-20, 2^16] and no later page gives one
// above 2^16; the exponent argument is then the score itself.  Otherwise the
// max is raised as in valu_phase (on the first page: set to the page's row
// max), and from then on (`eng`, wave-uniform) the wave subtracts it from
// every score.  Every p stays at most 2^16 and, after the first page, every
// row sum at least 2^-20, so neither the sums overflow nor the rows that
// keep a zero max lose their weight to underflow.
constexpr uint32_t kSumFloorBits = 0x35800000u;  // 2^-20

template <int NJ>
__device__ __forceinline__ void valu_phase_qs(f32x16 (&sc)[2][NJ], float (&m)[NJ], float (&l)[NJ],
                                              f32x16 (&o)[2][NJ], bf16x8 (&pf)[NJ][4], bool first, bool& eng) {
  if (eng) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt][j][r] -= m[j];
  }
  float psum[NJ], shift[NJ];
  page_exp<NJ, false>(sc, shift, pf, psum);
  bool out = false;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t b = __builtin_bit_cast(uint32_t, psum[j]);
    out |= b > kSumLimitBits || (first && b < kSumFloorBits);
  }
  if (__any(out)) {
    raise_max<NJ>(sc, m, l, o, shift, first);
    page_exp<NJ, true>(sc, shift, pf, psum);
    eng = true;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) l[j] += psum[j];
}

// Copy rows r0 .. r0+7 of a 64-wide bf16 tile into LDS, swizzled (chunk c of
// row r at swz(r, c)): lane l takes source chunk (l & 7) ^ ((r >> 1) & 7) of
// row r0 + (l >> 3) into LDS position 8r + (l & 7); `src_row` gives the
// row's address (rows past the valid ones repeat a valid one).
template <class RowPtr>
__device__ __forceinline__ void copy_rows8(uint16_t* tile, int r0, int lane, RowPtr src_row) {
  const int r = r0 + (lane >> 3), pc = lane & 7;
  __builtin_amdgcn_global_load_lds(src_row(r) + ((pc ^ ((r >> 1) & 7)) << 3), tile + r0 * kHeadDim, 16, 0, 0);
}

// The same for a slot-major V tile (chunk c of row r at c ^ vswz(r), read
// back with the transposing LDS read at the offsets vrow_offset gives).
template <class RowPtr>
__device__ __forceinline__ void copy_vrows8(uint16_t* tile, int r0, int lane, RowPtr src_row) {
  const int r = r0 + (lane >> 3), pc = lane & 7;
  __builtin_amdgcn_global_load_lds(src_row(r) + ((pc ^ vswz(r)) << 3), tile + r0 * kHeadDim, 16, 0, 0);
}

// Issue the copy of physical page pg into ring slot `slot` (K and V tiles):
// lane l of wave w fetches the 16-byte chunk that belongs at LDS position
// 64w + l of the swizzled tile.
__device__ __forceinline__ void stage_page(const AttnArgs& a, uint16_t (&ring)[2 * kRing][kTileElems],
                                           int slot, int pg, int h, int tid) {
  const size_t off = ((size_t)pg * a.H + h) * (kPage * kHeadDim);
  // the wave index is uniform: as a scalar the LDS destinations stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row = wave * 8 + (lane >> 3), pc = lane & 7;
  const int src = row * 64 + ((pc ^ ((row >> 1) & 7)) << 3);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.kpool) + off + src;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.vpool) + off + src;
  __builtin_amdgcn_global_load_lds(kp, &ring[slot][wave * 512], 16, 0, 0);
  __builtin_amdgcn_global_load_lds(vp, &ring[kRing + slot][wave * 512], 16, 0, 0);
}

// Frame-mode copy of page j of the frame's own rows (valid slots `valid`)
// into ring slot `slot`: K as stage_page lays it out, V slot-major (vswz).
// Slots past the frame's last row repeat that row: their scores are masked,
// so they only need to be finite.
__device__ __forceinline__ void stage_frame_page(const AttnArgs& a, uint16_t (&ring)[2 * kRing][kTileElems],
                                                 int slot, int f, int j, int valid, int h, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row = wave * 8 + (lane >> 3), pc = lane & 7;
  const int r = row < valid ? row : valid - 1;
  const size_t base = ((size_t)(f * a.Lq + j * kPage + r) * a.H + h) * kHeadDim;
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k_in) + base + ((pc ^ ((row >> 1) & 7)) << 3);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v_in) + base + ((pc ^ vswz(row)) << 3);
  __builtin_amdgcn_global_load_lds(kp, &ring[slot][wave * 512], 16, 0, 0);
  __builtin_amdgcn_global_load_lds(vp, &ring[kRing + slot][wave * 512], 16, 0, 0);
}

// Copy of the 64 query rows of wave `wave` (rows 64 wave .. +63 of frame f,
// head h; rows past the frame repeat its last row) into that wave's own LDS
// tile, laid out as stage_page lays out K (chunk c of row r at c ^ ((r >> 1)
// & 7)): eight 1 KB copies.
__device__ __forceinline__ void stage_q_rows(const AttnArgs& a, uint16_t* tile, int f, int h, int wave, int lane) {
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  // (called inside the page loop: keep the per-lane addresses from being
  // hoisted out of it into registers)
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = i * 8 + (lane >> 3), pc = lane & 7;
    int row = wave * 64 + rr;
    row = row < a.Lq ? row : a.Lq - 1;
    const uint16_t* src = q + ((size_t)(f * a.Lq + row) * a.H + h) * kHeadDim + ((pc ^ ((rr >> 1) & 7)) << 3);
    __builtin_amdgcn_global_load_lds(src, tile + i * 512, 16, 0, 0);
  }
}

// MFMA phase of page j: QK^T of page j (K from slot sk), the empty slots of
// its scores masked, then PV of page j-1 (P from the previous VALU phase, V^T
// from slot sv) with, beside it, the scores turned in place into
// x = s * c2 - m (c2 = scale * log2 e): the VALU works while the matrix core
// does, and its work fills the waits on the V operand reads.
struct NoHook {
  __device__ void operator()() const {}
};

template <int NJ, bool kArgs = true, bool kVRow = false, class AfterV = NoHook>
__device__ __forceinline__ void mfma_phase(const uint16_t* sk, const uint16_t* sv, const bf16x8 (&qf)[NJ][4],
                                           const bf16x8 (&pf)[NJ][4], f32x16 (&o)[2][NJ], f32x16 (&sc)[2][NJ],
                                           const float (&m)[NJ], float c2, int valid, int l32, int hf,
                                           int vo0 = 0, int vo1 = 0, const AfterV& after_v = AfterV{}) {
  if (sk != nullptr) {
    const f32x16 zero = {};
    if constexpr (GCA_KPREFETCH) {
      // d-chunk outer, key tile inner: the two K fragments of chunk c + 1
      // are read right after the first of the four products of chunk c,
      // so each read lands behind three MFMAs, and no read is younger than
      // the ones the next wait is for
      auto kfrag = [&](int kt, int c) {
        return *reinterpret_cast<const bf16x8*>(&sk[swz(kt * 32 + l32, c * 2 + hf)]);
      };
      bf16x8 kb[2][2] = {{kfrag(0, 0), kfrag(1, 0)}, {}};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int u = 0; u < 2 * NJ; ++u) {
          const int kt = u / NJ, j = u % NJ;
          sc[kt][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c % 2][kt], qf[j][c], c == 0 ? zero : sc[kt][j], 0, 0, 0);
          // the scheduler would otherwise sink the reads next to their use
          // to save registers
          if (u == 0 && c + 1 < 4) {
            __builtin_amdgcn_sched_barrier(0);
            kb[(c + 1) % 2][0] = kfrag(0, c + 1);
            kb[(c + 1) % 2][1] = kfrag(1, c + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = kt * 32 + l32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sk[swz(row, c * 2 + hf)]);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            sc[kt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j][c], c == 0 ? zero : sc[kt][j], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (valid < kPage) mask_page<NJ>(sc, valid, hf);
  }
  __builtin_amdgcn_sched_barrier(0);
  // PV: V fragment i (kc = i / 2, dt = i % 2) is read two fragments ahead;
  // after each of its MFMAs come four of the 64 multiply-adds, and a
  // scheduling fence after each fragment keeps that order
  // (kVRow: V slot-major, read transposed at the offsets vrow_offset gives)
  auto vfrag = [&](int i) {
    if constexpr (kVRow) {
      const uint16_t* b = sv + ((i % 2) ? vo1 : vo0) + (i / 2) * 1024;
      const bf16x4 lo = lds_read_tr(b), hi = lds_read_tr(b + 512);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const bf16x8*>(&sv[swz((i % 2) * 32 + l32, (i / 2) * 2 + hf)]);
    }
  };
  bf16x8 vbuf[2] = {vfrag(0), vfrag(1)};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16x8 vf = vbuf[i % 2];
    if (i + 2 < 8) vbuf[i % 2] = vfrag(i + 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      o[i % 2][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j][i / 2], o[i % 2][j], 0, 0, 0);
      if (kArgs && sk != nullptr) {
        // multiply-adds 4u .. 4u+3 of the 64 (u = 2i + j): tile (u / 8, u / 4 % 2), registers 4(u % 4) ..
        const int u = 2 * i + j;
        const int kt = (u >> 3) & 1, jq = (u >> 2) & 1, r0 = (u & 3) * 4;
#pragma unroll
        for (int r = r0; r < r0 + 4; ++r) sc[kt][jq][r] = __builtin_fmaf(sc[kt][jq][r], c2, -m[jq]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // after_v runs once the last V fragment has been read (the transposing
    // reads wait for every copy in flight: what is issued after them has a
    // whole page to land)
    if (i == 5) after_v();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kArgs && sk != nullptr) {
    // keep the multiply-adds here: without a use the compiler would sink them
    // into the VALU phase
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(sc[kt][j]));
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Write the appended frame's pages that fall in [p0, p1) to their pool pages:
// K rows as they are, V rows transposed (through the ring slots) with slot s
// at column swap23(s); slots past the frame's last row are zero.  Up to eight
// pages go per round: all their rows are loaded first, so the round pays one
// memory latency.  Only this workgroup reads these pages back in this launch
// (workgroups of other query blocks with the same split write the same
// bytes), and wave w stores exactly the tile rows 8w .. 8w+7 that its own
// copies later fetch (see stage_page), so the stores need no fence: the
// copies of a wave issue after its stores, and the vector-memory counter the
// page loop waits on completes in order, so every store has completed before
// a copy issued after the next such wait.  The caller waits explicitly when
// a written page is staged before the loop's first wait.
constexpr int kFreshBatch = 8;

__device__ __forceinline__ void write_fresh_pages(const AttnArgs& a, uint16_t (&ring)[2 * kRing][kTileElems], int p0,
                                  int p1, int h, int tid) {
  static_assert(2 * kRing >= kFreshBatch, "one LDS tile per page of a round");
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt + a.pl.fresh_cnt;
  const int f0 = npg - a.pl.fresh_cnt;
  const int lo = p0 > f0 ? p0 : f0;
  if (lo >= p1) return;  // uniform
  const int H = a.H;
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(a.k_in);
  const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v_in);
  uint16_t* kpool = reinterpret_cast<uint16_t*>(a.kpool);
  uint16_t* vpool = reinterpret_cast<uint16_t*>(a.vpool);
  const int row = tid >> 3, ch = tid & 7;  // 512 threads: one 16-byte chunk of a 64x64 tile each
  const int col = swap23(row);
  for (int b0 = lo; b0 < p1; b0 += kFreshBatch) {
    uint4 kv[kFreshBatch], vv[kFreshBatch];
#pragma unroll
    for (int u = 0; u < kFreshBatch; ++u) {
      const int j = b0 + u - f0;
      const int valid = (j == a.pl.ppf - 1) ? a.pl.f_last_valid : kPage;
      kv[u] = make_uint4(0u, 0u, 0u, 0u);
      vv[u] = kv[u];
      if (b0 + u < p1 && row < valid) {
        const size_t src = ((size_t)(j * kPage + row) * H + h) * kHeadDim + ch * 8;
        kv[u] = *reinterpret_cast<const uint4*>(kin + src);
        vv[u] = *reinterpret_cast<const uint4*>(vin + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kFreshBatch; ++u) {
      if (b0 + u < p1) {
        const int j = b0 + u - f0;
        const int pg = fresh_page_ids()[j];
        const size_t off = ((size_t)pg * H + h) * (kPage * kHeadDim);
        const int valid = (j == a.pl.ppf - 1) ? a.pl.f_last_valid : kPage;
        if (a.rope != nullptr && row < valid)  // rotated keys are what the cache holds
          kv[u] = rope_bf16x8(kv[u], a.rope + (size_t)(j * kPage + row) * (kHeadDim / 2) + ch * 4);
        *reinterpret_cast<uint4*>(kpool + off + row * 64 + ch * 8) = kv[u];
        const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        // V^T element (d, col) sits at chunk (col >> 3) ^ (d >> 3) of row d:
        // the lanes of one store write rows d = 8ch + e, 1 KB apart, which
        // the XOR moves to eight different bank groups
#pragma unroll
        for (int e = 0; e < 8; ++e)
          ring[u][(ch * 8 + e) * 64 + (((col >> 3) ^ ch) << 3) + (col & 7)] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kFreshBatch; ++u) {
      if (b0 + u < p1) {
        const int pg = fresh_page_ids()[b0 + u - f0];
        const size_t off = ((size_t)pg * H + h) * (kPage * kHeadDim);
        *reinterpret_cast<uint4*>(vpool + off + row * 64 + ch * 8) =
            *reinterpret_cast<const uint4*>(&ring[u][row * 64 + ((ch ^ (row >> 3)) << 3)]);
      }
    }
    __syncthreads();  // the tiles are free again
  }
}

// f(jj + S, slot S) for S = S0 .. N-1 while jj + S < np, with S a constant:
// the ring loop is unrolled over its slots so every slot index is known.
template <int S0, int N, class F>
__device__ __forceinline__ void for_each_slot(int jj, int np, F& f) {
  if constexpr (S0 < N) {
    if (jj + S0 < np) f(jj + S0, std::integral_constant<int, S0>{});
    for_each_slot<S0 + 1, N>(jj, np, f);
  }
}

// Q^T fragments of a bf16 attention workgroup: tile j, d-chunk c: column
// q = 32j + l32, d = 16c + 8hf .. +7 (rotated when rotary angles are given;
// kScale: times scale * log2 e, rounded to bf16 once).
template <int NJ, bool kScale = false>
__device__ __forceinline__ void load_q(const AttnArgs& a, bf16x8 (&qf)[NJ][4], int h, int qb, int wave, int l32,
                                       int hf) {
  constexpr int D = kHeadDim;
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = qb * kQBlock + wave * 64 + j * 32 + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < a.Lq) {
        v = *reinterpret_cast<const uint4*>(qbase + ((size_t)row * a.H + h) * D + c * 16 + hf * 8);
        if (a.rope != nullptr)
          v = rope_bf16x8(v, a.rope + (size_t)row * (D / 2) + c * 8 + hf * 4, kScale ? a.scale_log2 : 1.f);
        else if (kScale)
          v = scale_bf16x8(v, a.scale_log2);
      }
      qf[j][c] = __builtin_bit_cast(bf16x8, v);
    }
  }
}

// Outputs of a bf16 attention workgroup: with one split, O / l rounded to
// bf16 and the LSE (natural log); otherwise the split's partial, O / l
// rounded to bf16 with (m, l) in fp32 (m in log2 units).  Each wave first
// writes its 64 rows into its own 8 KB LDS tile `stage` (16-byte chunk c of
// row r at chunk c ^ (r & 7)), then stores them as whole 128-byte rows, eight
// lanes per row: the register layout spreads a row over 32 lanes in 8-byte
// pieces, and storing that directly touches 32 rows per store instruction.
// The caller makes sure no other wave still reads or fills `stage`.
// What the epilogue of an attention workgroup writes to: final outputs
// (nsplit == 1) or the split partials.
struct EpiArgs {
  void* out;
  float* lse;
  void* part_o;
  float2* part_ml;
  int32_t H, Lq, Lq_pad, nsplit;
  __device__ explicit EpiArgs(const AttnArgs& a)
      : out(a.out), lse(a.lse), part_o(a.part_o), part_ml(a.part_ml), H(a.H), Lq(a.Lq), Lq_pad(a.Lq_pad),
        nsplit(a.nsplit) {}
  // outputs of frame f of a batched launch (bf16 rows)
  __device__ EpiArgs frame(size_t f) const {
    EpiArgs e = *this;
    e.out = static_cast<char*>(out) + f * (size_t)Lq * H * kHeadDim * 2;
    if (lse != nullptr) e.lse = lse + f * (size_t)H * Lq;
    return e;
  }
};

// kInLoop: called inside a page loop (the persistent frame mode), where
// only final outputs occur and the lane indices are passed through an empty
// asm so that the compiler does not hoist the per-lane addresses out of the
// loop into registers it then has to spill.
template <int NJ, bool kInLoop = false>
__device__ __forceinline__ void attn_epilogue(const EpiArgs& a, const f32x16 (&o)[2][NJ], const float (&m)[NJ],
                                              float (&l)[NJ], int h, int qb, int s, int wave, int l32, int hf,
                                              uint16_t* stage) {
  constexpr int D = kHeadDim;
  const int H = a.H;
  if constexpr (kInLoop) asm volatile("" : "+v"(l32), "+v"(hf));
#pragma unroll
  for (int j = 0; j < NJ; ++j) l[j] = half_pair_sum(l[j]);
  const bool final_out = kInLoop || a.nsplit == 1;
  const int row0 = qb * kQBlock + wave * 64;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int rr = j * 32 + l32;  // row of the wave's tile
    const float inv = 1.f / l[j];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // d = 32dt + 8g + 4hf .. +3: half hf of chunk 4dt + g
        const __bf16 b0v = (__bf16)(o[dt][j][4 * g + 0] * inv), b1v = (__bf16)(o[dt][j][4 * g + 1] * inv);
        const __bf16 b2v = (__bf16)(o[dt][j][4 * g + 2] * inv), b3v = (__bf16)(o[dt][j][4 * g + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0v) | ((uint32_t)__builtin_bit_cast(uint16_t, b1v) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2v) | ((uint32_t)__builtin_bit_cast(uint16_t, b3v) << 16);
        *reinterpret_cast<uint2*>(&stage[rr * 64 + (((4 * dt + g) ^ (rr & 7)) << 3) + 4 * hf]) = w;
      }
    const int row = row0 + rr;
    if (row < a.Lq && hf == 0) {
      if (final_out) {
        if (a.lse != nullptr) a.lse[(size_t)h * a.Lq + row] = m[j] * kLn2 + logf(l[j]);
      } else {
        a.part_ml[((size_t)h * a.nsplit + s) * a.Lq_pad + row] = make_float2(m[j], l[j]);
      }
    }
  }
  // the tile is this wave's alone: its own stores must land before its reads
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  const int c = l32 & 7;  // lane: 16-byte chunk c of row 8i + (lane >> 3)
#pragma unroll
  for (int i = 0; i < 64 / 8; ++i) {
    const int rr = i * 8 + ((hf * 32 + l32) >> 3);
    const int row = row0 + rr;
    const uint4 v = *reinterpret_cast<const uint4*>(&stage[rr * 64 + ((c ^ (rr & 7)) << 3)]);
    if (row < a.Lq) {
      uint16_t* dst = final_out
                          ? reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * H + h) * D
                          : reinterpret_cast<uint16_t*>(a.part_o) + (((size_t)h * a.nsplit + s) * a.Lq_pad + row) * D;
      *reinterpret_cast<uint4*>(dst + c * 8) = v;
    }
  }
}

// Arguments of frame f of a batched intra-frame launch: its rows, outputs,
// rotary angles and scratch pages follow those of the frames before it
// (identity for f == 0).
template <int kElemBytes>
__device__ __forceinline__ AttnArgs frame_of(const AttnArgs& in, size_t f) {
  AttnArgs a = in;
  const size_t rows = (size_t)in.Lq * in.H * kHeadDim * kElemBytes;
  const size_t pages = (size_t)in.pl.ppf * in.H * kPage * kHeadDim * kElemBytes;
  a.q = static_cast<const char*>(in.q) + f * rows;
  a.k_in = static_cast<const char*>(in.k_in) + f * rows;
  a.v_in = static_cast<const char*>(in.v_in) + f * rows;
  a.out = static_cast<char*>(in.out) + f * rows;
  a.kpool = static_cast<char*>(in.kpool) + f * pages;
  a.vpool = static_cast<char*>(in.vpool) + f * pages;
  if (in.lse != nullptr) a.lse = in.lse + f * in.H * in.Lq;
  if (in.rope != nullptr) a.rope = in.rope + f * in.Lq * (kHeadDim / 2);
  return a;
}

// Arguments of frame blockIdx.y (batched launches put frames on grid rows).
template <int kElemBytes>
__device__ __forceinline__ AttnArgs batch_frame(const AttnArgs& in) {
  return frame_of<kElemBytes>(in, blockIdx.y);
}

// kFrame: intra-frame attention of a batch of frames, one split, every page
// the frame's own rows (K and V staged from k_in / v_in, V slot-major and
// read transposed), no rotary angles and no cache bookkeeping.  kPersist
// (frame mode only): workgroups walk several (frame, head) items each, see
// below; otherwise one item per workgroup.
template <int NW, bool kFrame, bool kPersist = false>
__global__ __launch_bounds__(NW * 64) void k_attn_bf16(AttnArgs a_in) {
  const AttnArgs a = batch_frame<2>(a_in);
  static_assert(NW == 8, "the staging layout assumes 512 threads");
  constexpr int NJ = 2;
  constexpr int D = kHeadDim;
  constexpr bool kQS = GCA_QSCALE != 0 && !kFrame;  // Q pre-scaled, see valu_phase_qs
  // One LDS array holds the ring (tiles 0 .. 2*kRing-1) and the page list
  // (the tiles after it): with a single LDS object the compiler can tell the
  // ring slots apart and waits on the copies only where this code asks it to.
  // (the frame mode has no page list; its tiles after the ring hold each
  // wave's next query rows)
  constexpr int kListTiles = kListCap * 4 / (kTileElems * 2);
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kRing + (kPersist ? NW : kListTiles)][kTileElems];
  auto& ring = *reinterpret_cast<uint16_t(*)[2 * kRing][kTileElems]>(&lds[0][0]);
  uint32_t* plist = reinterpret_cast<uint32_t*>(&lds[2 * kRing][0]);  // the split's pages, see page_entry

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  PhaseClock pc;
  pc.start(a.clock != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && (wave == 0 || wave == 4));
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const unsigned long long cyc0 = __builtin_amdgcn_s_memtime(), ref0 = __builtin_amdgcn_s_memrealtime();
  const int H = a.H;
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt + a.pl.fresh_cnt;
  // Frame mode: workgroup w takes the (frame, head) items w, w + G, w + 2G,
  // ... (G workgroups; item i = frame i / H, head i % H; one query block per
  // frame).  Persistent (kPersist), it walks their pages as one list, item
  // after item, so the ring runs on across items: at each switch (see
  // switch_item) a wave loads the next item's query rows from its own LDS
  // tile and writes out the finished item through that tile, and one page
  // into the new item it starts copying the following item's rows there.
  const int nitems = kPersist ? (a.batch * H - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 1;
  int fcur = 0;  // frame of the item being walked (frame mode)
  if constexpr (kFrame) {
    fcur = (int)blockIdx.x / H;
    h = (int)blockIdx.x - fcur * H;
    qb = 0;
    s = 0;
  }
  const int p0 = kFrame ? 0 : split_begin(a, s);
  const int p1 = kFrame ? nitems * npg : split_begin(a, s + 1);
  if (!kFrame && a.pl.fresh_cnt > 0 && a.fresh_frame >= 0 && blockIdx.x == 0) record_fresh_frame(a);
  // The prologue issues its loads (the first list entries, Q, the appended
  // frame's rows) before it waits on any of them.
  // The split's pages are resolved once (p1 - p0 <= kListCap: the host picks
  // enough splits); the loop then reads page ids from LDS instead of walking
  // the page tables with scalar code.
  int valid0 = 0, raw0 = 0;
  if constexpr (!kFrame) raw0 = *page_source(a, p0 + tid < p1 ? p0 + tid : p1 - 1, valid0);

  bf16x8 qf[NJ][4];
  if constexpr (kFrame)
    load_q<NJ>(frame_of<2>(a, fcur), qf, h, qb, wave, l32, hf);
  else
    load_q<NJ, kQS>(a, qf, h, qb, wave, l32, hf);
  pc.lap(0);

  const int f0 = npg - a.pl.fresh_cnt;  // first page of the appended frame
  const int np = p1 - p0;                // >= 1: there are never more splits than pages
  if constexpr (!kFrame) {
    if (a.pl.fresh_cnt > 0) write_fresh_pages(a, ring, p0, p1, h, tid);
    if (p0 + tid < p1) plist[tid] = page_entry(a, raw0, valid0);
    for (int i = p0 + tid + NW * 64; i < p1; i += NW * 64) {
      int valid;
      const int raw = *page_source(a, i, valid);
      plist[i - p0] = page_entry(a, raw, valid);
    }
    __syncthreads();
  }
  pc.lap(1);
  // list entry (page id << 7 | valid slots) of split page i, clamped to the
  // last one (the ring is kept full past the end with copies of that page);
  // in the frame mode the page id is the frame's page index
  auto entry = [&](int i) -> uint32_t { return __builtin_amdgcn_readfirstlane(plist[i < np ? i : np - 1]); };
  // The frame mode's entries come from a generator instead, in list order
  // (the loop asks for them in that order), as frame << 22 | head << 10 |
  // page << 7 | valid slots, so that no page needs a division.  Items
  // advance by G = gridDim.x: head by G % H, frame by G / H, with a carry.
  const int ppf = a.pl.ppf;
  int g_c = 0, g_j = 0, g_f = fcur, g_h = h, dF = 0, dH = 0;
  if constexpr (kFrame) {
    dF = (int)gridDim.x / H;
    dH = (int)gridDim.x - dF * H;
  }
  auto gen = [&]() -> uint32_t {
    const uint32_t e = ((uint32_t)g_f << 22) | ((uint32_t)g_h << 10) | ((uint32_t)g_j << 7) |
                       (uint32_t)(g_j == ppf - 1 ? a.pl.f_last_valid : kPage);
    if (g_c + 1 < np) {  // past the end it keeps giving the last page
      ++g_c;
      if (++g_j == ppf) {
        g_j = 0;
        g_h += dH;
        g_f += dF;
        if (g_h >= H) {
          g_h -= H;
          ++g_f;
        }
      }
    }
    return e;
  };
  // frame and head of the workgroup's item k (frame mode; once per item)
  auto item_frame_head = [&](int k, int& f, int& hh) {
    const int it = (int)blockIdx.x + k * (int)gridDim.x;
    f = it / H;
    hh = it - f * H;
  };
  // staging of the page with list entry e into ring slot u
  auto stage = [&](int u, uint32_t e) {
    if constexpr (kFrame)
      stage_frame_page(a, ring, u, (int)(e >> 22), (int)((e >> 7) & 7u), (int)(e & 127u), (int)((e >> 10) & 4095u),
                       tid);
    else
      stage_page(a, ring, u, (int)(e >> 7), h, tid);
  };
  uint16_t* const qtile = kPersist ? &lds[2 * kRing + wave][0] : nullptr;  // this wave's next query rows
  int item = 0;                  // item being walked (frame mode)
  int item_start = 0;            // its first page
  int next_start = npg;          // the next item's first page
  const int vo0 = kFrame ? vrow_offset(0, lane) : 0, vo1 = kFrame ? vrow_offset(1, lane) : 0;

  f32x16 o[2][NJ];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
  float m[NJ], l[NJ];  // running max (log2 units; 0 until a split's first page sets it), row sum
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    m[j] = 0.f;
    l[j] = 0.f;
  }
  const float c2 = a.scale_log2;
  bool eng = false;  // some row of this wave has a nonzero max (kQS)

  // Ping-pong.  Every wave runs the same per-page sequence -- an MFMA phase
  // (QK^T of page j, then PV of page j-1 beside the exponent arguments of page
  // j), a barrier, a VALU phase (the rest of page j's softmax), a barrier --
  // but waves 4-7 (group B) start one barrier later than
  // waves 0-3 (group A).  The two groups share the SIMDs one to one, so while
  // one wave of a SIMD issues MFMAs the other works on the VALU.  Barriers
  // count arrivals, not code positions: in global phase 2j group A is in its
  // MFMA phase of page j and group B in its VALU phase of page j-1; in phase
  // 2j+1 the roles swap.  In its VALU phase of page j a wave issues its part of
  // the copy of page j+kAhead into the slot page j+kAhead-kRing left, and
  // before the next barrier it waits for its part of page j+2: B reads page
  // j+2 two phases after that barrier but A already one phase after it.
  const bool grp_a = GCA_PINGPONG ? wave < 4 : true;
  // prologue: pages p0 .. p0+kAhead-1 staged, p0 and p0+1 landed; a page
  // this workgroup has just written is only staged after its stores completed
  if (!kFrame && a.pl.fresh_cnt > 0 && f0 < p1 && f0 - p0 < kAhead) GCA_WAIT_VMCNT(0);
  // V tile of slot kRing-1 (read by the first page's MFMA phase) to zero; no
  // copy writes that slot before the first page's VALU phase
  static_assert(kTileElems * 2 == NW * 64 * 16, "one 16-byte store per thread clears a tile");
  *reinterpret_cast<uint4*>(&ring[2 * kRing - 1][tid * 8]) = make_uint4(0u, 0u, 0u, 0u);
  // ent[s]: list entry of the page in ring slot s, kept in scalar registers
  // from its staging on, so that no phase waits on an LDS read for it
  uint32_t ent[kRing];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) {
    ent[u] = kFrame ? gen() : entry(u);
    stage(u, ent[u]);
  }
  uint32_t ent_ahead = kFrame ? gen() : entry(kAhead);
  GCA_WAIT_VMCNT(2 * (kAhead - 2));
  wg_barrier();
  if (!grp_a) wg_barrier();  // group B runs one phase behind
  pc.lap(2);

  f32x16 sc[2][NJ];
  // the MFMA phase of the first page multiplies this zero P with the V tile
  // of ring slot kRing-1, which the prologue zeroed, so O stays zero
  bf16x8 pf[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[j][kc][e] = (__bf16)0.f;
  // Frame mode, the switch to the workgroup's next item, whose first page is
  // `first`: the finished item's last PV (P of the page before `first`, V
  // tile `sv`), its output (through this wave's tile, free once the new
  // item's query rows have been read from it), then zero O, l, max and P
  // (the new item's first exponent arguments start from a zero max, as on
  // a workgroup's first page, and the PV of that page's MFMA phase
  // multiplies the zero P).
  auto switch_item = [&](const uint16_t* sv, int first) __attribute__((always_inline)) {
    // the query rows, copied on the finished item's second page: the page
    // copies issued after them (two on each of its later pages but this one)
    // may stay in flight (the counter completes loads in order)
    switch (npg) {
      case 3: GCA_WAIT_VMCNT(2); break;
      case 4: GCA_WAIT_VMCNT(4); break;
      case 5: GCA_WAIT_VMCNT(6); break;
      case 6: GCA_WAIT_VMCNT(8); break;
      case 7: GCA_WAIT_VMCNT(10); break;
      case 8: GCA_WAIT_VMCNT(12); break;
      default: GCA_WAIT_VMCNT(0); break;
    }
    int lq = l32, hq = hf;  // addresses computed here, not held across the loop
    asm volatile("" : "+v"(lq), "+v"(hq));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        qf[j][c] = *reinterpret_cast<const bf16x8*>(&qtile[swz(j * 32 + lq, c * 2 + hq)]);
    mfma_phase<NJ, true, true>(nullptr, sv, qf, pf, o, sc, m, c2, kPage, l32, hf, vo0, vo1);
    int f, hh;
    item_frame_head(item, f, hh);
    attn_epilogue<NJ, true>(EpiArgs(a).frame(f), o, m, l, hh, 0, 0, wave, l32, hf, qtile);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      m[j] = 0.f;
      l[j] = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[j][kc][e] = (__bf16)0.f;
    }
    item += 1;
    item_start = first;
    next_start = first + npg;
  };
  // the page loop; kA: this wave computes its exponent arguments in its
  // softmax phase (group A of the asymmetric variant), else beside its MFMAs.
  // The two kinds of wave run separate copies of the loop.
  auto run_pages = [&](auto asym_c) {
    constexpr bool kA = decltype(asym_c)::value;
    auto page_step = [&](int jj, auto slot_c) {
      constexpr int S = decltype(slot_c)::value;  // ring slot of page p0 + jj
      constexpr int SA = (S + kAhead) % kRing;    // slot page p0 + jj + kAhead goes to
      // the entry after that one is read before the MFMA phase's own LDS reads,
      // so it has landed by the time it is used
      const uint32_t raw_next = kFrame ? gen() : plist[jj + kAhead + 1 < np ? jj + kAhead + 1 : np - 1];
      // frame mode: the first page of an item after the first.  Group A
      // switches items at the start of that page (its MFMA phase), group B
      // at the end of the page before (its softmax phase, the same global
      // phase), so the two switches overlap.
      const bool new_item = kPersist && jj == next_start;
      if (__builtin_expect(kPersist && new_item && grp_a, 0)) switch_item(ring[kRing + (S + kRing - 1) % kRing], jj);
      // the copy of the next item's query rows, one page after a boundary
      const bool q_copy = kPersist && jj == item_start + 1 && item + 1 < nitems;
      // the frame mode stages page jj + kAhead in this MFMA phase, after its
      // V reads, into the slot of page jj - 2, which both groups have read
      // by now (group A in its MFMA phase of page jj - 1, group B one phase
      // later, before group A's MFMA phase of page jj)
      auto stage_ahead = [&]() {
        ent[SA] = ent_ahead;
        stage(SA, ent_ahead);
        ent_ahead = __builtin_amdgcn_readfirstlane(raw_next);
        if constexpr (kPersist) {
          if (__builtin_expect(q_copy, 0)) {
            int f, hh;
            item_frame_head(item + 1, f, hh);
            stage_q_rows(a, qtile, f, hh, wave, lane);
          }
        }
      };
      if constexpr (kFrame)
        mfma_phase<NJ, !kA, true>(ring[S], ring[kRing + (S + kRing - 1) % kRing], qf, pf, o, sc, m, c2,
                                  (int)(ent[S] & 127u), l32, hf, vo0, vo1, stage_ahead);
      else if constexpr (GCA_STAGE_MFMA != 0)
        mfma_phase<NJ, !kA && !kQS, false>(ring[S], ring[kRing + (S + kRing - 1) % kRing], qf, pf, o, sc, m, c2,
                                           (int)(ent[S] & 127u), l32, hf, 0, 0, stage_ahead);
      else
        mfma_phase<NJ, !kA && !kQS>(ring[S], ring[kRing + (S + kRing - 1) % kRing], qf, pf, o, sc, m, c2,
                                    (int)(ent[S] & 127u), l32, hf);
      pc.lap(3);
      if (GCA_PINGPONG) wg_barrier();
      pc.lap(5);
      if constexpr (!kFrame && GCA_STAGE_MFMA == 0) stage_ahead();
      if constexpr (kQS)
        valu_phase_qs<NJ>(sc, m, l, o, pf, jj == item_start, eng);
      else
        valu_phase<NJ, kA, kFrame>(sc, m, l, o, pf, jj == item_start, c2);
      if (__builtin_expect(kPersist && !grp_a && jj + 1 == next_start && item + 1 < nitems, 0))
        switch_item(ring[kRing + S], jj + 1);
      pc.lap(4);
      // this wave's part of page j+2 has landed (in the frame mode the eight
      // copies of query rows issued on page j or j-1 come after it as well)
      if (kPersist && (jj == item_start + 1 || jj == item_start + 2) && item + 1 < nitems)
        GCA_WAIT_VMCNT(2 * (kAhead - 2) + 8);
      else
        GCA_WAIT_VMCNT(2 * (kAhead - 2));
      wg_barrier();
      pc.lap(5);
    };
    for (int jj = 0; jj < np; jj += kRing) for_each_slot<0, kRing>(jj, np, page_step);
  };
  if (kAsymArgs && !kQS && grp_a)
    run_pages(std::true_type{});
  else
    run_pages(std::false_type{});
  // PV of the last page; group A then takes the barrier that group B took
  // first, so both have passed the same number
  mfma_phase<NJ, true, kFrame>(nullptr, ring[kRing + (np - 1) % kRing], qf, pf, o, sc, m, c2, kPage, l32, hf,
                               vo0, vo1);
  if (GCA_PINGPONG && grp_a) wg_barrier();
  GCA_WAIT_VMCNT(0);  // no copy into LDS outlives the workgroup
  __syncthreads();    // every wave's copies have landed and its last PV has read the ring

  if constexpr (kFrame) {
    int f, hh;
    item_frame_head(item, f, hh);
    attn_epilogue<NJ>(EpiArgs(a).frame(f), o, m, l, hh, 0, 0, wave, l32, hf, &ring[wave][0]);
  } else {
    attn_epilogue<NJ>(EpiArgs(a), o, m, l, h, qb, s, wave, l32, hf, &ring[wave][0]);
  }
  if (a.clock != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    atomicAdd(&a.clock[0], __builtin_amdgcn_s_memtime() - cyc0);
    atomicAdd(&a.clock[1], __builtin_amdgcn_s_memrealtime() - ref0);
  }
  if constexpr (kPhaseTiming) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the output stores have completed
    pc.lap(6);
    pc.flush(a.clock, wave >= 4, np, lane == 0);
  }
}

// Intra-frame attention of one (frame, head) per workgroup, the frame at most
// kFrameTiles pages long (the calls with rotary angles; the others run in the
// frame mode of k_attn_bf16): its rotated K tiles are built once in LDS from
// the input rows and its V pages copied there slot-major, so the page loop
// reads no memory.  The loop is the ping-pong of the stream kernel without the
// copies.  Launches batch frames on grid rows and run one split (final
// outputs).

__global__ __launch_bounds__(kAttnWaves * 64) void k_frame_attn_bf16(AttnArgs a_in) {
  const AttnArgs a = batch_frame<2>(a_in);
  constexpr int NJ = 2;
  // tiles 0 .. ppf-1: K; kFrameTiles .. kFrameTiles+ppf-1: V^T; the last: zero
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kFrameTiles + 1][kTileElems];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const unsigned long long cyc0 = __builtin_amdgcn_s_memtime(), ref0 = __builtin_amdgcn_s_memrealtime();
  const int ppf = a.pl.ppf;  // <= kFrameTiles (checked at launch)
  const int p0 = 0, np = ppf;  // one split: every page of the frame
  bf16x8 qf[NJ][4];

  // K row r, chunk c of page j at swz(r, c) of tile j (rotated, empty slots
  // zero); V slot-major in tile kFrameTiles + j (chunk c of slot r at
  // c ^ vswz(r); slots past the frame repeat its last row, where P is 0),
  // copied straight into LDS by wave j and read with the transposing read
  {
    const uint16_t* kin = reinterpret_cast<const uint16_t*>(a.k_in);
    const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v_in);
    const int row = tid >> 3, ch = tid & 7;  // K: one 16-byte chunk of each tile per thread
    // Every load of the prologue is issued before any is used, and without
    // branches, so that the rotations wait for the loads they need and not
    // for the V copies issued last: query rows past the frame, pages past the
    // frame's and rows past a page's valid ones read the last row, and waves
    // past the frame's pages copy its last page into their V tile, which is
    // never read.  The Q fragments are the ones load_q reads.
    uint4 qv[NJ][4];
    float2 qcs[NJ][4][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int qrow = min(qb * kQBlock + wave * 64 + j * 32 + l32, a.Lq - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        qv[j][c] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                   ((size_t)qrow * a.H + h) * kHeadDim + c * 16 + hf * 8);
    }
    if (a.rope != nullptr) {  // uniform
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int qrow = min(qb * kQBlock + wave * 64 + j * 32 + l32, a.Lq - 1);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) qcs[j][c][e] = a.rope[(size_t)qrow * (kHeadDim / 2) + c * 8 + hf * 4 + e];
      }
    }
    uint4 kv[kFrameTiles];
    float2 cs[kFrameTiles][4];
#pragma unroll
    for (int j = 0; j < kFrameTiles; ++j) {
      const int pj = min(p0 + j, ppf - 1);
      const int valid = (pj == ppf - 1) ? a.pl.f_last_valid : kPage;
      kv[j] = *reinterpret_cast<const uint4*>(kin + ((size_t)(pj * kPage + min(row, valid - 1)) * a.H + h) * kHeadDim + ch * 8);
    }
    if (a.rope != nullptr) {  // uniform
#pragma unroll
      for (int j = 0; j < kFrameTiles; ++j) {
        const int pj = min(p0 + j, ppf - 1);
        const int valid = (pj == ppf - 1) ? a.pl.f_last_valid : kPage;
        const float2* t = a.rope + (size_t)(pj * kPage + min(row, valid - 1)) * (kHeadDim / 2) + ch * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[j][e] = t[e];
      }
    }
    {
      const int vpj = min(p0 + wave, ppf - 1);
      const int vvalid = (vpj == ppf - 1) ? a.pl.f_last_valid : kPage;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        copy_vrows8(&lds[kFrameTiles + wave][0], i * 8, lane, [&](int r) {
          return vin + ((size_t)(vpj * kPage + min(r, vvalid - 1)) * a.H + h) * kHeadDim;
        });
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool in = qb * kQBlock + wave * 64 + j * 32 + l32 < a.Lq;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (in) v = a.rope != nullptr ? rope_bf16x8(qv[j][c], qcs[j][c]) : qv[j][c];
        qf[j][c] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int j = 0; j < kFrameTiles; ++j) {
      if (j < np) {
        const int pj = p0 + j;
        const int valid = (pj == ppf - 1) ? a.pl.f_last_valid : kPage;
        if (row >= valid)
          kv[j] = make_uint4(0u, 0u, 0u, 0u);
        else if (a.rope != nullptr)
          kv[j] = rope_bf16x8(kv[j], cs[j]);
        *reinterpret_cast<uint4*>(&lds[j][swz(row, ch)]) = kv[j];
      }
    }
    static_assert(kTileElems * 2 == kAttnWaves * 64 * 16, "one 16-byte store per thread clears a tile");
    *reinterpret_cast<uint4*>(&lds[2 * kFrameTiles][tid * 8]) = make_uint4(0u, 0u, 0u, 0u);
  }
  GCA_WAIT_VMCNT(0);  // this wave's V copies have landed
  __syncthreads();
  const int vo0 = vrow_offset(0, lane), vo1 = vrow_offset(1, lane);

  f32x16 o[2][NJ];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
  float m[NJ], l[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    m[j] = 0.f;
    l[j] = 0.f;
  }
  const float c2 = a.scale_log2;
  f32x16 sc[2][NJ];
  bf16x8 pf[NJ][4];  // zero P meets the zero V tile on the first page
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[j][kc][e] = (__bf16)0.f;
  const bool grp_a = wave < 4;  // ping-pong as in k_attn_bf16
  if (!grp_a) wg_barrier();
  for (int jj = 0; jj < np; ++jj) {
    const int valid = (p0 + jj == ppf - 1) ? a.pl.f_last_valid : kPage;
    mfma_phase<NJ, true, true>(lds[jj], lds[jj == 0 ? 2 * kFrameTiles : kFrameTiles + jj - 1], qf, pf, o, sc, m, c2,
                               valid, l32, hf, vo0, vo1);
    wg_barrier();
    valu_phase<NJ, false, true>(sc, m, l, o, pf, jj == 0);
    wg_barrier();
  }
  mfma_phase<NJ, true, true>(nullptr, lds[kFrameTiles + np - 1], qf, pf, o, sc, m, c2, kPage, l32, hf, vo0, vo1);
  if (grp_a) wg_barrier();
  __syncthreads();  // every wave's last PV has read the tiles

  attn_epilogue<NJ>(EpiArgs(a), o, m, l, h, qb, s, wave, l32, hf, &lds[wave][0]);
  if (a.clock != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    atomicAdd(&a.clock[0], __builtin_amdgcn_s_memtime() - cyc0);
    atomicAdd(&a.clock[1], __builtin_amdgcn_s_memrealtime() - ref0);
  }
}

// Intra-frame attention with the keys split over the waves of a workgroup:
// one workgroup per (frame, head, 32-row query block), wave w takes page w
// of the frame (keys 64w .. 64w+63).  The Q block and each wave's K page are
// copied into swizzled LDS tiles with full-row (coalesced) copies; each wave
// copies its V page slot-major into an LDS tile of its own and reads it with
// the transposing LDS read (GCA_WS_VROW=0: transposes it through registers
// instead), then computes its page's scores, their softmax against its own
// row max and the PV product.  The V copies are issued last and waited for
// only before the PV product.  The waves' (m, l, O) are combined in LDS in fp32.
// kRope: the calls with rotary angles (Q and K rotated as their fragments
// are read from LDS).  Nothing passes through
// memory between these steps and there is no merge launch, so a lone frame
// costs one short launch: the latency-bound case (one frame per call) that
// the page-pipelined frame kernel, built for many frames, does not serve well.
constexpr int kWsRows = 32;           // query rows per workgroup
constexpr int kWsPad = kHeadDim + 4;  // padded row of the O exchange: rows fall on different banks
static_assert(kFrameTiles == kAttnWaves, "one page of the frame per wave");
// LDS: Q tile (32 rows), then each wave's K tile and V^T tile; after the PV
// products the O exchange reuses the space from the start
constexpr int kWsQElems = kWsRows * kHeadDim;
constexpr int kWsTilesBytes = (kWsQElems + 2 * kAttnWaves * kTileElems) * 2;
constexpr int kWsExBytes = kAttnWaves * kWsRows * kWsPad * 4;
static_assert(kWsExBytes <= kWsTilesBytes, "the O exchange fits in the tiles' space");


template <bool kRope>
__global__ __launch_bounds__(kAttnWaves * 64) void k_frame_wsplit_bf16(AttnArgs a_in) {
  const AttnArgs a = batch_frame<2>(a_in);
  constexpr int D = kHeadDim;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kWsTilesBytes];
  __shared__ float2 mlx[kAttnWaves][kWsRows];  // each wave's (m, l) per query row
  uint16_t* qt = reinterpret_cast<uint16_t*>(lds_raw);
  auto kt_of = [&](int w) { return qt + kWsQElems + w * kTileElems; };
  auto vt_of = [&](int w) { return qt + kWsQElems + (kAttnWaves + w) * kTileElems; };
  auto ox = reinterpret_cast<float(*)[kWsRows][kWsPad]>(lds_raw);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  const int qbs = (a.Lq + kWsRows - 1) / kWsRows;
  const int h = blockIdx.x / qbs, qb = blockIdx.x - h * qbs;
  const unsigned long long cyc0 = __builtin_amdgcn_s_memtime(), ref0 = __builtin_amdgcn_s_memrealtime();
  const int H = a.H, ppf = a.pl.ppf;  // ppf <= kAttnWaves (checked at launch)
  // valid keys of this wave's page (0: the frame has fewer pages than waves)
  const int valid = wave < ppf ? (wave == ppf - 1 ? a.pl.f_last_valid : kPage) : 0;
  const int key0 = wave * kPage;
  const uint16_t* qin = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(a.k_in);
  const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v_in);

  // copies: waves 0-3 each take 8 rows of the Q block (rows past the frame
  // repeat its last row; their outputs are not stored), every wave with keys
  // its K page (rows past the valid ones repeat the last valid row: their
  // scores are masked)
  uint4 vr[8];
  const int cg = lane >> 3, ch = lane & 7;
  if (valid > 0 && GCA_WS_VROW) {  // uniform; rows past the valid ones repeat the last (P is 0 there)
    // K first, then the Q block, then V: QK^T and the softmax start once
    // the first two have landed, while V is still on its way
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy_rows8(kt_of(wave), i * 8, lane, [&](int r) {
        return kin + ((size_t)(key0 + min(r, valid - 1)) * H + h) * D;
      });
  }
  if (wave < kWsRows / 8)
    copy_rows8(qt, wave * 8, lane, [&](int r) {
      const int row = min(qb * kWsRows + r, a.Lq - 1);
      return qin + ((size_t)row * H + h) * D;
    });
  if (valid > 0 && GCA_WS_VROW) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy_vrows8(vt_of(wave), i * 8, lane, [&](int r) {
        return vin + ((size_t)(key0 + min(r, valid - 1)) * H + h) * D;
      });
  } else if (valid > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy_rows8(kt_of(wave), i * 8, lane, [&](int r) {
        return kin + ((size_t)(key0 + min(r, valid - 1)) * H + h) * D;
      });
    // V rows for the transposition: lane (cg, ch) fills V^T chunk cg
    // (columns 8cg .. 8cg+7) of rows d = 8ch .. 8ch+7.  Column 8cg + i holds
    // key swap23(8cg + i) = 16(cg >> 1) + 8(i >> 2) + 4(cg & 1) + i % 4, whose
    // 16-byte chunk ch of V it loads; keys past the valid ones are zero.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 16 * (cg >> 1) + 8 * (i >> 2) + 4 * (cg & 1) + (i & 3);
      vr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (key < valid) vr[i] = *reinterpret_cast<const uint4*>(vin + ((size_t)(key0 + key) * H + h) * D + ch * 8);
    }
    // V^T element (d, col), col = swap23(key), at swz(d, col / 8) + col % 8 as
    // in the pool: one 16-byte store per row d, word w = loads 2w and 2w+1
    uint16_t* vt = vt_of(wave);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wd[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = (&vr[2 * w].x)[e >> 1], x1 = (&vr[2 * w + 1].x)[e >> 1];
        wd[w] = (e & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      }
      *reinterpret_cast<uint4*>(&vt[swz(ch * 8 + e, cg)]) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }
  if (GCA_WS_VROW && valid > 0)
    GCA_WAIT_VMCNT(8);  // this wave's K and Q copies have landed (its eight V copies may not)
  else
    GCA_WAIT_VMCNT(0);  // this wave's copies have landed
  // and every wave's: the Q tile comes from waves 0-3.  Before this point
  // only copies write the LDS (with GCA_WS_VROW), so the barrier needs no
  // fence, whose wait would also hold the V copies
  if constexpr (GCA_WS_VROW != 0)
    wg_barrier();
  else
    __syncthreads();

  // Q^T fragments: query row qb*32 + l32, d = 16c + 8hf .. +7 (the angles
  // are loaded here, where they are used: loading them with the copies
  // measured 10 % slower)
  const int qrow = qb * kWsRows + l32;
  bf16x8 qf[1][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = *reinterpret_cast<const uint4*>(&qt[swz(l32, c * 2 + hf)]);
    if (kRope && qrow < a.Lq) v = rope_bf16x8(v, a.rope + (size_t)qrow * (D / 2) + c * 8 + hf * 4);
    qf[0][c] = __builtin_bit_cast(bf16x8, v);
  }

  float mrow = -INFINITY, lrow = 0.f;  // this wave's row max (log2 units) and row sum for query l32
  f32x16 o[2][1];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][0][r] = 0.f;
  if (valid > 0) {  // uniform
    const uint16_t* kt_ = kt_of(wave);
    f32x16 sc[2][1];
    const f32x16 zero = {};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // K fragment: key 32kt + l32 of the page, d = 16c + 8hf .. +7
        const int key = kt * 32 + l32;
        uint4 kv = *reinterpret_cast<const uint4*>(&kt_[swz(key, c * 2 + hf)]);
        if (kRope && key < valid) kv = rope_bf16x8(kv, a.rope + (size_t)(key0 + key) * (D / 2) + c * 8 + hf * 4);
        sc[kt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qf[0][c],
                                                            c == 0 ? zero : sc[kt][0], 0, 0, 0);
      }
    if (valid < kPage) mask_page<1>(sc, valid, hf);
    // row max of the page (key 0 is always valid), then P = exp2(s c2 - m)
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt][0][r]);
    mrow = half_pair_max(mx) * a.scale_log2;
    bf16x8 pf[1][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pf[0][kt * 2 + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][0][r], a.scale_log2, -mrow));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float acc = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pf[0][kc][e], pf[0][kc][e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
      }
    lrow = half_pair_sum(acc);
    // O^T += V^T P^T: fragment i is d-tile i % 2, 16-key chunk i / 2
    const uint16_t* vt = vt_of(wave);
    const int vo[2] = {vrow_offset(0, lane), vrow_offset(1, lane)};
    GCA_WAIT_VMCNT(0);  // this wave's V copies (read by this wave only)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x8 vf;
      if constexpr (GCA_WS_VROW != 0) {
        const uint16_t* b = vt + vo[i % 2] + (i / 2) * 1024;
        vf = __builtin_shufflevector(lds_read_tr(b), lds_read_tr(b + 512), 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        vf = *reinterpret_cast<const bf16x8*>(&vt[swz((i % 2) * 32 + l32, (i / 2) * 2 + hf)]);
      }
      o[i % 2][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[0][i / 2], o[i % 2][0], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the tiles: the exchange reuses them
  // exchange: register r of d-tile dt holds d = 32dt + 8(r/4) + 4hf + r%4 of query l32
  if (hf == 0) mlx[wave][l32] = make_float2(mrow, lrow);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&ox[wave][l32][dt * 32 + 8 * g + 4 * hf]) =
          make_float4(o[dt][0][4 * g], o[dt][0][4 * g + 1], o[dt][0][4 * g + 2], o[dt][0][4 * g + 3]);
  __syncthreads();
  // combine: thread t finishes query q = t / 16, d = 4 (t % 16) .. +3
  const int q = tid >> 4, d4 = (tid & 15) * 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, mlx[w][q].x);
  float L = 0.f, r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    const float2 e = mlx[w][q];
    const float sw = __builtin_amdgcn_exp2f(e.x - M);  // 0 for a wave without keys (m = -inf)
    const float4 v = *reinterpret_cast<const float4*>(&ox[w][q][d4]);
    L += sw * e.y;
    r0 += sw * v.x;
    r1 += sw * v.y;
    r2 += sw * v.z;
    r3 += sw * v.w;
  }
  const int row = qb * kWsRows + q;
  if (row < a.Lq) {
    const float inv = 1.f / L;
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r0 * inv)) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r1 * inv)) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r2 * inv)) |
          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r3 * inv)) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * H + h) * D + d4) = w;
    if (a.lse != nullptr && (tid & 15) == 0) a.lse[(size_t)h * a.Lq + row] = M * kLn2 + logf(L);
  }
  if (a.clock != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    atomicAdd(&a.clock[0], __builtin_amdgcn_s_memtime() - cyc0);
    atomicAdd(&a.clock[1], __builtin_amdgcn_s_memrealtime() - ref0);
  }
}

// fp32 attention on the matrix cores (v_mfma_f32_32x32x2_f32): one workgroup
// = (head, 256 query rows, one key split), 4 waves; wave w owns query rows
// [64w, 64w+64) of the block as two 32-row tiles j.  Per 64-slot page:
//   S^T[key][q] = K Q^T   A = K (LDS), B = Q^T (registers); step i of the 32
//                         contracts d = i in lane half 0 and d = 32 + i in
//                         lane half 1
//   exact online softmax per query column: the page's row max, then
//                         p = exp2((s - m) * scale * log2 e) in fp32
//   O^T[d][q] += V^T P^T  A = V^T (LDS), B = P^T: step r of a 32-key tile
//                         contracts the two keys register r of the S^T
//                         accumulator holds in the two lane halves (keys
//                         8(r/4) + 4h + r%4), so P^T comes straight from that
//                         register; the V^T columns are in the pool's swap23
//                         order, which puts a lane's four keys of register
//                         group r/4 in one 16-byte chunk
// Operand layout of the 32x32x2 MFMA: A lane l holds row l%32, k = l/32; B
// lane l holds column l%32, same k; accumulator as in k_attn_bf16.
// Tiles are fp32 [64][64] with 16-byte chunk c of row r at chunk c ^ (r & 15),
// so reads of one chunk column by 16 lanes of different rows hit 16 different
// bank groups.  Two page slots: page j+1 is copied into LDS with
// global_load_lds while page j is computed.  Pages of the appended frame are
// built from the input rows instead (keys rotated when rotary angles are
// given, values transposed) and written to their pool pages by the
// workgroups of query block 0.
constexpr int kF32Waves = kF32Rows / 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// float index of 16-byte chunk c of row r in a swizzled fp32 64x64 tile
__device__ __forceinline__ int swz32(int r, int c) { return r * 64 + ((c ^ (r & 15)) << 2); }

// Copy one fp32 64x64 tile (16 KB) from memory into a swizzled LDS tile:
// instruction u of wave w moves rows 4(4w + u) .. +3, lane l fetching the
// source chunk that belongs at LDS chunk position l & 15 of row l >> 4.
__device__ __forceinline__ void copy_tile_f32(const float* src, float* tile, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r0 = (wave * 4 + u) * 4;
    const int r = r0 + (lane >> 4), pc = lane & 15;
    __builtin_amdgcn_global_load_lds(src + r * 64 + ((pc ^ (r & 15)) << 2), tile + r0 * 64, 16, 0, 0);
  }
}

// Tiles of page fj of the appended frame from the input rows (all 256
// threads): K rows (rotated when rotary angles are given), V transposed into
// columns swap23(slot); slots past `valid` are zero.
__device__ __forceinline__ void build_fresh_f32(const AttnArgs& a, float* kt, float* vt, int fj, int valid, int h,
                                                int tid) {
  constexpr int D = kHeadDim;
  const float* kin = reinterpret_cast<const float*>(a.k_in);
  const float* vin = reinterpret_cast<const float*>(a.v_in);
  for (int e = tid; e < kPage * D / 4; e += kF32Rows) {
    const int r = e >> 4, c = e & 15;  // slot r, channels 4c .. 4c+3
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (r < valid) {
      const size_t row = (size_t)fj * kPage + r;
      const size_t src = (row * a.H + h) * D + 4 * c;
      kv = *reinterpret_cast<const float4*>(kin + src);
      vv = *reinterpret_cast<const float4*>(vin + src);
      if (a.rope != nullptr) {
        rope_rotate(kv.x, kv.y, a.rope[row * (D / 2) + 2 * c]);
        rope_rotate(kv.z, kv.w, a.rope[row * (D / 2) + 2 * c + 1]);
      }
    }
    *reinterpret_cast<float4*>(&kt[swz32(r, c)]) = kv;
    const int col = swap23(r);
    vt[swz32(4 * c + 0, col >> 2) + (col & 3)] = vv.x;
    vt[swz32(4 * c + 1, col >> 2) + (col & 3)] = vv.y;
    vt[swz32(4 * c + 2, col >> 2) + (col & 3)] = vv.z;
    vt[swz32(4 * c + 3, col >> 2) + (col & 3)] = vv.w;
  }
}

// The built tiles of an appended-frame page into its pool page (the caller
// has synchronised the workgroup after building them).
__device__ __forceinline__ void store_fresh_f32(const AttnArgs& a, const float* kt, const float* vt, int pg, int h,
                                                int tid) {
  const size_t off = ((size_t)pg * a.H + h) * (kPage * kHeadDim);
  float* kpool = reinterpret_cast<float*>(a.kpool) + off;
  float* vpool = reinterpret_cast<float*>(a.vpool) + off;
  for (int e = tid; e < kPage * kHeadDim / 4; e += kF32Rows) {
    const int r = e >> 4, c = e & 15;
    *reinterpret_cast<float4*>(kpool + r * 64 + 4 * c) = *reinterpret_cast<const float4*>(&kt[swz32(r, c)]);
    *reinterpret_cast<float4*>(vpool + r * 64 + 4 * c) = *reinterpret_cast<const float4*>(&vt[swz32(r, c)]);
  }
}

__global__ __launch_bounds__(kF32Rows) void k_attn_f32(AttnArgs a_in) {
  const AttnArgs a = batch_frame<4>(a_in);
  constexpr int D = kHeadDim, NJ = 2;
  // two page slots, each a K tile and a V^T tile
  __shared__ __attribute__((aligned(16))) float lds[2][2][64 * 64];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const int H = a.H;
  const int p0 = split_begin(a, s);
  const int p1 = split_begin(a, s + 1);
  const int np = p1 - p0;  // >= 1
  if (a.pl.fresh_cnt > 0 && a.fresh_frame >= 0 && blockIdx.x == 0) record_fresh_frame(a);

  // Q^T fragments: qf[j][i] = Q[row 32j + l32 of the wave][32hf + i]
  float qf[NJ][32];
  const float* qin = reinterpret_cast<const float*>(a.q);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = qb * kF32Rows + wave * 64 + j * 32 + l32;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < a.Lq) {
        v = *reinterpret_cast<const float4*>(qin + ((size_t)row * H + h) * D + 32 * hf + 4 * u);
        if (a.rope != nullptr) {
          const float2* cs = a.rope + (size_t)row * (D / 2) + 16 * hf + 2 * u;
          rope_rotate(v.x, v.y, cs[0]);
          rope_rotate(v.z, v.w, cs[1]);
        }
      }
      qf[j][4 * u + 0] = v.x;
      qf[j][4 * u + 1] = v.y;
      qf[j][4 * u + 2] = v.z;
      qf[j][4 * u + 3] = v.w;
    }
  }

  f32x16 o[2][NJ];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
  float m[NJ], l[NJ];  // running row max (raw score units) and this lane's share of the row sum
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
  }
  const float c2 = a.scale_log2;
  const float* kpool = reinterpret_cast<const float*>(a.kpool);
  const float* vpool = reinterpret_cast<const float*>(a.vpool);

  // page i of the split into slot sl: a cached page by DMA (returns true),
  // an appended-frame page not (it is built when its turn comes)
  auto stage = [&](int i, int sl) {
    int valid, fj;
    const int pg = map_page(a, p0 + i, valid, fj);
    if (fj >= 0) return false;
    const size_t off = ((size_t)pg * H + h) * (kPage * D);
    copy_tile_f32(kpool + off, lds[sl][0], wave, lane);
    copy_tile_f32(vpool + off, lds[sl][1], wave, lane);
    return true;
  };
  bool staged = stage(0, 0);
  for (int jj = 0; jj < np; ++jj) {
    const int sl = jj & 1;
    const bool next = jj + 1 < np && stage(jj + 1, sl ^ 1);
    // this wave's copies of page jj have landed (8 copies of page jj+1 may be in flight)
    if (next)
      GCA_WAIT_VMCNT(8);
    else
      GCA_WAIT_VMCNT(0);
    __syncthreads();
    int valid, fj;
    const int pg = map_page(a, p0 + jj, valid, fj);
    float* kt = lds[sl][0];
    float* vt = lds[sl][1];
    if (!staged && fj >= 0) {  // uniform: the appended frame's page, built here
      build_fresh_f32(a, kt, vt, fj, valid, h, tid);
      __syncthreads();
      if (qb == 0) store_fresh_f32(a, kt, vt, pg, h, tid);
    }
    staged = next;

    // S^T = K Q^T
    f32x16 sc[2][NJ];
#pragma unroll
    for (int kt_i = 0; kt_i < 2; ++kt_i) {
      const int row = kt_i * 32 + l32;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kt_i][j][r] = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(&kt[swz32(row, 8 * hf + u)]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            sc[kt_i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[j][4 * u + e], sc[kt_i][j], 0, 0, 0);
      }
    }
    if (valid < kPage) mask_page<NJ>(sc, valid, hf);
    // online softmax: the page's row max raises m, l and O are rescaled
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt_i = 0; kt_i < 2; ++kt_i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kt_i][j][r]);
      const float m_new = fmaxf(m[j], half_pair_max(mx));  // finite: every page holds a visible key
      const float alpha = exp2f((m[j] - m_new) * c2);    // 0 on the split's first page
      const float mc = m_new * c2;
      float ps = 0.f;
#pragma unroll
      for (int kt_i = 0; kt_i < 2; ++kt_i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt_i][j][r], c2, -mc));
          sc[kt_i][j][r] = p;
          ps += p;
        }
      l[j] = l[j] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][j][r] *= alpha;
      m[j] = m_new;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int drow = dt * 32 + l32;
#pragma unroll
      for (int kt_i = 0; kt_i < 2; ++kt_i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // keys 32kt + 8g + 4hf + q (q = 0..3) sit at columns 32kt + 16(g>>1) + 8hf + 4(g&1) + q
          const f32x4 vf = *reinterpret_cast<const f32x4*>(
              &vt[swz32(drow, 8 * kt_i + 4 * (g >> 1) + 2 * hf + (g & 1))]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              o[dt][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[q], sc[kt_i][j][4 * g + q], o[dt][j], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with slot sl: page jj+2 may go there
  }

  // outputs: register r of o[dt][j] holds d = 32dt + 8(r/4) + 4hf + r%4 of row 32j + l32
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float lt = half_pair_sum(l[j]);
    const int row = qb * kF32Rows + wave * 64 + j * 32 + l32;
    if (row >= a.Lq) continue;
    if (a.nsplit == 1) {
      const float inv = 1.f / lt;
      float* out = reinterpret_cast<float*>(a.out) + ((size_t)row * H + h) * D;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(out + 32 * dt + 8 * g + 4 * hf) =
              make_float4(o[dt][j][4 * g] * inv, o[dt][j][4 * g + 1] * inv, o[dt][j][4 * g + 2] * inv,
                          o[dt][j][4 * g + 3] * inv);
      if (a.lse != nullptr && hf == 0) a.lse[(size_t)h * a.Lq + row] = m[j] * a.scale + logf(lt);
    } else {
      float* po = reinterpret_cast<float*>(a.part_o) + (((size_t)h * a.nsplit + s) * a.Lq_pad + row) * D;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(po + 32 * dt + 8 * g + 4 * hf) =
              make_float4(o[dt][j][4 * g], o[dt][j][4 * g + 1], o[dt][j][4 * g + 2], o[dt][j][4 * g + 3]);
      if (hf == 0) a.part_ml[((size_t)h * a.nsplit + s) * a.Lq_pad + row] = make_float2(m[j], lt);
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the key splits + eviction, one launch
// ---------------------------------------------------------------------------

// Merge: O = sum_s w_s O_s / sum_s w_s l_s with w_s = exp2((m_s - max m) *
// scale * log2 e); LSE = scale * max m + ln(sum).  Block = 16 query rows x 16
// four-float chunks of one head.
template <bool kF32>
__device__ void merge_block(const AttnArgs& a, int h, int rb) {
  constexpr int D = kHeadDim;
  const int row = rb * 16 + (threadIdx.x >> 4);
  const int d4 = (threadIdx.x & 15) * 4;
  if (row >= a.Lq) return;
  const int ns = a.nsplit;
  const float2* ml = a.part_ml + (size_t)h * ns * a.Lq_pad + row;
  float M = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[(size_t)s * a.Lq_pad].x);
  const float c2 = a.scale_log2;
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const size_t first = ((size_t)h * ns * a.Lq_pad + row) * D + d4, stride = (size_t)a.Lq_pad * D;
  if (kF32) {
    // unnormalised fp32 partials: split s adds 2^((m_s - M) c2) (O_s, l_s)
    const float* po = reinterpret_cast<const float*>(a.part_o) + first;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const float2 v = ml[(size_t)s * a.Lq_pad];
      const float w = exp2f((v.x - M) * c2);
      L = __builtin_fmaf(w, v.y, L);
      const float4 x = *reinterpret_cast<const float4*>(po + s * stride);
      acc.x = __builtin_fmaf(w, x.x, acc.x);
      acc.y = __builtin_fmaf(w, x.y, acc.y);
      acc.z = __builtin_fmaf(w, x.z, acc.z);
      acc.w = __builtin_fmaf(w, x.w, acc.w);
    }
  } else {
    // normalised bf16 partials O_s / l_s with m_s in log2 units: split s
    // weighs 2^(m_s - M) l_s
    const uint16_t* po = reinterpret_cast<const uint16_t*>(a.part_o) + first;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const float2 v = ml[(size_t)s * a.Lq_pad];
      const float w = exp2f(v.x - M) * v.y;
      L += w;
      const uint2 x = *reinterpret_cast<const uint2*>(po + s * stride);
      acc.x = __builtin_fmaf(w, __builtin_bit_cast(float, x.x << 16), acc.x);
      acc.y = __builtin_fmaf(w, __builtin_bit_cast(float, x.x & 0xffff0000u), acc.y);
      acc.z = __builtin_fmaf(w, __builtin_bit_cast(float, x.y << 16), acc.z);
      acc.w = __builtin_fmaf(w, __builtin_bit_cast(float, x.y & 0xffff0000u), acc.w);
    }
  }
  const float inv = 1.f / L;
  const size_t o = ((size_t)row * a.H + h) * D + d4;
  if (kF32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    const __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv);
    const __bf16 b2 = (__bf16)(acc.z * inv), b3 = (__bf16)(acc.w * inv);
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o) = w;
  }
  if (d4 == 0 && a.lse != nullptr) a.lse[(size_t)h * a.Lq + row] = M * (kF32 ? a.scale : kLn2) + logf(L);
}

// Eviction, one workgroup per head: zero the head's slice of a new summary
// page, copy the frame's S summary rows (K rows and V^T columns) into the
// summary slots.  The head-0 workgroup also updates the page table: set the
// new page, append it to the summary list, free the frame's pages.  Copies
// read page contents only and the bookkeeping writes metadata only, so the
// workgroups need no ordering among themselves.
template <typename T>
__device__ void evict_block(const LayerDev& L, const EvictPlan& e, int h, int H) {
  constexpr int D = kHeadDim, P = kPage;
  T* kp = reinterpret_cast<T*>(L.kpool);
  T* vp = reinterpret_cast<T*>(L.vpool);
  if (e.new_page >= 0) {
    const size_t base = ((size_t)e.new_page * H + h) * P * D;
    for (int x = threadIdx.x; x < P * D; x += blockDim.x) {
      kp[base + x] = T(0);
      vp[base + x] = T(0);
    }
    __syncthreads();
  }
  for (int x = threadIdx.x; x < e.S * D; x += blockDim.x) {
    const int r = x / D, d = x % D;
    const int sp = e.src.p[r / P], ss = r % P;
    const int g = e.g0 + r;
    const int dp = (g / P == e.tail_index) ? e.tail_page : e.new_page, ds = g % P;
    kp[(((size_t)dp * H + h) * P + ds) * D + d] = kp[(((size_t)sp * H + h) * P + ss) * D + d];
    vp[(((size_t)dp * H + h) * D + d) * P + swap23(ds)] =
        vp[(((size_t)sp * H + h) * D + d) * P + swap23(ss)];
  }
  if (h == 0) {
    if ((int)threadIdx.x < e.ppf) {
      const int p = e.src.p[threadIdx.x];
      atomicAnd(&L.bitmap[p >> 5], ~(1u << (p & 31)));
      L.ftab[e.frame * e.ppf + threadIdx.x] = -1;
    }
    if (threadIdx.x == 0) {
      int used = -e.ppf;
      if (e.new_page >= 0) {
        atomicOr(&L.bitmap[e.new_page >> 5], 1u << (e.new_page & 31));
        L.slist[e.new_index] = e.new_page;
        L.ctr[kCtrSumPages] = e.new_index + 1;
        used += 1;
      }
      L.ctr[kCtrTraj] += 1;
      atomicAdd(&L.ctr[kCtrUsed], used);
    }
  }
}

template <bool kF32>
__global__ __launch_bounds__(256) void k_merge_evict(AttnArgs a, EvictPlan e, int merge_rowblocks,
                                                     int merge_heads) {
  const int b = blockIdx.x;
  const int nmerge = merge_rowblocks * merge_heads;
  if (b < nmerge) {
    merge_block<kF32>(a, b / merge_rowblocks, b % merge_rowblocks);
  } else {
    using T = typename std::conditional<kF32, float, uint16_t>::type;
    evict_block<T>(a.L, e, b - nmerge, a.H);
  }
}

// ---------------------------------------------------------------------------
// Static split-K scratch (gca_step_noalloc)
// ---------------------------------------------------------------------------

// The split partials of gca_step_noalloc live here instead of in the
// caller's workspace.  Host code never uses this name as an address: each
// device's copy sits at its own address, which static_scratch_address looks
// up once per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<void*> addr;  // per device
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launch wrappers
// ---------------------------------------------------------------------------

hipError_t launch_reset(const LayerDev& L, int pool_words, int ftab_entries, int slist_entries,
                        hipStream_t st) {
  int n = pool_words > ftab_entries ? pool_words : ftab_entries;
  n = n > slist_entries ? n : slist_entries;
  n = n > kCtrCount ? n : kCtrCount;
  int blocks = (n + 255) / 256;
  blocks = blocks > 1024 ? 1024 : blocks;
  hipLaunchKernelGGL(k_reset, dim3(blocks), dim3(256), 0, st, L, pool_words, ftab_entries,
                     slist_entries);
  return hipGetLastError();
}

hipError_t launch_append(const LayerDev& L, const void* k, const void* v, int frame,
                         const FramePages& pages, int ppf, int F, int H, bool f32,
                         const float2* rope, hipStream_t st) {
  dim3 grid(ppf, H);
  if (f32)
    hipLaunchKernelGGL(k_append<float>, grid, dim3(256), 0, st, L, (const float*)k,
                       (const float*)v, frame, pages, ppf, F, H, rope);
  else
    hipLaunchKernelGGL(k_append<uint16_t>, grid, dim3(256), 0, st, L, (const uint16_t*)k,
                       (const uint16_t*)v, frame, pages, ppf, F, H, rope);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool f32, hipStream_t st) {
  const int grid = a.H * a.qblocks * a.nsplit;
  if (a.batch < 1 || (a.batch > 1 && (a.nsplit != 1 || a.pl.fresh_cnt != a.pl.ppf))) return hipErrorInvalidValue;
  if (a.nsplit > 1 && (a.part_o == nullptr || a.part_ml == nullptr)) return hipErrorInvalidValue;
  const dim3 g3(grid, a.batch);
  // the bf16 kernel keeps its split's page list in LDS (the split count is
  // chosen so it always fits; checked here before anything is launched)
  for (int sp = 0; !f32 && sp < a.nsplit; ++sp)
    if (split_begin(a, sp + 1) - split_begin(a, sp) > kListCap) return hipErrorInvalidValue;
  // intra-frame attention (every page fresh, one split, no cache bookkeeping)
  // of a frame that fits the LDS tiles: the LDS-resident frame kernel
  const bool frame = a.pl.a_cnt == 0 && a.pl.s_cnt == 0 && a.pl.w_cnt == 0 && a.fresh_frame < 0 &&
                     a.pl.fresh_cnt == a.pl.ppf && a.pl.ppf <= kFrameTiles && a.Lq == a.F && a.nsplit == 1;
  if (f32)
    hipLaunchKernelGGL(k_attn_f32, g3, dim3(256), 0, st, a);
  else if (frame && a.rope == nullptr && GCA_FRAME_RING && a.batch < 1024) {  // (the frame fits its entry field)
    // one workgroup per (frame, head) item while they fit the CUs at once;
    // past that, persistent workgroups, one per CU (items of a single page
    // keep a workgroup each)
    const int items = a.H * a.batch;
    if (a.pl.ppf >= 2 && items > kTargetWgs && GCA_FRAME_PERSIST)
      hipLaunchKernelGGL((k_attn_bf16<kAttnWaves, true, true>), dim3(kTargetWgs), dim3(kAttnWaves * 64), 0, st, a);
    else
      hipLaunchKernelGGL((k_attn_bf16<kAttnWaves, true, false>), dim3(items), dim3(kAttnWaves * 64), 0, st, a);
  }
  else if (frame)
    hipLaunchKernelGGL(k_frame_attn_bf16, g3, dim3(kAttnWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_bf16<kAttnWaves, false>), g3, dim3(kAttnWaves * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_frame_wsplit(const AttnArgs& a, hipStream_t st) {
  if (a.batch < 1 || a.nsplit != 1 || a.pl.ppf < 1 || a.pl.ppf > kAttnWaves || a.Lq != a.F || a.H < 1)
    return hipErrorInvalidValue;
  const dim3 g3(a.H * ((a.Lq + kWsRows - 1) / kWsRows), a.batch);
  if (a.rope != nullptr)
    hipLaunchKernelGGL(k_frame_wsplit_bf16<true>, g3, dim3(kAttnWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(k_frame_wsplit_bf16<false>, g3, dim3(kAttnWaves * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_evict(const AttnArgs& a, const EvictPlan* ev, bool f32, hipStream_t st) {
  if (a.nsplit > 1 && (a.part_o == nullptr || a.part_ml == nullptr)) return hipErrorInvalidValue;
  const int rowblocks = a.nsplit > 1 ? (a.Lq + 15) / 16 : 0;
  const int mheads = a.nsplit > 1 ? a.H : 0;
  const int eblocks = ev != nullptr ? a.H : 0;
  const int grid = rowblocks * mheads + eblocks;
  if (grid == 0) return hipSuccess;
  EvictPlan e{};
  if (ev != nullptr) e = *ev;
  if (f32)
    hipLaunchKernelGGL(k_merge_evict<true>, dim3(grid), dim3(256), 0, st, a, e, rowblocks, mheads);
  else
    hipLaunchKernelGGL(k_merge_evict<false>, dim3(grid), dim3(256), 0, st, a, e, rowblocks, mheads);
  return hipGetLastError();
}

}  // namespace gca
