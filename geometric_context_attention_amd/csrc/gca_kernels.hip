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

#include <type_traits>

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

// Grid (ppf, H): copy one head's 64 slots of one page of frame `frame` into
// the page the host chose for it.  K rows are copied as they are; V rows are
// transposed through LDS.  Slots past the frame's last row are zero-filled.
// Workgroup (0, 0) records the pages in the frame table and the bitmap.
// T = uint16_t (bf16 bits) or float.
template <typename T>
__global__ __launch_bounds__(256) void k_append(LayerDev L, const T* __restrict__ kin,
                                                const T* __restrict__ vin, int frame,
                                                FramePages pages, int ppf, int F, int H) {
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
__device__ __forceinline__ int map_page(const AttnArgs& a, int i, int& valid, int& fj) {
  const PageList& pl = a.pl;
  fj = -1;
  int pg;
  if (i < pl.a_cnt) {
    valid = (i % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = a.ftab[i];
  } else if ((i -= pl.a_cnt) < pl.s_cnt) {
    valid = (i == pl.s_cnt - 1) ? pl.s_last_valid : kPage;
    pg = a.slist[i];
  } else if ((i -= pl.s_cnt) < pl.w_cnt) {
    const int e = pl.w_first + i;
    valid = (e % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = a.ftab[e];
  } else {
    i -= pl.w_cnt;
    fj = i;
    valid = (i == pl.ppf - 1) ? pl.f_last_valid : kPage;
    pg = a.fresh.p[i];
  }
  if ((unsigned)pg >= (unsigned)a.pool) {
    valid = 0;
    fj = -1;
    pg = 0;
  }
  return pg;
}

// Zero the V^T entries of slots >= valid in a 16-byte chunk of one d row
// (stored columns 8*ch .. 8*ch+7), so that a masked key (probability 0) never
// meets a non-finite value in the PV product.
__device__ __forceinline__ uint4 mask_vt_chunk(uint4 v, int ch, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (swap23(ch * 8 + e) >= valid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
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
    const int p = a.fresh.p[threadIdx.x];
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
// tiles j.  Keys are taken in 32-key tiles (two per 64-slot page):
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
// Software pipeline: while the VALU computes the softmax of key tile u, the
// MFMA pipe works on QK^T of tile u+1 and on PV of tile u-1; the three are
// independent, so one wave keeps both units busy.  Pages are staged through
// a triple LDS buffer (K runs one page ahead of V), one barrier per page.
// The running max is only moved (and O rescaled) when it grows by more than
// 2^8 in probability units, which keeps p <= 256 and the sums in fp32 range.
// Pages of the frame being appended are read from k_in / v_in, staged like any
// page, and written to their pool pages by the query-block-0 workgroups.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct PageInfo {
  int valid;
  int fj;       // index within the appended frame, or -1
  size_t off;   // element offset of the head's slice in the pools
};

constexpr float kLazyRescaleLog2 = 8.0f;
#ifndef GCA_ATTN_WAVES
#define GCA_ATTN_WAVES 8
#endif
constexpr int kAttnWaves = GCA_ATTN_WAVES;  // 8 waves = 2 per SIMD

template <int NJ>
__device__ __forceinline__ void qk_tile(const uint16_t* sKb, int kt, const bf16x8 (&qf)[NJ][4],
                                        f32x16 (&sc)[NJ], int l32, int hf) {
  constexpr int LR = 72;
  const f32x16 zero = {};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sKb[(kt * 32 + l32) * LR + c * 16 + hf * 8]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      sc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j][c], c == 0 ? zero : sc[j], 0, 0, 0);
  }
}

template <int NJ>
__device__ __forceinline__ void mask_tile(f32x16 (&sc)[NJ], int valid, int kt, int hf) {
  if (valid >= kt * 32 + 32) return;  // wave-uniform
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
    if (key >= valid) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) sc[j][r] = -INFINITY;
    }
  }
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max of a lane's value and the value of the lane 32 apart (the two halves of
// a wave hold the two key halves of the same query column)
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

// Running max of tile sc; moves it (and rescales l and O) only when some
// column's max grew by more than thr (raw score units).  O must already hold
// every tile before this one.
template <int NJ>
__device__ __forceinline__ void softmax_max(const f32x16 (&sc)[NJ], float (&m)[NJ], float (&l)[NJ],
                                            f32x16 (&o)[2][NJ], float c2, float thr) {
  float mx[NJ];
  bool need = false;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const f32x16& v = sc[j];
    const float a = max3f(v[0], v[1], v[2]), b = max3f(v[3], v[4], v[5]);
    const float c = max3f(v[6], v[7], v[8]), d = max3f(v[9], v[10], v[11]);
    const float e = max3f(v[12], v[13], v[14]);
    mx[j] = half_pair_max(fmaxf(max3f(a, b, c), max3f(d, e, v[15])));
    need |= mx[j] - m[j] > thr;
  }
  if (__any(need)) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float mnew = fmaxf(m[j], mx[j]);
      const float alpha = __builtin_amdgcn_exp2f((m[j] - mnew) * c2);
      l[j] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][j][r] *= alpha;
        o[1][j][r] *= alpha;
      }
      m[j] = mnew;
    }
  }
}

// p = exp2((s - m) * scale * log2 e) as packed bf16 P^T fragments; the row
// sums accumulate the same rounded values (v_dot2 with (1, 1)).
template <int NJ>
__device__ __forceinline__ void softmax_exp(const f32x16 (&sc)[NJ], const float (&m)[NJ],
                                            float (&l)[NJ], bf16x8 (&pf)[NJ][2], float c2) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const float mc = m[j] * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pf[j][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[j][r], c2, -mc));
    float acc = l[j];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pf[j][hh][e], pf[j][hh][e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
      }
    l[j] = acc;
  }
  // Keep the exponentials in this block, next to the MFMAs they overlap
  // with, instead of letting the compiler sink them towards their use in the
  // next page step (an empty statement that only reads the fragments).
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) asm volatile("" ::"v"(pf[j][hh]));
}

// Scheduling hint for a block holding 8 QK^T MFMAs and the softmax VALU work
// of one tile: alternate one MFMA with a run of VALU instructions.
__device__ __forceinline__ void interleave_hint() {
#ifdef GCA_SCHED_HINTS
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, GCA_SCHED_HINTS, 0);
  }
#endif
}

template <int NJ>
__device__ __forceinline__ void pv_tile(const uint16_t* sVb, int kt, const bf16x8 (&pf)[NJ][2],
                                        f32x16 (&o)[2][NJ], int l32, int hf) {
  constexpr int LR = 72;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int kc = kt * 2 + hh;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sVb[(dt * 32 + l32) * LR + kc * 16 + hf * 8]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        o[dt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j][hh], o[dt][j], 0, 0, 0);
    }
  }
}

// NW waves of 64 lanes; wave w owns query rows [w*32*NJ, (w+1)*32*NJ) of the
// 512-row block as NJ tiles of 32 rows (NW * NJ = 16).
template <int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_bf16(AttnArgs a) {
  constexpr int NJ = 16 / NW;
  constexpr int NT = NW * 64;          // threads
  constexpr int CPT = 512 / NT;        // 16-byte chunks of an 8 KB tile per thread
  constexpr int D = kHeadDim, P = kPage, LR = 72;  // LDS row: 64 bf16 + 8 pad
  constexpr int TILE = P * LR;
  __shared__ __attribute__((aligned(16))) uint16_t sK[3][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const int H = a.H;
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt + a.pl.fresh_cnt;
  const int p0 = (int)((long long)npg * s / a.nsplit);
  const int p1 = (int)((long long)npg * (s + 1) / a.nsplit);
  if (a.pl.fresh_cnt > 0 && blockIdx.x == 0) record_fresh_frame(a);

  // Q^T fragments: tile j, d-chunk c: column q = 32j + l32, d = 16c + 8hf .. +7
  bf16x8 qf[NJ][4];
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = qb * kQBlock + wave * 32 * NJ + j * 32 + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < a.Lq)
        v = *reinterpret_cast<const uint4*>(qbase + ((size_t)row * H + h) * D + c * 16 + hf * 8);
      qf[j][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

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
    m[j] = -INFINITY;
    l[j] = 0.f;
  }
  const float c2 = a.scale_log2;
  const float thr = kLazyRescaleLog2 / c2;  // in raw score units

  uint16_t* kpool = reinterpret_cast<uint16_t*>(a.kpool);
  uint16_t* vpool = reinterpret_cast<uint16_t*>(a.vpool);
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(a.k_in);
  const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v_in);

  auto info_of = [&](int i) {
    PageInfo pi;
    const int pg = map_page(a, i, pi.valid, pi.fj);
    pi.off = ((size_t)pg * H + h) * (P * D);
    return pi;
  };
  // chunk x of a tile = 16 bytes at element 8x: row x/8, column chunk x%8
  auto load_k = [&](const PageInfo& pi, uint4 (&kv)[CPT]) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + u * NT, row = x >> 3, ch = x & 7;
      if (pi.fj < 0) {
        kv[u] = *reinterpret_cast<const uint4*>(kpool + pi.off + x * 8);
      } else {
        kv[u] = make_uint4(0u, 0u, 0u, 0u);
        if (row < pi.valid)
          kv[u] = *reinterpret_cast<const uint4*>(kin + ((size_t)(pi.fj * P + row) * H + h) * D + ch * 8);
        if (qb == 0) *reinterpret_cast<uint4*>(kpool + pi.off + x * 8) = kv[u];
      }
    }
  };
  auto load_v = [&](const PageInfo& pi, uint4 (&vv)[CPT]) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + u * NT, row = x >> 3, ch = x & 7;
      vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (pi.fj < 0) {
        vv[u] = *reinterpret_cast<const uint4*>(vpool + pi.off + x * 8);
        if (pi.valid < P) vv[u] = mask_vt_chunk(vv[u], ch, pi.valid);
      } else if (row < pi.valid) {
        vv[u] = *reinterpret_cast<const uint4*>(vin + ((size_t)(pi.fj * P + row) * H + h) * D + ch * 8);
      }
    }
  };
  auto store_k = [&](int b, const uint4 (&kv)[CPT]) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + u * NT;
      *reinterpret_cast<uint4*>(&sK[b][(x >> 3) * LR + (x & 7) * 8]) = kv[u];
    }
  };
  auto store_v = [&](int b, const uint4 (&vv)[CPT], int fj) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + u * NT, row = x >> 3, ch = x & 7;
      if (fj < 0) {
        *reinterpret_cast<uint4*>(&sV[b][row * LR + ch * 8]) = vv[u];
      } else {  // rows of the input: transpose into V^T on the way
        const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        const int col = swap23(row);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sV[b][(ch * 8 + e) * LR + col] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
      }
    }
  };

  // prologue: K and V of page p0, K of page p0+1; the V buffer of "page
  // p0-1" is zeroed so that the first PV of the loop (with P = 0) is a no-op
  PageInfo pi0 = info_of(p0);
  PageInfo pi1{P, -1, 0}, pi2{P, -1, 0};
  {
    uint4 kv[CPT], vv[CPT];
    load_k(pi0, kv);
    load_v(pi0, vv);
    store_k(0, kv);
    store_v(0, vv, pi0.fj);
    if (p0 + 1 < p1) {
      pi1 = info_of(p0 + 1);
      load_k(pi1, kv);
      store_k(1, kv);
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int x = tid + u * NT;
      *reinterpret_cast<uint4*>(&sV[2][(x >> 3) * LR + (x & 7) * 8]) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();

  f32x16 s_cur[NJ], s_nxt[NJ];
  bf16x8 p_cur[NJ][2], p_prev[NJ][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) p_prev[j][hh][e] = (__bf16)0.0f;
  qk_tile<NJ>(sK[0], 0, qf, s_cur, l32, hf);

  int b0 = 0, b1 = 1, b2 = 2;  // buffers of pages i, i+1, i+2 (V of page i-1 is in b2)
  // One page: tiles u = (i, 0) and (i, 1).  Each half: mask the tile whose
  // QK^T was issued in the previous half, issue PV of the previous tile, move
  // the running max, then one branch-free block with QK^T of the next tile on
  // the MFMA pipe and the exponentials of this tile on the VALU.
  auto page_step = [&](int i, auto has1_c, auto has2_c, auto masked_c) {
    constexpr bool has1 = decltype(has1_c)::value, has2 = decltype(has2_c)::value;
    constexpr bool masked = decltype(masked_c)::value;  // page i has empty slots
    uint4 kn[CPT], vn[CPT];
    if (has2) {
      pi2 = info_of(i + 2);
      load_k(pi2, kn);
    }
    if (has1) load_v(pi1, vn);
    if (pi0.fj >= 0 && qb == 0) {  // the appended frame's V^T tile goes to its pool page
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int x = tid + u * NT;
        *reinterpret_cast<uint4*>(vpool + pi0.off + x * 8) =
            *reinterpret_cast<const uint4*>(&sV[b0][(x >> 3) * LR + (x & 7) * 8]);
      }
    }
    // half 0: tile (i, 0)
    if (masked) mask_tile<NJ>(s_cur, pi0.valid, 0, hf);
    pv_tile<NJ>(sV[b2], 1, p_prev, o, l32, hf);
    softmax_max<NJ>(s_cur, m, l, o, c2, thr);
    qk_tile<NJ>(sK[b0], 1, qf, s_nxt, l32, hf);
    softmax_exp<NJ>(s_cur, m, l, p_cur, c2);
    interleave_hint();
    // half 1: tile (i, 1)
    if (masked) mask_tile<NJ>(s_nxt, pi0.valid, 1, hf);
    pv_tile<NJ>(sV[b0], 0, p_cur, o, l32, hf);
    softmax_max<NJ>(s_nxt, m, l, o, c2, thr);
    if (has1) qk_tile<NJ>(sK[b1], 0, qf, s_cur, l32, hf);
    softmax_exp<NJ>(s_nxt, m, l, p_prev, c2);
    interleave_hint();

    if (has2) store_k(b2, kn);
    if (has1) store_v(b1, vn, pi1.fj);
    pi0 = pi1;
    pi1 = pi2;
    const int t0 = b0;
    b0 = b1;
    b1 = b2;
    b2 = t0;
    __syncthreads();
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  // full pages take a body without any masking code (no branch splits the
  // MFMA/VALU block); the few partial pages (a frame's last page, the
  // summary tail) take the masked body
  int i = p0;
  for (; i + 2 < p1; ++i) {
    if (pi0.valid == P)
      page_step(i, T_{}, T_{}, F_{});
    else
      page_step(i, T_{}, T_{}, T_{});
  }
  if (i + 1 < p1) page_step(i++, T_{}, F_{}, T_{});
  page_step(i, F_{}, F_{}, T_{});
  pv_tile<NJ>(sV[b2], 1, p_prev, o, l32, hf);  // tile (p1-1, 1)

  // epilogue
#pragma unroll
  for (int j = 0; j < NJ; ++j) l[j] = half_pair_sum(l[j]);
  const bool final_out = a.nsplit == 1;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = qb * kQBlock + wave * 32 * NJ + j * 32 + l32;
    if (final_out) {
      if (row < a.Lq) {
        const float inv = 1.f / l[j];
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * H + h) * D;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * hf;
            __bf16 b0v = (__bf16)(o[dt][j][4 * g + 0] * inv), b1v = (__bf16)(o[dt][j][4 * g + 1] * inv);
            __bf16 b2v = (__bf16)(o[dt][j][4 * g + 2] * inv), b3v = (__bf16)(o[dt][j][4 * g + 3] * inv);
            uint2 w;
            w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0v) | ((uint32_t)__builtin_bit_cast(uint16_t, b1v) << 16);
            w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2v) | ((uint32_t)__builtin_bit_cast(uint16_t, b3v) << 16);
            *reinterpret_cast<uint2*>(out + d) = w;
          }
        if (a.lse != nullptr && hf == 0) a.lse[(size_t)h * a.Lq + row] = m[j] * a.scale + logf(l[j]);
      }
    } else {
      float* po = a.part_o + (((size_t)h * a.nsplit + s) * a.Lq_pad + row) * D;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = dt * 32 + 8 * g + 4 * hf;
          *reinterpret_cast<float4*>(po + d) =
              make_float4(o[dt][j][4 * g + 0], o[dt][j][4 * g + 1], o[dt][j][4 * g + 2], o[dt][j][4 * g + 3]);
        }
      if (hf == 0) a.part_ml[((size_t)h * a.nsplit + s) * a.Lq_pad + row] = make_float2(m[j], l[j]);
    }
  }
}

// fp32 attention: one thread per query row (256-row blocks).  Each page is
// staged in LDS; keys are taken one at a time with an online softmax.
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  constexpr int D = kHeadDim, P = kPage;
  __shared__ float sK[P][D + 1];
  __shared__ float sV[D][P + 1];
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const int H = a.H;
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt + a.pl.fresh_cnt;
  const int p0 = (int)((long long)npg * s / a.nsplit);
  const int p1 = (int)((long long)npg * (s + 1) / a.nsplit);
  if (a.pl.fresh_cnt > 0 && blockIdx.x == 0) record_fresh_frame(a);
  const int row = qb * kF32Rows + threadIdx.x;
  const bool live = row < a.Lq;
  const float* q = reinterpret_cast<const float*>(a.q);
  float qv[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = live ? q[((size_t)row * H + h) * D + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c2 = a.scale_log2;
  float* kpool = reinterpret_cast<float*>(a.kpool);
  float* vpool = reinterpret_cast<float*>(a.vpool);
  const float* kin = reinterpret_cast<const float*>(a.k_in);
  const float* vin = reinterpret_cast<const float*>(a.v_in);
  for (int i = p0; i < p1; ++i) {
    int valid, fj;
    const int pg = map_page(a, i, valid, fj);
    const size_t off = ((size_t)pg * H + h) * (P * D);
    __syncthreads();
    if (fj < 0) {
      for (int e = threadIdx.x; e < P * D; e += 256) {
        sK[e / D][e % D] = kpool[off + e];
        sV[e / P][e % P] = vpool[off + e];
      }
    } else {
      for (int e = threadIdx.x; e < P * D; e += 256) {
        const int r = e / D, d = e % D;
        float kv = 0.f, vv = 0.f;
        if (r < valid) {
          const size_t src = ((size_t)(fj * P + r) * H + h) * D + d;
          kv = kin[src];
          vv = vin[src];
        }
        sK[r][d] = kv;
        sV[d][swap23(r)] = vv;
      }
    }
    __syncthreads();
    if (fj >= 0 && qb == 0) {
      for (int e = threadIdx.x; e < P * D; e += 256) {
        kpool[off + e] = sK[e / D][e % D];
        vpool[off + e] = sV[e / P][e % P];
      }
    }
#pragma unroll 1
    for (int key = 0; key < valid; ++key) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qv[d], sK[key][d], acc);
      if (acc > m) {
        const float alpha = exp2f((m - acc) * c2);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        m = acc;
      }
      const float p = exp2f((acc - m) * c2);
      l += p;
      const int col = swap23(key);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, sV[d][col], o[d]);
    }
  }
  if (!live) return;
  if (a.nsplit == 1) {
    const float inv = 1.f / l;
    float* out = reinterpret_cast<float*>(a.out) + ((size_t)row * H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) out[d] = o[d] * inv;
    if (a.lse != nullptr) a.lse[(size_t)h * a.Lq + row] = m * a.scale + logf(l);
  } else {
    float* po = a.part_o + (((size_t)h * a.nsplit + s) * a.Lq_pad + row) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) po[d] = o[d];
    a.part_ml[((size_t)h * a.nsplit + s) * a.Lq_pad + row] = make_float2(m, l);
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
  const float* po = a.part_o + ((size_t)h * ns * a.Lq_pad + row) * D + d4;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float2 v = ml[(size_t)s * a.Lq_pad];
    const float w = exp2f((v.x - M) * c2);
    L = __builtin_fmaf(w, v.y, L);
    const float4 x = *reinterpret_cast<const float4*>(po + (size_t)s * a.Lq_pad * D);
    acc.x = __builtin_fmaf(w, x.x, acc.x);
    acc.y = __builtin_fmaf(w, x.y, acc.y);
    acc.z = __builtin_fmaf(w, x.z, acc.z);
    acc.w = __builtin_fmaf(w, x.w, acc.w);
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
  if (d4 == 0 && a.lse != nullptr) a.lse[(size_t)h * a.Lq + row] = M * a.scale + logf(L);
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
                         hipStream_t st) {
  dim3 grid(ppf, H);
  if (f32)
    hipLaunchKernelGGL(k_append<float>, grid, dim3(256), 0, st, L, (const float*)k,
                       (const float*)v, frame, pages, ppf, F, H);
  else
    hipLaunchKernelGGL(k_append<uint16_t>, grid, dim3(256), 0, st, L, (const uint16_t*)k,
                       (const uint16_t*)v, frame, pages, ppf, F, H);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool f32, hipStream_t st) {
  const int grid = a.H * a.qblocks * a.nsplit;
  if (f32)
    hipLaunchKernelGGL(k_attn_f32, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_attn_bf16<kAttnWaves>, dim3(grid), dim3(kAttnWaves * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_evict(const AttnArgs& a, const EvictPlan* ev, bool f32, hipStream_t st) {
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
