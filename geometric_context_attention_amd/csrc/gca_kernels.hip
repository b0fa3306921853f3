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

// One workgroup: take the ppf*nframes lowest free pages; frame first_frame+f
// gets ranks [f*ppf, (f+1)*ppf) in ascending page order.
__global__ __launch_bounds__(1024) void k_alloc_frames(LayerDev L, int pool_pages, int ppf,
                                                       int first_frame, int nframes) {
  const int need = ppf * nframes;
  const int nwords = (pool_pages + 31) >> 5;
  __shared__ int s_scan[1024];
  __shared__ int s_base;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  for (int w0 = 0; w0 < nwords; w0 += 1024) {
    const int base = s_base;
    if (base >= need) break;  // uniform: read after a barrier
    const int w = w0 + (int)threadIdx.x;
    uint32_t word = 0u, freebits = 0u;
    if (w < nwords) {
      word = L.bitmap[w];
      const int tail = pool_pages & 31;
      const uint32_t valid = (w == nwords - 1 && tail) ? ((1u << tail) - 1u) : 0xffffffffu;
      freebits = ~word & valid;
    }
    const int cnt = __popc(freebits);
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = (int)threadIdx.x >= off ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += v;
      __syncthreads();
    }
    const int incl = s_scan[threadIdx.x];
    int rank = base + incl - cnt;
    uint32_t taken = 0u;
    while (freebits && rank < need) {
      const int b = __ffs(freebits) - 1;
      freebits &= freebits - 1u;
      const int page = w * 32 + b;
      L.ftab[(first_frame + rank / ppf) * ppf + rank % ppf] = page;
      taken |= 1u << b;
      ++rank;
    }
    if (taken) L.bitmap[w] = word | taken;
    __syncthreads();
    if (threadIdx.x == 1023) s_base = base + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int got = s_base < need ? s_base : need;
    if (got < need) L.ctr[kCtrError] = 1;
    L.ctr[kCtrFrames] = first_frame + nframes;
    L.ctr[kCtrUsed] += got;
  }
}

// Grid (nframes*ppf, H): copy one head's 64 slots of one frame page.  K rows
// are copied as they are; V rows are transposed through LDS.  Slots past the
// frame's last row are zero-filled.  T = uint16_t (bf16 bits) or float.
template <typename T>
__global__ __launch_bounds__(256) void k_append(LayerDev L, const T* __restrict__ kin,
                                                const T* __restrict__ vin, int first_frame,
                                                int ppf, int F, int H) {
  constexpr int D = kHeadDim, P = kPage;
  const int pg = blockIdx.x, h = blockIdx.y;
  const int fl = pg / ppf, j = pg % ppf;
  const int page = L.ftab[(first_frame + fl) * ppf + j];
  if (page < 0) {
    if (threadIdx.x == 0) L.ctr[kCtrError] = 2;
    return;
  }
  T* kdst = reinterpret_cast<T*>(L.kpool) + ((size_t)page * H + h) * P * D;
  T* vdst = reinterpret_cast<T*>(L.vpool) + ((size_t)page * H + h) * D * P;
  __shared__ T tile[P][D + 1];
  const int row0 = fl * F + j * P;
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
}

// Lowest free page of the pool (block-wide), or -1.
__device__ int block_lowest_free(const uint32_t* bitmap, int pool_pages, int* s_min) {
  if (threadIdx.x == 0) *s_min = 0x7fffffff;
  __syncthreads();
  const int nwords = (pool_pages + 31) >> 5;
  for (int w = threadIdx.x; w < nwords; w += blockDim.x) {
    const int tail = pool_pages & 31;
    const uint32_t valid = (w == nwords - 1 && tail) ? ((1u << tail) - 1u) : 0xffffffffu;
    const uint32_t fb = ~bitmap[w] & valid;
    if (fb) {
      atomicMin(s_min, w * 32 + __ffs(fb) - 1);
      break;  // later words of this thread hold larger pages
    }
  }
  __syncthreads();
  const int p = *s_min;
  __syncthreads();
  return p == 0x7fffffff ? -1 : p;
}

// One workgroup: move frame `frame`'s S summary rows to the trajectory memory
// (new tail page first if needed), then free the frame's pages.
template <typename T>
__global__ __launch_bounds__(256) void k_evict(LayerDev L, int pool_pages, int frame, int ppf,
                                               int S, int H) {
  constexpr int D = kHeadDim, P = kPage;
  __shared__ int s_min;
  __shared__ int s_ctr[2];
  if (threadIdx.x == 0) {
    s_ctr[0] = L.ctr[kCtrTraj];
    s_ctr[1] = L.ctr[kCtrSumPages];
  }
  __syncthreads();
  const int traj = s_ctr[0];
  const int nsp_old = s_ctr[1];
  const int g0 = S * traj;
  const int need = (g0 + S - 1) / P + 1 - nsp_old;  // 0 or 1 for S <= 64
  int new_page = -1;
  if (need > 0) {
    new_page = block_lowest_free(L.bitmap, pool_pages, &s_min);
    if (new_page < 0) {
      if (threadIdx.x == 0) L.ctr[kCtrError] = 3;
      return;
    }
    if (threadIdx.x == 0) {
      L.bitmap[new_page >> 5] |= 1u << (new_page & 31);
      L.slist[nsp_old] = new_page;
    }
  }
  const int nsp = nsp_old + need;
  T* kp = reinterpret_cast<T*>(L.kpool);
  T* vp = reinterpret_cast<T*>(L.vpool);
  if (need > 0) {  // a new summary page starts as zeros: its unused slots stay finite
    const size_t base = (size_t)new_page * H * P * D;
    for (int e = threadIdx.x; e < H * P * D; e += 256) {
      kp[base + e] = T(0);
      vp[base + e] = T(0);
    }
    __syncthreads();
  }
  if (L.ftab[frame * ppf] < 0) {  // the frame is not resident: corrupt state
    if (threadIdx.x == 0) L.ctr[kCtrError] = 4;
    return;
  }
  for (int e = threadIdx.x; e < S * H * D; e += 256) {
    const int r = e / (H * D), h = (e / D) % H, d = e % D;
    const int sp = L.ftab[frame * ppf + r / P], ss = r % P;
    const int g = g0 + r;
    const int dp = (g / P < nsp_old) ? L.slist[g / P] : new_page, ds = g % P;
    kp[(((size_t)dp * H + h) * P + ds) * D + d] = kp[(((size_t)sp * H + h) * P + ss) * D + d];
    vp[(((size_t)dp * H + h) * D + d) * P + swap23(ds)] =
        vp[(((size_t)sp * H + h) * D + d) * P + swap23(ss)];
  }
  __syncthreads();
  if ((int)threadIdx.x < ppf) {
    const int e = frame * ppf + threadIdx.x;
    const int p = L.ftab[e];
    if (p >= 0 && p < pool_pages) atomicAnd(&L.bitmap[p >> 5], ~(1u << (p & 31)));
    L.ftab[e] = -1;
  }
  if (threadIdx.x == 0) {
    L.ctr[kCtrTraj] = traj + 1;
    L.ctr[kCtrSumPages] = nsp;
    L.ctr[kCtrUsed] += need - ppf;
  }
}

// ---------------------------------------------------------------------------
// Attention over the page list
// ---------------------------------------------------------------------------

__device__ __forceinline__ int map_page(const AttnArgs& a, int i, int& valid) {
  const PageList& pl = a.pl;
  if (i < pl.a_cnt) {
    valid = (i % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
    return a.ftab[i];
  }
  i -= pl.a_cnt;
  if (i < pl.s_cnt) {
    valid = (i == pl.s_cnt - 1) ? pl.s_last_valid : kPage;
    return a.slist[i];
  }
  const int e = pl.w_first + (i - pl.s_cnt);
  valid = (e % pl.ppf == pl.ppf - 1) ? pl.f_last_valid : kPage;
  return a.ftab[e];
}

// map_page with a range guard: a page index outside the pool (only possible
// if the page table is corrupt) reads page 0 with every slot masked.
__device__ __forceinline__ int map_page_safe(const AttnArgs& a, int i, int& valid) {
  const int pg = map_page(a, i, valid);
  if ((unsigned)pg >= (unsigned)a.pool) {
    valid = 0;
    return 0;
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

// bf16 attention, one workgroup = (head, 512 query rows, one key split).
// 8 waves, wave w owns query rows [64w, 64w+64) of the block as two 32-row
// tiles.  Per 64-key page, staged in LDS (double buffered):
//   S^T[key][q] = K Q^T   v_mfma_f32_32x32x16_bf16, A = K (LDS), B = Q^T (regs)
//   online softmax per query column, p = exp2((s - m) * scale * log2 e)
//   O^T[d][q] += V^T P^T  A = V^T (LDS), B = P^T straight from the S^T
//                         accumulator: lane half h holds keys {4h..4h+3,
//                         8+4h..8+4h+3} of each 16-key chunk, which is the
//                         order the V page stores them in (swap23).
// Operand layout of the 32x32x16 MFMA: A lane l holds row l%32, k 8(l/32)..+7;
// B lane l holds column l%32, same k; accumulator register r of lane l is row
// 8(r/4) + 4(l/32) + r%4, column l%32.
__global__ __launch_bounds__(512, 1) void k_attn_bf16(AttnArgs a) {
  constexpr int D = kHeadDim, P = kPage, LR = 72;  // LDS row: 64 bf16 + 8 pad
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][P * LR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * LR];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const int H = a.H;
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt;
  const int p0 = (int)((long long)npg * s / a.nsplit);
  const int p1 = (int)((long long)npg * (s + 1) / a.nsplit);

  // Q^T fragments: tile j, d-chunk c: column q = 32j + l32, d = 16c + 8hf .. +7
  bf16x8 qf[2][4];
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = qb * kQBlock + wave * 64 + j * 32 + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < a.Lq)
        v = *reinterpret_cast<const uint4*>(qbase + ((size_t)row * H + h) * D + c * 16 + hf * 8);
      qf[j][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[2][2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const float c2 = a.scale_log2;

  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.kpool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.vpool);
  const int ld_row = tid >> 3, ld_ch = tid & 7;  // 512 threads x 16 B = one 8 KB tile

  int valid_cur = P;
  if (p0 < p1) {
    const int pg = map_page_safe(a, p0, valid_cur);
    const size_t off = ((size_t)pg * H + h) * (P * D);
    const uint4 kv = *reinterpret_cast<const uint4*>(kpool + off + tid * 8);
    uint4 vv = *reinterpret_cast<const uint4*>(vpool + off + tid * 8);
    if (valid_cur < P) vv = mask_vt_chunk(vv, ld_ch, valid_cur);
    *reinterpret_cast<uint4*>(&sK[0][ld_row * LR + ld_ch * 8]) = kv;
    *reinterpret_cast<uint4*>(&sV[0][ld_row * LR + ld_ch * 8]) = vv;
  }
  __syncthreads();

  for (int i = p0; i < p1; ++i) {
    const int buf = (i - p0) & 1;
    // prefetch page i+1 into registers
    uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
    int valid_next = P;
    const bool has_next = i + 1 < p1;
    if (has_next) {
      const int pg = map_page_safe(a, i + 1, valid_next);
      const size_t off = ((size_t)pg * H + h) * (P * D);
      kn = *reinterpret_cast<const uint4*>(kpool + off + tid * 8);
      vn = *reinterpret_cast<const uint4*>(vpool + off + tid * 8);
    }

    // S^T = K Q^T
    f32x16 sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][j][r] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[buf][(kt * 32 + l32) * LR + c * 16 + hf * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          sacc[kt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j][c], sacc[kt][j], 0, 0, 0);
      }
    }
    if (valid_cur < P) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= valid_cur) {
            sacc[kt][0][r] = -INFINITY;
            sacc[kt][1][r] = -INFINITY;
          }
        }
    }

    // online softmax, one query column per lane and tile
    bf16x8 pf[2][4];  // [j][16-key chunk]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float mx = sacc[0][j][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][j][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[j], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[j] - mnew) * c2);
      const float mc = mnew * c2;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][j][r], c2, -mc));
          sum += p;
          pf[j][kt * 2 + (r >> 3)][r & 7] = (__bf16)p;
        }
      l[j] = l[j] * alpha + sum;
      m[j] = mnew;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][j][r] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sV[buf][(dt * 32 + l32) * LR + kc * 16 + hf * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[dt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j][kc], o[dt][j], 0, 0, 0);
      }
    }

    if (has_next) {
      if (valid_next < P) vn = mask_vt_chunk(vn, ld_ch, valid_next);
      *reinterpret_cast<uint4*>(&sK[buf ^ 1][ld_row * LR + ld_ch * 8]) = kn;
      *reinterpret_cast<uint4*>(&sV[buf ^ 1][ld_row * LR + ld_ch * 8]) = vn;
    }
    valid_cur = valid_next;
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int j = 0; j < 2; ++j) l[j] += __shfl_xor(l[j], 32);
  const bool final_out = a.nsplit == 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = qb * kQBlock + wave * 64 + j * 32 + l32;
    if (final_out) {
      if (row < a.Lq) {
        const float inv = 1.f / l[j];
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * H + h) * D;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * hf;
            __bf16 b0 = (__bf16)(o[dt][j][4 * g + 0] * inv), b1 = (__bf16)(o[dt][j][4 * g + 1] * inv);
            __bf16 b2 = (__bf16)(o[dt][j][4 * g + 2] * inv), b3 = (__bf16)(o[dt][j][4 * g + 3] * inv);
            uint2 w;
            w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
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
constexpr int kF32Rows = 256;

__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  constexpr int D = kHeadDim, P = kPage;
  __shared__ float sK[P][D + 1];
  __shared__ float sV[D][P + 1];
  int h, qb, s;
  decode_wg(a, h, qb, s);
  const int H = a.H;
  const int npg = a.pl.a_cnt + a.pl.s_cnt + a.pl.w_cnt;
  const int p0 = (int)((long long)npg * s / a.nsplit);
  const int p1 = (int)((long long)npg * (s + 1) / a.nsplit);
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
  const float* kpool = reinterpret_cast<const float*>(a.kpool);
  const float* vpool = reinterpret_cast<const float*>(a.vpool);
  for (int i = p0; i < p1; ++i) {
    int valid;
    const int pg = map_page_safe(a, i, valid);
    const size_t off = ((size_t)pg * H + h) * (P * D);
    __syncthreads();
    for (int e = threadIdx.x; e < P * D; e += 256) {
      sK[e / D][e % D] = kpool[off + e];
      sV[e / P][e % P] = vpool[off + e];
    }
    __syncthreads();
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

// Merge of the key splits: O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = exp2((m_s - max m) * scale * log2 e); LSE = scale * max m + ln(sum).
// Block = 16 query rows x 16 four-float chunks of one head.
template <bool kF32>
__global__ __launch_bounds__(256) void k_merge(AttnArgs a) {
  constexpr int D = kHeadDim;
  const int h = blockIdx.y;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int d4 = (threadIdx.x & 15) * 4;
  if (row >= a.Lq) return;
  const int ns = a.nsplit;
  const float2* ml = a.part_ml + (size_t)h * ns * a.Lq_pad + row;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[(size_t)s * a.Lq_pad].x);
  const float c2 = a.scale_log2;
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < ns; ++s) {
    const float2 v = ml[(size_t)s * a.Lq_pad];
    const float w = exp2f((v.x - M) * c2);
    L = __builtin_fmaf(w, v.y, L);
    const float4 po = *reinterpret_cast<const float4*>(
        a.part_o + (((size_t)h * ns + s) * a.Lq_pad + row) * D + d4);
    acc.x = __builtin_fmaf(w, po.x, acc.x);
    acc.y = __builtin_fmaf(w, po.y, acc.y);
    acc.z = __builtin_fmaf(w, po.z, acc.z);
    acc.w = __builtin_fmaf(w, po.w, acc.w);
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

hipError_t launch_alloc_frames(const LayerDev& L, int pool_pages, int ppf, int first_frame,
                               int nframes, hipStream_t st) {
  hipLaunchKernelGGL(k_alloc_frames, dim3(1), dim3(1024), 0, st, L, pool_pages, ppf,
                     first_frame, nframes);
  return hipGetLastError();
}

hipError_t launch_append(const LayerDev& L, const void* k, const void* v, int first_frame,
                         int nframes, int ppf, int F, int H, bool f32, hipStream_t st) {
  dim3 grid(nframes * ppf, H);
  if (f32)
    hipLaunchKernelGGL(k_append<float>, grid, dim3(256), 0, st, L, (const float*)k,
                       (const float*)v, first_frame, ppf, F, H);
  else
    hipLaunchKernelGGL(k_append<uint16_t>, grid, dim3(256), 0, st, L, (const uint16_t*)k,
                       (const uint16_t*)v, first_frame, ppf, F, H);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool f32, hipStream_t st) {
  const int grid = a.H * a.qblocks * a.nsplit;
  if (f32)
    hipLaunchKernelGGL(k_attn_f32, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_attn_bf16, dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, bool f32, hipStream_t st) {
  dim3 grid((a.Lq + 15) / 16, a.H);
  if (f32)
    hipLaunchKernelGGL(k_merge<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_merge<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_evict(const LayerDev& L, int pool_pages, int frame, int ppf, int S, int H,
                        bool f32, hipStream_t st) {
  if (f32)
    hipLaunchKernelGGL(k_evict<float>, dim3(1), dim3(256), 0, st, L, pool_pages, frame, ppf, S, H);
  else
    hipLaunchKernelGGL(k_evict<uint16_t>, dim3(1), dim3(256), 0, st, L, pool_pages, frame, ppf, S, H);
  return hipGetLastError();
}

}  // namespace gca
