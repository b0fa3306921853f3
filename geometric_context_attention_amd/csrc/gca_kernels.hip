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
// Pages of the frame being appended are read from k_in / v_in, staged like any
// page, and written to their pool pages by the query-block-0 workgroups.
__global__ __launch_bounds__(512, 1) void k_attn_bf16(AttnArgs a) {
  constexpr int D = kHeadDim, P = kPage, LR = 72;  // LDS row: 64 bf16 + 8 pad
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][P * LR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * LR];

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

  uint16_t* kpool = reinterpret_cast<uint16_t*>(a.kpool);
  uint16_t* vpool = reinterpret_cast<uint16_t*>(a.vpool);
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(a.k_in);
  const uint16_t* vin = reinterpret_cast<const uint16_t*>(a.v_in);
  const int ld_row = tid >> 3, ld_ch = tid & 7;  // 512 threads x 16 B = one 8 KB tile

  // global -> registers for logical page i
  auto load_page = [&](int i, uint4& kv, uint4& vv, int& valid, int& fj, size_t& off) {
    const int pg = map_page(a, i, valid, fj);
    off = ((size_t)pg * H + h) * (P * D);
    if (fj < 0) {
      kv = *reinterpret_cast<const uint4*>(kpool + off + tid * 8);
      vv = *reinterpret_cast<const uint4*>(vpool + off + tid * 8);
      if (valid < P) vv = mask_vt_chunk(vv, ld_ch, valid);
    } else {
      kv = make_uint4(0u, 0u, 0u, 0u);
      vv = kv;
      if (ld_row < valid) {
        const size_t src = ((size_t)(fj * P + ld_row) * H + h) * D + ld_ch * 8;
        kv = *reinterpret_cast<const uint4*>(kin + src);
        vv = *reinterpret_cast<const uint4*>(vin + src);
      }
      if (qb == 0) *reinterpret_cast<uint4*>(kpool + off + tid * 8) = kv;
    }
  };
  // registers -> LDS buffer b (V of a fresh page is transposed on the way)
  auto store_page = [&](int b, const uint4& kv, const uint4& vv, int fj) {
    *reinterpret_cast<uint4*>(&sK[b][ld_row * LR + ld_ch * 8]) = kv;
    if (fj < 0) {
      *reinterpret_cast<uint4*>(&sV[b][ld_row * LR + ld_ch * 8]) = vv;
    } else {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
      const int col = swap23(ld_row);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sV[b][(ld_ch * 8 + e) * LR + col] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
  };

  int valid_cur = P, fj_cur = -1;
  size_t off_cur = 0;
  if (p0 < p1) {
    uint4 kv, vv;
    load_page(p0, kv, vv, valid_cur, fj_cur, off_cur);
    store_page(0, kv, vv, fj_cur);
  }
  __syncthreads();

  for (int i = p0; i < p1; ++i) {
    const int buf = (i - p0) & 1;
    // prefetch page i+1 into registers
    uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
    int valid_next = P, fj_next = -1;
    size_t off_next = 0;
    const bool has_next = i + 1 < p1;
    if (has_next) load_page(i + 1, kn, vn, valid_next, fj_next, off_next);
    // a fresh page just staged: its transposed V tile goes to the pool
    if (fj_cur >= 0 && qb == 0)
      *reinterpret_cast<uint4*>(vpool + off_cur + tid * 8) =
          *reinterpret_cast<const uint4*>(&sV[buf][ld_row * LR + ld_ch * 8]);

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

    if (has_next) store_page(buf ^ 1, kn, vn, fj_next);
    valid_cur = valid_next;
    fj_cur = fj_next;
    off_cur = off_next;
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
    hipLaunchKernelGGL(k_attn_bf16, dim3(grid), dim3(512), 0, st, a);
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
