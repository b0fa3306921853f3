// Issue rates of the softmax's VALU instructions on gfx950, alone and beside
// MFMAs (a diagnostic executable, not part of the library).
//
// Each workgroup has 512 threads, two waves per SIMD.  Waves 0-3 issue
// v_mfma_f32_32x32x16_bf16 back to back on four independent accumulators;
// waves 4-7 issue one kind of VALU instruction on eight independent chains.
// Each wave times its own loop with s_memtime (shader cycles).  Three modes
// per kind: MFMAs alone, the VALU stream alone, both together.  The program
// prints cycles per MFMA and per VALU instruction, averaged over all waves
// of 256 workgroups.  The attention kernel's page loop pairs the waves the
// same way (one wave's MFMAs beside the other wave's softmax).  The last
// kinds are sequences for two scores of a softmax, reported per pair:
// two exponentials and their bf16 pack, then the row sum either by v_dot2
// over the packed pair (the attention kernel's sequence), by two v_add_f32 of
// the fp32 values, or not at all.
//
// Build: python -m geometric_context_attention_amd.build --probe
// Run:   geometric_context_attention_amd/issue_rate_probe
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlocks = 256, kThreads = 512, kIters = 2000;
constexpr int kChains = 8, kUnroll = 4;  // VALU instructions per loop iteration: 32

enum Kind { kExp, kFma, kAdd, kDot2, kCvtPk, kMixDot2, kMixAdd, kMixNoSum, kKinds };
constexpr int kFirstMix = kMixDot2;
const char* const kNames[kKinds] = {"v_exp_f32", "v_fma_f32", "v_add_f32", "v_dot2c_f32_bf16",
                                    "v_cvt_pk_bf16_f32", "pair: exp, exp, cvt_pk, dot2",
                                    "pair: exp, exp, cvt_pk, add, add", "pair: exp, exp, cvt_pk"};

template <int K>
__device__ __forceinline__ float valu_op(float x, float seed, bf16x2 v) {
  if constexpr (K == kExp) return __builtin_amdgcn_exp2f(x);
  if constexpr (K == kFma) return __builtin_fmaf(x, seed, 0.5f);
  if constexpr (K == kAdd) return x + seed;
  if constexpr (K == kDot2) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(v, ones, x, false);
  }
  const bf16x2 t = {(__bf16)x, (__bf16)x};
  return __builtin_bit_cast(float, t);
}

// mode bit 0: waves 0-3 issue MFMAs; bit 1: waves 4-7 issue the VALU stream
template <int K>
__global__ __launch_bounds__(kThreads) void probe(unsigned long long* cycles, int mode, float seed) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  float sink = 0.f;
  if (wave < 4) {
    if (mode & 1) {
      bf16x8 a, b;
      for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(seed * (lane + e));
        b[e] = (__bf16)(seed * (lane - e));
      }
      f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int i = 0; i < kIters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
      sink = c0[0] + c1[1] + c2[2] + c3[3];
    }
  } else if (mode & 2) {
    float acc[kChains];
    for (int k = 0; k < kChains; ++k) acc[k] = seed * (lane + k);
    const bf16x2 v = {(__bf16)(seed * lane), (__bf16)(seed * 2.f)};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float sc[16];  // the mix's scores: opaque to the compiler on every iteration
    for (int k = 0; k < 16; ++k) sc[k] = -seed * (lane + k);
    for (int i = 0; i < kIters; ++i) {
      if constexpr (K >= kFirstMix) {
#pragma unroll
        for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(sc[k]));
        // 8 pairs per iteration
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float e0 = __builtin_amdgcn_exp2f(sc[2 * c]), e1 = __builtin_amdgcn_exp2f(sc[2 * c + 1]);
          const bf16x2 p = {(__bf16)e0, (__bf16)e1};
          if constexpr (K == kMixDot2) acc[c % kChains] = __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc[c % kChains], false);
          if constexpr (K == kMixAdd) {
            acc[c % kChains] += e0;
            acc[(c + 4) % kChains] += e1;
          }
          if constexpr (K != kMixDot2) {  // the pack is kept (the MFMA would read it)
            float w = __builtin_bit_cast(float, p);
            asm volatile("" : "+v"(w));
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int k = 0; k < kChains; ++k) acc[k] = valu_op<K>(acc[k], seed, v);
      }
      // one loop iteration issues exactly kChains * kUnroll of them
#pragma unroll
      for (int k = 0; k < kChains; ++k) asm volatile("" : "+v"(acc[k]));
    }
    for (int k = 0; k < kChains; ++k) sink += acc[k];
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  // sink keeps the loops alive; it never equals the sentinel
  if (lane == 0) cycles[blockIdx.x * 8 + wave] = (t1 - t0) + (sink == -12345.f ? 1 : 0);
}

template <int K>
bool launch(unsigned long long* d, int mode) {
  hipLaunchKernelGGL(probe<K>, dim3(kBlocks), dim3(kThreads), 0, 0, d, mode, 1e-3f);
  return hipDeviceSynchronize() == hipSuccess;
}

bool run(int kind, int mode, unsigned long long* d) {
  switch (kind) {
    case kExp: return launch<kExp>(d, mode);
    case kFma: return launch<kFma>(d, mode);
    case kAdd: return launch<kAdd>(d, mode);
    case kDot2: return launch<kDot2>(d, mode);
    case kCvtPk: return launch<kCvtPk>(d, mode);
    case kMixDot2: return launch<kMixDot2>(d, mode);
    case kMixAdd: return launch<kMixAdd>(d, mode);
    default: return launch<kMixNoSum>(d, mode);
  }
}

}  // namespace

int main() {
  unsigned long long* d = nullptr;
  const size_t n = (size_t)kBlocks * 8;
  if (hipMalloc(&d, n * sizeof(unsigned long long)) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  std::vector<unsigned long long> h(n);
  auto mean = [&](int w0) {
    double s = 0;
    for (int b = 0; b < kBlocks; ++b)
      for (int w = w0; w < w0 + 4; ++w) s += (double)h[(size_t)b * 8 + w];
    return s / (kBlocks * 4.0);
  };
  // the first launch warms the clock up and is not reported
  if (!run(kExp, 3, d)) return 1;
  printf("instruction or pair | alone (cycles) | beside MFMAs (cycles) | MFMA beside it (cycles/MFMA)\n");
  for (int kind = 0; kind < kKinds; ++kind) {
    double alone = 0, beside = 0, mfma = 0;
    // single instructions: 32 per iteration; sequences: 8 pairs per iteration
    const double per = kind >= kFirstMix ? kIters * 8.0 : kIters * (double)(kChains * kUnroll);
    if (!run(kind, 2, d) || hipMemcpy(h.data(), d, n * sizeof(h[0]), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    alone = mean(4) / per;
    if (!run(kind, 3, d) || hipMemcpy(h.data(), d, n * sizeof(h[0]), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    beside = mean(4) / per;
    mfma = mean(0) / (kIters * 4.0);
    printf("%s | %.2f | %.2f | %.1f\n", kNames[kind], alone, beside, mfma);
  }
  if (!run(kExp, 1, d) || hipMemcpy(h.data(), d, n * sizeof(h[0]), hipMemcpyDeviceToHost) != hipSuccess) return 1;
  printf("MFMAs alone | %.1f cycles/MFMA\n", mean(0) / (kIters * 4.0));
  return hipFree(d) == hipSuccess ? 0 : 1;
}
