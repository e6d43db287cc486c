// Measurement probes for the benchmark (not part of the attention library):
// the achievable HBM bandwidth of a plain copy, the achievable bf16 matrix-core
// rate of a loop of independent MFMAs, and the cost of an empty launch.  They
// give measured denominators beside the chip's published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sa_probe.h"

namespace {

constexpr int kThreads = 256;

// Grid-stride copy of n 16-byte words, one load and one store per lane per
// step, four workgroups per compute unit: of the plain copies measured on
// MI355X (one to eight words in flight per lane, 4 to 64 workgroups per
// compute unit, with and without non-temporal stores) the fastest.
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(uint4* __restrict__ dst,
                                                              const uint4* __restrict__ src, int64_t n) {
  const int64_t lanes = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += lanes) dst[i] = src[i];
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// kChains independent accumulator chains of v_mfma_f32_32x32x16_bf16 per
// wavefront, `iters` rounds: enough independent work that the matrix core's
// issue rate, not the chain latency, sets the pace.  One value per wavefront
// is stored so that nothing is optimised away.
constexpr int kChains = 4;
__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(seed * (float)(threadIdx.x + e));
    b[e] = static_cast<__bf16>(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

__global__ void probe_empty_kernel() {}

// Issue-rate probe: per round, NM v_mfma_f32_32x32x16_bf16 (two independent
// chains), NV v_fma_f32 and NE v_exp_f32 (16 independent chains each), all
// independent of each other, so the SIMD may overlap the matrix core with the
// vector ALU.  Each wavefront stores the ticks of s_memtime and of the
// constant-rate s_memrealtime its `iters` rounds took; with four wavefronts
// per SIMD (a grid of four workgroups per compute unit), time / iters is the
// SIMD time of one round of each of the four wavefronts.
template <int NM, int NV, int NE>
__global__ __launch_bounds__(kThreads) void probe_mix_kernel(float* out, int iters, float a, float b) {
  bf16x8 x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = static_cast<__bf16>(1e-3f * (float)(threadIdx.x + e));
    y[e] = static_cast<__bf16>(0.5f - 0.01f * (float)e);
  }
  f32x16 c0, c1;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = 0.f;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 1e-3f * (float)(threadIdx.x + i);
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < NM / 2; ++m) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < NV / 16; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], a, b);
#pragma unroll
    for (int r = 0; r < NE / 16; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_exp2f(v[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i] + c0[i] + c1[i];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    out[4 * w] = (float)(t1 - t0);
    out[4 * w + 1] = (float)(r1 - r0);
    out[4 * w + 2] = s;  // keeps the work
    out[4 * w + 3] = 0.f;
  }
}

struct MixVariant {
  int nm, nv, ne;
};
constexpr MixVariant kMix[] = {{8, 0, 0}, {0, 128, 0}, {8, 128, 0}, {0, 0, 32}, {8, 0, 32}};
constexpr int kNumMix = sizeof(kMix) / sizeof(kMix[0]);

}  // namespace

extern "C" int sa_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (dst == nullptr || src == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(dst) & 15u) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return 1;
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 256 * 4) blocks = 256 * 4;  // four workgroups per compute unit, then grid-stride
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int sa_probe_mfma_flops(int blocks, int iters, double* flops) {
  if (blocks < 1 || iters < 1 || flops == nullptr) return 1;
  *flops = (double)blocks * (kThreads / 64) * iters * kChains * (2.0 * 32 * 32 * 16);
  return 0;
}

extern "C" int sa_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     out, iters, 1e-3f);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int sa_probe_empty(void* stream) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int sa_probe_mix_variants(void) { return kNumMix; }

extern "C" int sa_probe_mix_counts(int variant, int* n_mfma, int* n_fma, int* n_exp) {
  if (variant < 0 || variant >= kNumMix || n_mfma == nullptr || n_fma == nullptr || n_exp == nullptr) return 1;
  *n_mfma = kMix[variant].nm;
  *n_fma = kMix[variant].nv;
  *n_exp = kMix[variant].ne;
  return 0;
}

extern "C" int sa_probe_mix(int variant, float* out, int blocks, int iters, void* stream) {
  if (variant < 0 || variant >= kNumMix || out == nullptr || blocks < 1 || iters < 1) return 1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(blocks), b(kThreads);
  switch (variant) {
    case 0: hipLaunchKernelGGL((probe_mix_kernel<8, 0, 0>), g, b, 0, st, out, iters, 0.999f, 0.5f); break;
    case 1: hipLaunchKernelGGL((probe_mix_kernel<0, 128, 0>), g, b, 0, st, out, iters, 0.999f, 0.5f); break;
    case 2: hipLaunchKernelGGL((probe_mix_kernel<8, 128, 0>), g, b, 0, st, out, iters, 0.999f, 0.5f); break;
    case 3: hipLaunchKernelGGL((probe_mix_kernel<0, 0, 32>), g, b, 0, st, out, iters, 0.999f, 0.5f); break;
    default: hipLaunchKernelGGL((probe_mix_kernel<8, 0, 32>), g, b, 0, st, out, iters, 0.999f, 0.5f); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
