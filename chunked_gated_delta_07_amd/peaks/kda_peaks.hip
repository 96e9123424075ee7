// kda_peaks.hip -- matrix-core and VALU microbenchmarks for the MI355X peaks
// (declared in include/kda_peaks.h).  gfx950 only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename V> __device__ __forceinline__ float first_sum(const V& v) { return v[0] + v[1]; }

template <int KIND>
__global__ __launch_bounds__(512) void kda_peaks_kernel(int iters, float* __restrict__ sink) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds at compile time
  const float x = 0.125f * (float)(tid & 7) + 0.5f;
  float out = 0.0f;
  // independent FMA chains (a x + b with |a| < 1 keeps them bounded)
  float v0 = x, v1 = x + 1.0f, v2 = x + 2.0f, v3 = x + 3.0f;
  float v4 = x + 4.0f, v5 = x + 5.0f, v6 = x + 6.0f, v7 = x + 7.0f;
  const float fa = 0.999f, fb = 0.001f * x;
  auto valu8 = [&] {
    v0 = fmaf(v0, fa, fb); v1 = fmaf(v1, fa, fb); v2 = fmaf(v2, fa, fb); v3 = fmaf(v3, fa, fb);
    v4 = fmaf(v4, fa, fb); v5 = fmaf(v5, fa, fb); v6 = fmaf(v6, fa, fb); v7 = fmaf(v7, fa, fb);
  };
  if constexpr (KIND == KDA_PEAK_MFMA_FP32) {
    const float a = x, b = 1.0f - x;
    f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c3, 0, 0, 0);
    }
    out = first_sum(c0) + first_sum(c1) + first_sum(c2) + first_sum(c3);
  } else if constexpr (KIND == KDA_PEAK_VALU) {
    for (int it = 0; it < iters; ++it) valu8();
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(x * (float)(i + 1) * 0.01f);
      b[i] = (__bf16)((1.0f - x) * (float)(8 - i) * 0.01f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      if constexpr (KIND == KDA_PEAK_MFMA_BF16) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      } else {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        if constexpr (KIND == KDA_PEAK_CHAIN_BF16_VALU) valu8();
      }
    }
    out = first_sum(c0) + first_sum(c1) + first_sum(c2) + first_sum(c3);
  }
  out += v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
  sink[(size_t)blockIdx.x * blockDim.x + tid] = out;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kda_peaks_copy_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  // four independent 16-byte loads in flight per thread, then their stores
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

template <int KIND>
int launch(int iters, int blocks, int threads, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL((kda_peaks_kernel<KIND>), dim3((unsigned)blocks), dim3((unsigned)threads), 0,
                     stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace

extern "C" KDA_PEAKS_API int kda_peaks_probe(int kind, int iters, int blocks, int threads,
                                             float* sink, hipStream_t stream) {
  if (iters < 1 || blocks < 1 || sink == nullptr) return 1;
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512) return 1;
  switch (kind) {
    case KDA_PEAK_MFMA_BF16: return launch<KDA_PEAK_MFMA_BF16>(iters, blocks, threads, sink, stream);
    case KDA_PEAK_MFMA_FP32: return launch<KDA_PEAK_MFMA_FP32>(iters, blocks, threads, sink, stream);
    case KDA_PEAK_CHAIN_BF16: return launch<KDA_PEAK_CHAIN_BF16>(iters, blocks, threads, sink, stream);
    case KDA_PEAK_CHAIN_BF16_VALU:
      return launch<KDA_PEAK_CHAIN_BF16_VALU>(iters, blocks, threads, sink, stream);
    case KDA_PEAK_VALU: return launch<KDA_PEAK_VALU>(iters, blocks, threads, sink, stream);
    default: return 1;
  }
}

extern "C" KDA_PEAKS_API int kda_peaks_copy(const void* src, void* dst, size_t bytes, int blocks,
                                            hipStream_t stream) {
  if (src == nullptr || dst == nullptr || blocks < 1 || bytes % 16 != 0) return 1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(kda_peaks_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
