// kda_common.hpp -- device-side building blocks shared by the libkda kernels.
//
// gfx950 (CDNA4) only.  Wave size is 64.  Matrix products use the MFMA
// instructions below; their lane layouts (checked on the hardware) are:
//   v_mfma_f32_16x16x32_bf16 : A[m][k] in lane m%16 + 16*(k/8), element k%8;
//                              B[k][n] in lane n + 16*(k/8); C[m][n] in lane
//                              n + 16*(m/4), element m%4.
//   v_mfma_f32_32x32x16_bf16 : A[m][k] in lane m + 32*(k/8); B[k][n] in lane
//                              n + 32*(k/8); C[m][n] in lane n + 32*((m/4)%2),
//                              element 4*(m/8) + m%4.
//   v_mfma_f32_16x16x4f32    : A[m][k] in lane m + 16*k; B[k][n] in lane n + 16*k.
//   v_mfma_f32_32x32x2f32    : A[m][k] in lane m + 32*k; B[k][n] in lane n + 32*k.
// Any permutation of the contracted index k that is applied identically to A
// and B leaves a product unchanged; the kernels use that to let every lane
// read one contiguous run of memory per operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int CHUNK = 64;   // tokens per chunk
constexpr int DH = 128;     // head dimension (d_k = d_v)
constexpr int WAVE = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Two consecutive elements -> float2.
__device__ __forceinline__ f32x2 load2(const bf16* p) {
  bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
  return f32x2{(float)v[0], (float)v[1]};
}
__device__ __forceinline__ f32x2 load2(const float* p) { return *reinterpret_cast<const f32x2*>(p); }

__device__ __forceinline__ void store2(bf16* p, float a, float b) {
  *reinterpret_cast<bf16x2*>(p) = bf16x2{(bf16)a, (bf16)b};
}
__device__ __forceinline__ void store2(float* p, float a, float b) {
  *reinterpret_cast<f32x2*>(p) = f32x2{a, b};
}
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// ---------------------------------------------------------------- MFMA tiles
// A 16x16 output tile accumulated over K, for element type MT.  K-steps:
// bf16 contracts 32 per instruction (8 per lane), f32 contracts 4 (1 per lane).
template <typename MT> struct Mma16;

template <> struct Mma16<bf16> {
  static constexpr int KPI = 32;  // contracted elements per instruction
  static constexpr int PER_LANE = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma16<float> {
  static constexpr int KPI = 4;
  static constexpr int PER_LANE = 1;
  typedef float frag;
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// C[16][16] += A[16][K] * B[K][16] where A rows and B columns are both stored
// as rows of K contiguous elements ("row-of-K" layout): A row m at a + m*lda,
// B column n at b + n*ldb.  Lane l reads row (l%16) and contracts over the
// K-range [g*K/4, (g+1)*K/4) with g = l/16, so every lane reads one
// contiguous run from each operand.
template <typename MT, int K>
__device__ __forceinline__ f32x4 mma16_rows(const MT* a, int lda, const MT* b, int ldb, f32x4 c,
                                            int lane) {
  typedef Mma16<MT> M;
  constexpr int KG = K / 4;                       // contracted range per lane group
  const int r = lane & 15, g = lane >> 4;
  const MT* pa = a + r * lda + g * KG;
  const MT* pb = b + r * ldb + g * KG;
  if constexpr (M::PER_LANE == 8) {
#pragma unroll
    for (int s = 0; s < KG / 8; ++s) c = M::mma(M::load(pa + 8 * s), M::load(pb + 8 * s), c);
  } else {
    // fp32: one 16-byte read per operand feeds four instructions
#pragma unroll 2
    for (int s = 0; s < KG / 4; ++s) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(pa + 4 * s);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(pb + 4 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) c = M::mma(a4[e], b4[e], c);
    }
  }
  return c;
}

// fp32 C[16][16] += A[16][K] * B[K][16], A row-major (lda), B k-major
// (B[k][n] at b + k*ldb + n).  K multiple of 4.
template <int K>
__device__ __forceinline__ f32x4 mma16_f32_kn(const float* a, int lda, const float* b, int ldb,
                                              f32x4 c, int lane) {
  constexpr int KG = K / 4;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < KG; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * lda + g * KG + s], b[(g * KG + s) * ldb + r], c,
                                             0, 0, 0);
  return c;
}

// fp32 C[16][16] += A[16][K] * B[K][16] with A supplied transposed
// (A[m][k] at at + k*ldat + m) and B k-major.  K multiple of 4.
template <int K>
__device__ __forceinline__ f32x4 mma16_f32_tn(const float* at, int ldat, const float* b, int ldb,
                                              f32x4 c, int lane) {
  constexpr int KG = K / 4;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < KG; ++s) {
    const int kk = g * KG + s;
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(at[kk * ldat + r], b[kk * ldb + r], c, 0, 0, 0);
  }
  return c;
}

// 32x32 tiles for the state pass.
template <typename MT> struct Mma32;
template <> struct Mma32<bf16> {
  static constexpr int PER_LANE = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma32<float> {
  static constexpr int PER_LANE = 1;
  typedef float frag;
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Accumulator element e of a 32x32 tile holds row (row32(e, lane)), column lane%32.
__device__ __forceinline__ int row32(int e, int lane) { return 8 * (e >> 2) + 4 * ((lane >> 5) & 1) + (e & 3); }

// ---------------------------------------------------------------- math
// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32, about 1 ulp).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
constexpr float LOG2E = 1.4426950408889634f;

// Per-token decay a = exp(g), g = -lam * softplus(x), computed in base 2:
//   softplus(x) log2(e) = max(x,0) log2(e) + log2(1 + 2^(-|x| log2 e)).
// Only the absolute error of g matters (it is the relative error of a); the
// log2(1 + t) form has absolute error ~1e-7 for every x.  lam = 0 gives a = 1.
__device__ __forceinline__ float decay_from_gate(float x, float lam) {
  const float t = exp2_hw(-fabsf(x) * LOG2E);
  const float sp2 = fmaxf(x, 0.0f) * LOG2E + log2_hw(1.0f + t);
  return exp2_hw(-lam * sp2);
}
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_hw(-x * LOG2E));
}
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}


// ---------------------------------------------------------------- split products
// FP32 operands on bf16 matrix cores.  Each FP32 value x is split into three
// bf16 pieces x = h + m + l: h is x rounded to nearest even, m the same for
// x - h, l for x - h - m (both remainders are exact in FP32, and for a normal
// x the three pieces hold all 24 significand bits, so the split is exact).  A
// product x y is the sum of the six piece products of order >= 2^-16,
//   h h' + (h m' + m h') + (h l' + m m' + l h'),
// the "bf16x6" scheme of Henry, Tang and Heinecke ("Leveraging the bfloat16
// artificial intelligence datatype for higher-precision computations", ARITH
// 2019).  The omitted terms m l' + l m' + l l' stay below 2^-23 |x y| and the
// matrix core accumulates in FP32, so a contraction agrees with an FP32 one to
// within FP32 rounding.  Cost per 16 contracted values of a 32x32 tile: six
// v_mfma_f32_32x32x16_bf16 (32 cycles each) instead of eight
// v_mfma_f32_32x32x2f32 (64 cycles each).  A factor exact in bf16 (one piece)
// needs only the three products with the other factor's pieces.
typedef unsigned u32;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// the two bf16 of a packed pair as FP32 (exact)
__device__ __forceinline__ f32x2 bf16x2_as_f32(u32 v) {
  return f32x2{__builtin_bit_cast(float, v << 16), __builtin_bit_cast(float, v & 0xffff0000u)};
}
__device__ __forceinline__ u32 cvt_pair(f32x2 x) {
  return __builtin_bit_cast(u32, __builtin_convertvector(x, bf16x2));  // RNE, one instruction
}
// pieces of two FP32 values, each piece packed as a bf16 pair
struct Pieces2 { u32 h, m, l; };
__device__ __forceinline__ Pieces2 split2(f32x2 x) {
  Pieces2 o;
  o.h = cvt_pair(x);
  const f32x2 r = x - bf16x2_as_f32(o.h);
  o.m = cvt_pair(r);
  o.l = cvt_pair(r - bf16x2_as_f32(o.m));
  return o;
}
// four FP32 values -> their pieces at p, p + stride, p + 2 stride
__device__ __forceinline__ void store_pieces4(bf16* p, int stride, const f32x4& v) {
  const Pieces2 p0 = split2(f32x2{v[0], v[1]}), p1 = split2(f32x2{v[2], v[3]});
  *reinterpret_cast<u32x2*>(p) = u32x2{p0.h, p1.h};
  *reinterpret_cast<u32x2*>(p + stride) = u32x2{p0.m, p1.m};
  *reinterpret_cast<u32x2*>(p + 2 * stride) = u32x2{p0.l, p1.l};
}
// pieces of eight FP32 values (a then b), one bf16x8 per piece
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8 (&o)[3]) {
  const Pieces2 p0 = split2(f32x2{a[0], a[1]}), p1 = split2(f32x2{a[2], a[3]});
  const Pieces2 p2 = split2(f32x2{b[0], b[1]}), p3 = split2(f32x2{b[2], b[3]});
  o[0] = __builtin_bit_cast(bf16x8, u32x4{p0.h, p1.h, p2.h, p3.h});
  o[1] = __builtin_bit_cast(bf16x8, u32x4{p0.m, p1.m, p2.m, p3.m});
  o[2] = __builtin_bit_cast(bf16x8, u32x4{p0.l, p1.l, p2.l, p3.l});
}
// C += A B over 32 contracted values, A exact in bf16 (one piece), B as its
// three pieces (smallest terms first)
__device__ __forceinline__ f32x4 mma_x3(const bf16x8& a, const bf16x8 (&b)[3], f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], c, 0, 0, 0);
}
// C += A B over 32 contracted values from the pieces of both (the six terms
// of order >= 2^-16, smallest first)
__device__ __forceinline__ f32x4 mma_x6_16(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[1], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[0], c, 0, 0, 0);
}

// C += A B over 32 contracted values, A as its three pieces, B exact in bf16
__device__ __forceinline__ f32x4 mma_x3b(const bf16x8 (&a)[3], const bf16x8& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b, c, 0, 0, 0);
}

}  // namespace kda
