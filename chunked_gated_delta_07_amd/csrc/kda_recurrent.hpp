// kda_recurrent.hpp -- token-serial KDA forward (the serving / decode form).
//
// The same operator as the chunked path, taken one token at a time with an
// FP32 state: the serving-side FP32 recurrence that xtuner PR #2301 compares
// its chunked training path against (sections Problem and Validation), with
// the start/end states of PR #2153's sequence-parallel hand-off.  Per head
// and token:
//   S <- Diag(a) S;   u = v - S^T k^;   S <- S + beta k^ u^T;   o = scale S^T q^
// with a = exp(g), g = -exp(A_log) softplus(f + dt_bias), beta = sigmoid(b),
// q^, k^ L2-normalised (eps 1e-6).  This is the form for decode steps and
// short sequences; long prefills belong to the chunked path.
//
// One workgroup of 128 threads per (sequence, head); thread j keeps column j
// of S (all 128 key channels, FP32) in registers for the whole sequence.  Per
// token the raw q, k and the decay a go to LDS (double-buffered, one barrier
// per token) and every thread reads them as broadcasts; the two norms come
// from a wave reduction plus one LDS exchange.  L2 normalisation is folded in
// as two scalars: S^T k^ = rk S^T k and k^ u^T = rk k u^T.
#pragma once

#include "kda_common.hpp"

namespace kda {

struct RecArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* f;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu;
  const float* init;  // [N][H][128][128] or null
  float* fin;         // [N][H][128][128] or null
  void* out;          // [T][H][128]
  int N;
  int H;
  float eps;
  float scale;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <typename TA, typename TO>
__global__ __launch_bounds__(128) void kda_recurrent_kernel(RecArgs p) {
  // [buffer][q | k | a][128] plus the two waves' partial sums of q^2, k^2
  __shared__ __attribute__((aligned(16))) float vec[2][3][DH];
  __shared__ float part[2][2][2];
  const int pair = blockIdx.x;  // sequence * H + head
  const int n = pair / p.H, h = pair - n * p.H;
  const int j = threadIdx.x, w = j >> 6;
  const TA* __restrict__ gq = reinterpret_cast<const TA*>(p.q);
  const TA* __restrict__ gk = reinterpret_cast<const TA*>(p.k);
  const TA* __restrict__ gv = reinterpret_cast<const TA*>(p.v);
  const TA* __restrict__ gf = reinterpret_cast<const TA*>(p.f);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
  const float lam = expf(p.A_log[h]);  // exp(-inf) = 0: no decay
  const float dtb = p.dt_bias[(size_t)h * DH + j];
  // column j of S: S[i][j], i = key channel
  const size_t sbase = (size_t)pair * DH * DH + j;
  float S[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) S[i] = p.init ? p.init[sbase + (size_t)i * DH] : 0.0f;
  const int t0 = p.cu[n], t1 = p.cu[n + 1];
  int buf = 0;
  for (int t = t0; t < t1; ++t) {
    const size_t o = ((size_t)t * p.H + h) * DH + j;
    const float qj = to_f32(gq[o]), kj = to_f32(gk[o]), vj = to_f32(gv[o]);
    const float aj = decay_from_gate(to_f32(gf[o]) + dtb, lam);
    const float beta = sigmoid_f(to_f32(gb[(size_t)t * p.H + h]));
    const float sq = wave_sum(qj * qj), sk = wave_sum(kj * kj);
    vec[buf][0][j] = qj;
    vec[buf][1][j] = kj;
    vec[buf][2][j] = aj;
    if ((j & 63) == 0) { part[buf][w][0] = sq; part[buf][w][1] = sk; }
    __syncthreads();  // (double buffers: the next token writes the other set)
    const float rq = rsqrt_hw(part[buf][0][0] + part[buf][1][0] + p.eps);
    const float rk = rsqrt_hw(part[buf][0][1] + part[buf][1][1] + p.eps);
    const f32x4* vq = reinterpret_cast<const f32x4*>(vec[buf][0]);
    const f32x4* vk = reinterpret_cast<const f32x4*>(vec[buf][1]);
    const f32x4* va = reinterpret_cast<const f32x4*>(vec[buf][2]);
    // decay, then (S^T k)_j on the decayed state
    float dot0 = 0.0f, dot1 = 0.0f;
#pragma unroll
    for (int i4 = 0; i4 < DH / 4; ++i4) {
      const f32x4 a4 = va[i4], k4 = vk[i4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[4 * i4 + e] *= a4[e];
        if (e & 1) dot1 = fmaf(S[4 * i4 + e], k4[e], dot1);
        else dot0 = fmaf(S[4 * i4 + e], k4[e], dot0);
      }
    }
    const float bu = beta * rk * (vj - rk * (dot0 + dot1));
    // S += beta k^ u^T, then o_j = (S^T q^)_j
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int i4 = 0; i4 < DH / 4; ++i4) {
      const f32x4 k4 = vk[i4], q4 = vq[i4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[4 * i4 + e] = fmaf(k4[e], bu, S[4 * i4 + e]);
        if (e & 1) o1 = fmaf(S[4 * i4 + e], q4[e], o1);
        else o0 = fmaf(S[4 * i4 + e], q4[e], o0);
      }
    }
    out[o] = from_f32<TO>(p.scale * rq * (o0 + o1));
    buf ^= 1;
  }
  if (p.fin) {
#pragma unroll
    for (int i = 0; i < DH; ++i) p.fin[sbase + (size_t)i * DH] = S[i];
  }
}

}  // namespace kda
