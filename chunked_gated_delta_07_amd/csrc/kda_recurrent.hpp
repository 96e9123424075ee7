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
// One workgroup per (sequence, head), one thread per value channel (rounded up
// to whole waves, at least as many as key channels); thread j keeps column j
// of S (all d_k key channels, FP32) in registers for the whole sequence.  Per
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
  const float* init;  // [N][H][dk][dv] or null
  float* fin;         // [N][H][dk][dv] or null
  void* out;          // [T][H][dv]
  int N;
  int H;
  int dv;             // value channels (<= blockDim.x)
  float eps;
  float scale;
};

// DK key channels (q, k, f, dt_bias rows; state rows), p.dv value channels
// (v, out rows; state columns).  blockDim.x >= max(DK, dv), a multiple of 64,
// at most rec_max_threads(DK): a 128-entry state column needs more than the
// 256 registers a wave gets when four waves share a SIMD.
constexpr int REC_MAX_WAVES = 8;
__host__ __device__ constexpr int rec_max_threads(int dk) { return dk >= 128 ? 128 : 64 * REC_MAX_WAVES; }
template <typename TA, typename TO, int DK>
__global__ __launch_bounds__(rec_max_threads(DK)) void kda_recurrent_kernel(RecArgs p) {
  // [buffer][q | k | a][DK] plus each wave's partial sums of q^2, k^2
  __shared__ __attribute__((aligned(16))) float vec[2][3][DK];
  __shared__ float part[2][REC_MAX_WAVES][2];
  const int pair = blockIdx.x;  // sequence * H + head
  const int n = pair / p.H, h = pair - n * p.H;
  const int j = threadIdx.x, w = j >> 6, nw = blockDim.x >> 6;
  const int dv = p.dv;
  const bool key = j < DK, col = j < dv;
  const TA* __restrict__ gq = reinterpret_cast<const TA*>(p.q);
  const TA* __restrict__ gk = reinterpret_cast<const TA*>(p.k);
  const TA* __restrict__ gv = reinterpret_cast<const TA*>(p.v);
  const TA* __restrict__ gf = reinterpret_cast<const TA*>(p.f);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
  const float lam = expf(p.A_log[h]);  // exp(-inf) = 0: no decay
  const float dtb = key ? p.dt_bias[(size_t)h * DK + j] : 0.0f;
  // column j of S: S[i][j], i = key channel
  const size_t sbase = (size_t)pair * DK * dv + j;
  float S[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) S[i] = (p.init && col) ? p.init[sbase + (size_t)i * dv] : 0.0f;
  const int t0 = p.cu[n], t1 = p.cu[n + 1];
  int buf = 0;
  for (int t = t0; t < t1; ++t) {
    const size_t ok = ((size_t)t * p.H + h) * DK + j;
    const size_t ov = ((size_t)t * p.H + h) * dv + j;
    const float qj = key ? to_f32(gq[ok]) : 0.0f, kj = key ? to_f32(gk[ok]) : 0.0f;
    const float aj = key ? decay_from_gate(to_f32(gf[ok]) + dtb, lam) : 1.0f;
    const float vj = col ? to_f32(gv[ov]) : 0.0f;
    const float beta = sigmoid_f(to_f32(gb[(size_t)t * p.H + h]));
    const float sq = wave_sum(qj * qj), sk = wave_sum(kj * kj);
    if (key) {
      vec[buf][0][j] = qj;
      vec[buf][1][j] = kj;
      vec[buf][2][j] = aj;
    }
    if ((j & 63) == 0) { part[buf][w][0] = sq; part[buf][w][1] = sk; }
    __syncthreads();  // (double buffers: the next token writes the other set)
    float tq = 0.0f, tk = 0.0f;
    for (int x = 0; x < nw; ++x) { tq += part[buf][x][0]; tk += part[buf][x][1]; }
    const float rq = rsqrt_hw(tq + p.eps), rk = rsqrt_hw(tk + p.eps);
    if (col) {
      const f32x4* vq = reinterpret_cast<const f32x4*>(vec[buf][0]);
      const f32x4* vk = reinterpret_cast<const f32x4*>(vec[buf][1]);
      const f32x4* va = reinterpret_cast<const f32x4*>(vec[buf][2]);
      // decay, then (S^T k)_j on the decayed state
      float dot0 = 0.0f, dot1 = 0.0f;
#pragma unroll
      for (int i4 = 0; i4 < DK / 4; ++i4) {
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
      for (int i4 = 0; i4 < DK / 4; ++i4) {
        const f32x4 k4 = vk[i4], q4 = vq[i4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          S[4 * i4 + e] = fmaf(k4[e], bu, S[4 * i4 + e]);
          if (e & 1) o1 = fmaf(S[4 * i4 + e], q4[e], o1);
          else o0 = fmaf(S[4 * i4 + e], q4[e], o0);
        }
      }
      out[ov] = from_f32<TO>(p.scale * rq * (o0 + o1));
    }
    buf ^= 1;
  }
  if (p.fin && col) {
#pragma unroll
    for (int i = 0; i < DK; ++i) p.fin[sbase + (size_t)i * dv] = S[i];
  }
}

}  // namespace kda
