// kda_conv_bwd.hpp -- backward of the short causal convolution fused in front
// of the core (kda_chunk_fwd_conv): q, k and v each pass through their own
// depthwise causal convolution of width 4, the KDA module's q/k/v
// convolutions with FP32 master parameters (xtuner PR #2153, KDA module
// description), whose weight and bias gradients stay FP32.
//
// Per tensor, head and channel, with x the raw input, y = act(z) the
// convolution output (rounded to the activation dtype in the forward; the
// backward takes that rounding as the identity) and dy = dL/dy from the
// core's backward:
//   z_t  = b + sum_i w_i x_{t-3+i}                 (x = 0 before the sequence start)
//   dz_t = dy_t act'(z_t),   act'(z) = s (1 + z (1 - s)), s = sigmoid(z) (SiLU), else 1
//   dx_u = sum_i w_i dz_{u+3-i}                    (tokens of the same sequence)
//   dw_i = sum_t dz_t x_{t-3+i},   db = sum_t dz_t  (over every sequence)
// Three kernels: the convolution outputs (for the core's backward), the
// input gradients with per-chunk tap and bias partial sums, and the reduction
// of the partials in chunk order (deterministic).
#pragma once

#include "kda_common.hpp"
#include "kda_intra.hpp"

namespace kda {

struct ConvBwdArgs {
  const int32_t* cu;
  const int32_t* cfirst;  // [N+1] (always built here)
  int N;
  int H;
  const void* x[3];   // raw q, k, v [T][H][128], activation dtype
  void* y[3];         // convolution outputs [T][H][128], activation dtype
  const float* dy[3]; // dL/dy [T][H][128] FP32
  void* dx[3];        // dL/dx [T][H][128], gradient dtype
  const float* w;     // [3][H*128][4]
  const float* b;     // [3][H*128] or null
  int silu;
  float* part;        // [chunks][3][H][128][5]: tap and bias partial sums
  float* dw;          // [3][H*128][4]
  float* db;          // [3][H*128] or null (not written)
};

// Chunk c -> first token, length, sequence start and end (cfirst non-null).
__device__ __forceinline__ bool conv_chunk(const ConvBwdArgs& a, int c, int& t0, int& len,
                                           int& tseq, int& tend) {
  if (c >= a.cfirst[a.N]) return false;
  int lo = 0, hi = a.N;  // cfirst[lo] <= c < cfirst[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cfirst[mid] <= c) lo = mid; else hi = mid;
  }
  tseq = a.cu[lo];
  tend = a.cu[lo + 1];
  t0 = tseq + (c - a.cfirst[lo]) * CHUNK;
  len = min(CHUNK, tend - t0);
  return true;
}

// Four consecutive channels per thread: 8-byte (bf16) or 16-byte (FP32)
// accesses.  Grid (chunks, ceil(H / 8), 3 tensors) of 256 threads: thread t
// takes head 8 blockIdx.y + t / 32, channels 4 (t % 32) .. 4 (t % 32) + 3.
constexpr int CONV_CPT = 4;
constexpr int CONV_HEADS_PER_BLOCK = 256 / (DH / CONV_CPT);  // 8

__device__ __forceinline__ f32x4 ld4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Weights and bias of four channels, rounded to the activation dtype as the
// forward applies them.
template <typename TA>
__device__ __forceinline__ void conv_params4(const ConvBwdArgs& a, int tensor, size_t ch, float (&w)[4][4],
                                             float (&bias)[4]) {
  const size_t HD = (size_t)a.H * DH;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float* wt = a.w + (tensor * HD + ch + j) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[j][i] = to_f32(from_f32<TA>(wt[i]));
    bias[j] = a.b ? to_f32(from_f32<TA>(a.b[tensor * HD + ch + j])) : 0.0f;
  }
}

// Pre-activation of token t from the three tokens before it (h0 oldest) and
// its own input: the forward's order of operations.
__device__ __forceinline__ float conv_z(const float (&w)[4], float bias, float h0, float h1, float h2,
                                        float xt) {
  float acc = bias;
  acc = fmaf(w[0], h0, acc);
  acc = fmaf(w[1], h1, acc);
  acc = fmaf(w[2], h2, acc);
  return fmaf(w[3], xt, acc);
}

// Thread's (head, first channel) or false past the last head.
__device__ __forceinline__ bool conv_lane(const ConvBwdArgs& a, int& h, size_t& ch) {
  h = (int)blockIdx.y * CONV_HEADS_PER_BLOCK + (int)threadIdx.x / (DH / CONV_CPT);
  ch = (size_t)h * DH + CONV_CPT * (threadIdx.x % (DH / CONV_CPT));
  return h < a.H;
}

// The convolution outputs y (what the fused forward feeds the core).
template <typename TA>
__global__ __launch_bounds__(256) void kda_conv_apply_kernel(ConvBwdArgs a) {
  const int c = (int)blockIdx.x, tensor = (int)blockIdx.z;
  int h, t0, len, tseq, tend;
  size_t ch;
  if (!conv_lane(a, h, ch) || !conv_chunk(a, c, t0, len, tseq, tend)) return;
  const size_t HD = (size_t)a.H * DH;
  const TA* x = reinterpret_cast<const TA*>(a.x[tensor]);
  TA* y = reinterpret_cast<TA*>(a.y[tensor]);
  float w[4][4], bias[4];
  conv_params4<TA>(a, tensor, ch, w, bias);
  auto xat = [&](int t) { return t >= tseq ? ld4(x + (size_t)t * HD + ch) : f32x4{0, 0, 0, 0}; };
  f32x4 h0 = xat(t0 - 3), h1 = xat(t0 - 2), h2 = xat(t0 - 1);
  for (int t = t0; t < t0 + len; ++t) {
    const f32x4 xt = ld4(x + (size_t)t * HD + ch);
    f32x4 yv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float z = conv_z(w[j], bias[j], h0[j], h1[j], h2[j], xt[j]);
      if (a.silu) z *= sigmoid_f(z);
      yv[j] = z;
    }
    store4(y + (size_t)t * HD + ch, yv);
    h0 = h1; h1 = h2; h2 = xt;
  }
}

// Input gradients of one chunk (and partial tap / bias sums over its own
// tokens).  dz is formed for the chunk's tokens and the three after it inside
// the sequence; dx_u needs dz of tokens u .. u+3.
template <typename TA, typename TR>
__global__ __launch_bounds__(256) void kda_conv_bwd_kernel(ConvBwdArgs a) {
  const int c = (int)blockIdx.x, tensor = (int)blockIdx.z;
  int h, t0, len, tseq, tend;
  size_t ch;
  if (!conv_lane(a, h, ch) || !conv_chunk(a, c, t0, len, tseq, tend)) return;
  const size_t HD = (size_t)a.H * DH;
  const TA* x = reinterpret_cast<const TA*>(a.x[tensor]);
  const float* dy = a.dy[tensor];
  TR* dx = reinterpret_cast<TR*>(a.dx[tensor]);
  float w[4][4], bias[4];
  conv_params4<TA>(a, tensor, ch, w, bias);
  auto xat = [&](int t) { return t >= tseq ? ld4(x + (size_t)t * HD + ch) : f32x4{0, 0, 0, 0}; };
  f32x4 h0 = xat(t0 - 3), h1 = xat(t0 - 2), h2 = xat(t0 - 1);
  f32x4 d0 = {0, 0, 0, 0}, d1 = {0, 0, 0, 0}, d2 = {0, 0, 0, 0};  // dz of the three tokens before t
  float sw[4][4] = {}, sb[4] = {};
  const int own_end = t0 + len, tz_end = min(own_end + 3, tend);
  for (int t = t0; t < tz_end; ++t) {
    const f32x4 xt = ld4(x + (size_t)t * HD + ch);
    const f32x4 dyt = ld4(dy + (size_t)t * HD + ch);
    f32x4 dz;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float z = conv_z(w[j], bias[j], h0[j], h1[j], h2[j], xt[j]);
      float g = 1.0f;
      if (a.silu) {
        const float s = sigmoid_f(z);
        g = s * fmaf(z, 1.0f - s, 1.0f);
      }
      dz[j] = dyt[j] * g;
    }
    if (t < own_end) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sw[j][0] = fmaf(dz[j], h0[j], sw[j][0]);
        sw[j][1] = fmaf(dz[j], h1[j], sw[j][1]);
        sw[j][2] = fmaf(dz[j], h2[j], sw[j][2]);
        sw[j][3] = fmaf(dz[j], xt[j], sw[j][3]);
        sb[j] += dz[j];
      }
    }
    const int u = t - 3;  // its four dz are known now
    if (u >= t0) {
      f32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = w[j][3] * d0[j] + w[j][2] * d1[j] + w[j][1] * d2[j] + w[j][0] * dz[j];
      store4(dx + (size_t)u * HD + ch, o);
    }
    h0 = h1; h1 = h2; h2 = xt;
    d0 = d1; d1 = d2; d2 = dz;
  }
  // the last up to three tokens of a sequence: dz past its end is zero
  for (int u = max(t0, tz_end - 3); u < own_end; ++u) {
    const int k = u - (tz_end - 3);  // 0, 1, 2: position of dz_u in (d0, d1, d2)
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = k == 0 ? w[j][3] * d0[j] + w[j][2] * d1[j] + w[j][1] * d2[j]
           : k == 1 ? w[j][3] * d1[j] + w[j][2] * d2[j] : w[j][3] * d2[j];
    store4(dx + (size_t)u * HD + ch, o);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float* pp = a.part + (((size_t)c * 3 + tensor) * HD + ch + j) * 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[i] = sw[j][i];
    pp[4] = sb[j];
  }
}

// Tap and bias gradients: the chunk partials summed in chunk order.  Grid
// (H, 3), one thread per channel.
__global__ __launch_bounds__(128) void kda_conv_param_kernel(ConvBwdArgs a) {
  const int h = (int)blockIdx.x, tensor = (int)blockIdx.y;
  const size_t HD = (size_t)a.H * DH, ch = (size_t)h * DH + threadIdx.x;
  const int nc = a.cfirst[a.N];
  float s[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < nc; ++c) {
    const float* pp = a.part + (((size_t)c * 3 + tensor) * HD + ch) * 5;
#pragma unroll
    for (int k = 0; k < 5; ++k) s[k] += pp[k];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) a.dw[(tensor * HD + ch) * 4 + i] = s[i];
  if (a.db) a.db[tensor * HD + ch] = s[4];
}

// FP32 -> gradient dtype, n elements.
template <typename TR>
__global__ __launch_bounds__(256) void kda_cast_kernel(const float* __restrict__ src, void* dst, int64_t n) {
  TR* d = reinterpret_cast<TR*>(dst);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    d[i] = from_f32<TR>(src[i]);
}

}  // namespace kda
