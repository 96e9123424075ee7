// kda_scan.hpp -- chunk-to-chunk state pass fused with the output combine.
//
// For each chunk of a sequence, with S0 the state entering it (d_k x d_v,
// zero at the sequence start -- no initial/final state, xtuner PR #2301,
// section Change):
//   D      = U - W S0                       (corrected values)
//   out    = scale (Qt S0 + P D)            (inter- plus intra-chunk terms)
//   S_next = Diag(Gam) S0 + Kb^T D
// Columns of S are independent, so one workgroup owns a 32-wide block of
// value channels of one (sequence, head) and walks its chunks in order.  The
// running state stays FP32 in MFMA accumulators for the whole sequence; the
// copy used as a matrix operand is stored in the intermediate type.
//
// Work split inside a workgroup (4 waves, 32x32 MFMA tiles): wave w owns
// state rows 32w..32w+31 (key channels).  X = [W; Qt] S0 is 128 x 32: waves
// 0,1 form W S0 (-> D), waves 2,3 form Qt S0 (-> output).
#pragma once

#include "kda_common.hpp"
#include "kda_intra.hpp"

namespace kda {

struct ScanArgs {
  const int32_t* cu;
  const int32_t* cfirst;
  int N;
  int H;
  float scale;
  const float* gam;  // [chunks][H][128]
  const void* rec;   // [chunks][H][REC]
  void* out;         // [T][H][128]
};

constexpr int DVB = 32;  // value channels per workgroup

template <typename MT> struct ScanLds {
  static constexpr int SL = sizeof(MT) == 2 ? 136 : 132;  // S0^T row: 128 key channels
  static constexpr int DL = sizeof(MT) == 2 ? 72 : 68;    // D^T row: 64 tokens
  static constexpr int O_S = 0;
  static constexpr int O_D = O_S + DVB * SL * (int)sizeof(MT);
  static constexpr int BYTES = O_D + DVB * DL * (int)sizeof(MT);
};

// Workgroup id -> (sequence*H + head, value block).  The four value blocks of
// one (sequence, head) get ids that are equal mod 8, i.e. land on one XCD and
// share its L2 for the per-chunk matrices they all read.
__device__ __forceinline__ void scan_unit(int bid, int& pair, int& vb) {
  const int xcd = bid & 7, slot = bid >> 3;
  vb = slot & 3;
  pair = (slot >> 2) * 8 + xcd;
}

template <typename MT, typename TO>
__global__ __launch_bounds__(256) void kda_scan_kernel(ScanArgs p) {
  typedef ScanLds<MT> L;
  typedef Mma32<MT> M;
  constexpr int SL = L::SL, DL = L::DL;
  constexpr int PL = M::PER_LANE;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  MT* sS = reinterpret_cast<MT*>(smem + L::O_S);  // S0^T [32 dv][SL]
  MT* sD = reinterpret_cast<MT*>(smem + L::O_D);  // D^T  [32 dv][DL]

  int pair, vb;
  scan_unit(blockIdx.x, pair, vb);
  if (pair >= p.N * p.H) return;
  const int n = pair / p.H, h = pair - n * p.H;
  const int cbeg = p.cfirst[n], cend = p.cfirst[n + 1];
  if (cbeg == cend) return;
  const int tseq = p.cu[n], tend = p.cu[n + 1];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 31, g = l >> 5;  // MFMA column (value channel in block), lane group
  const int H = p.H;
  const MT* __restrict__ rec = reinterpret_cast<const MT*>(p.rec);
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);

  // running state rows 32w.. (key), columns vb*32.. (value), FP32
  f32x16 S;
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] = 0.0f;
  for (int x = tid; x < DVB * SL; x += 256) sS[x] = from_f32<MT>(0.0f);
  __syncthreads();

  for (int c = cbeg; c < cend; ++c) {
    const MT* R = rec + ((size_t)c * H + h) * REC;
    const int ctok = tseq + (c - cbeg) * CHUNK;
    const int len = min(CHUNK, tend - ctok);
    // X = A S0, A = W rows (waves 0,1) or Qt rows (waves 2,3); 128 key channels
    // contracted, lane group g covers channels [64g, 64g+64).
    const MT* A = R + (w < 2 ? OFF_W + (32 * w) * DH : OFF_QT + (32 * (w - 2)) * DH);
    f32x16 X;
#pragma unroll
    for (int e = 0; e < 16; ++e) X[e] = 0.0f;
    {
      const MT* pa = A + col * DH + 64 * g;
      const MT* pb = sS + col * SL + 64 * g;
#pragma unroll
      for (int s = 0; s < 64 / PL; ++s) X = M::mma(M::load(pa + s * PL), M::load(pb + s * PL), X);
    }
    if (w < 2) {
      // D = U - W S0 at tokens 32w + row32(e), value column col
      const MT* ut = R + OFF_UT + (size_t)(DVB * vb + col) * CHUNK + 32 * w;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int tk = 8 * e4 + 4 * g;
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = to_f32(ut[tk + i]) - X[4 * e4 + i];
        store4(sD + col * DL + 32 * w + tk, d);
      }
    }
    __syncthreads();
    if (w >= 2) {
      // out = scale (Qt S0 + P D): rows 32(w-2).. of P, 64 tokens contracted
      const MT* pa = R + OFF_P + (32 * (w - 2) + col) * CHUNK + 32 * g;
      const MT* pb = sD + col * DL + 32 * g;
#pragma unroll
      for (int s = 0; s < 32 / PL; ++s) X = M::mma(M::load(pa + s * PL), M::load(pb + s * PL), X);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tk = 32 * (w - 2) + row32(e, l);
        if (tk < len)
          out[((size_t)(ctok + tk) * H + h) * DH + DVB * vb + col] = from_f32<TO>(p.scale * X[e]);
      }
    }
    // S_next = Diag(Gam) S0 + Kb^T D, rows 32w.. of Kb^T, 64 tokens contracted
    {
      const float* gm = p.gam + ((size_t)c * H + h) * DH + 32 * w;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] *= gm[row32(e, l)];
      const MT* pa = R + OFF_KBT + (32 * w + col) * CHUNK + 32 * g;
      const MT* pb = sD + col * DL + 32 * g;
#pragma unroll
      for (int s = 0; s < 32 / PL; ++s) S = M::mma(M::load(pa + s * PL), M::load(pb + s * PL), S);
      // operand copy of the new state, transposed: sS[value][key]
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int kr = 32 * w + 8 * e4 + 4 * g;
        store4(sS + col * SL + kr, f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
      }
    }
    __syncthreads();
  }
}

}  // namespace kda
