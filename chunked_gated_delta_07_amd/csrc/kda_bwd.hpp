// kda_bwd.hpp -- backward (vector-Jacobian product) of the KDA chunked forward,
// recomputed in FP32.
//
// The pages' training path recomputes the backward in FP32 and returns only
// the input gradients in the activation dtype; its gradients of q,
// k, v, the gate and beta are checked against an independent FP64 recurrence
// VJP (xtuner PR #2301, sections Change and Validation), and dt_bias gradients
// are summed in FP32 (xtuner PR #2153, KDA module section).
//
// Notation (one chunk of n <= 64 tokens of one head, entering with state S0;
// G = chunk-local prefix of g, E = exp(G), F_r = exp(G_last - G_r),
// Gam = exp(G_last), Bw = Diag(beta)(k^ * E), Bu = Diag(beta) v):
//   M[r,i] = sum_c k^_rc k^_ic exp(G_rc - G_ic) (i < r),  A = Diag(beta) M
//   P[r,i] = sum_c q^_rc k^_ic exp(G_rc - G_ic) (i <= r)
//   T = (I + A)^{-1},  W = T Bw,  U = T Bu,  Qt = q^ * E,  Kb = k^ * F
//   D = U - W S0,  O = scale (Qt S0 + P D),  S_next = Diag(Gam) S0 + Kb^T D.
// Given dO and dSn = dL/dS_next, reverse-mode differentiation of these steps:
//   dD   = scale P^T dO + Kb dSn               (reverse state scan)
//   dS0  = Diag(Gam) dSn + scale Qt^T dO - W^T dD
//   dQt  = scale dO S0^T,   dP = scale dO D^T (i <= r),   dKb = D dSn^T,
//   dW   = -dD S0^T,        dGam_c = sum_j dSn_cj S0_cj
//   dBu  = T^T dD (dv = beta dBu),  dBw = T^T dW,  dT = dD Bu^T + dW Bw^T,
//   dA   = -(T^T dT T^T) strictly lower,
//   then through the decay-weighted sums with dA (for M, with beta) and dP:
//   alpha_rc = sum_{i<r} dA_ri k^_ic e^{G_rc-G_ic},  pi_rc = sum_{i<=r} dP_ri k^_ic e^{..},
//   rho_ic   = sum_{r>=i} (beta_r dA_ri k^_rc + dP_ri q^_rc) e^{G_rc-G_ic},
//   dq^ = pi + dQt E;  dk^ = beta alpha + rho + beta dBw E + dKb F;
//   dG  = beta k^ alpha + q^ pi - k^ rho + dQt Qt + beta dBw k^ E - dKb Kb
//         (+ sum_r dKb Kb + dGam Gam on the chunk's last row),
//   dbeta = sum_c (Bu dBu / beta + k^ alpha + dBw k^ E) (the first as v.dBu),
//   dg = reverse prefix of dG; x = f + dt_bias: df = dx = -exp(A_log) sigmoid(x) dg,
//   dA_log += sum dg g,  db = dbeta beta (1 - beta),
//   dq = (dq^ - q^ (q^.dq^)) rq,  dk likewise.
// Every exponential of a difference of G has a non-positive exponent
// (diagonal blocks per element; off-diagonal 8x8 blocks factorised about the
// first row of the row block), so no gate strength can overflow it.
//
// Kernel sequence (all intermediates FP32 in the workspace):
//   1. kda_intra_kernel<.., PlainRec, BWD>: records W, Qt^T, Kb^T, U^T, P^T, Gam, T, Bw,
//      W^T, Kb
//   2. kda_bwd_fscan_kernel: S0 of every chunk and D           (per sequence, head, 32 values)
//   3. kda_bwd_bscan_kernel: dSn of every chunk, dD, dS_init   (same, chunks in reverse)
//   4. kda_bwd_jprod_kernel: dQt, dP, dKb, dW, dGam            (per chunk, head)
//   5. kda_bwd_tprod_kernel: dv, dbeta part, dBw, dA          (per chunk, head)
//   6. kda_bwd_gate_kernel:  q^, k^, G, alpha, pi, rho         (per chunk, head)
//   7. kda_bwd_final_kernel: dq, dk, df, db, parameter parts   (per chunk, head)
//   8. kda_bwd_param_kernel: dA_log, dt_bias gradient          (per head, fixed order)
#pragma once

#include "kda_common.hpp"
#include "kda_intra.hpp"

namespace kda {

constexpr int MAT = CHUNK * DH;      // one [64][128] FP32 matrix
constexpr int SQM = CHUNK * CHUNK;   // one [64][64] matrix
constexpr int STM = DH * DH;         // one [128][128] state
constexpr int PPART = 132;           // per-chunk parameter partials: dt_bias[128], A_log, pad

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* f;
  const void* b;
  const void* dout;        // [T][H][128], dtype of the forward's output
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu;
  const int32_t* cfirst;
  const float* init;       // [N][H][128][128] or null
  const float* dfin;       // [N][H][128][128] or null
  int N;
  int H;
  float eps;
  float scale;
  // workspace (FP32), per (chunk, head) unless noted
  const float* rec;        // PlainRec record, REC floats
  const float* gam;        // [128]
  const float* tmat;       // T [64][64]
  const float* bw;         // Bw [64][128]
  const float* wt;         // W^T [128][64]
  const float* kbr;        // Kb [64][128]
  float* s0;               // state entering the chunk [128 key][128 value]
  float* dsn;              // dL/d(state leaving the chunk) [128][128]
  float* dmat;             // D [64][128]
  float* ddmat;            // dD [64][128]
  float* dqt;              // dQt [64][128]
  float* dkb;              // dKb [64][128]
  float* dw;               // dW [64][128]
  float* dbw;              // dBw [64][128]
  float* dpm;              // dP [64][64]
  float* dam;              // dA [64][64]
  float* dgam;             // dGam [128]
  float* db1;              // v . dBu per row [64]
  float* qn;               // q^ [64][128]
  float* kn;               // k^ [64][128]
  float* g2;               // G log2(e) [64][128]
  float* rqk;              // [64] rq, [64] rk
  float* al;               // alpha [64][128]
  float* pi;               // pi [64][128]
  float* rho;              // rho [64][128]
  float* ppart;            // [PPART]
  // outputs
  void* dq;
  void* dk;
  void* dv;
  void* df;
  void* db;
  float* dinit;            // [N][H][128][128] or null
  float* dA_log;           // [H]
  float* ddt_bias;         // [H][128]
};

// Blocks of the two state scans: four value blocks of 32 per (sequence, head)
// pair, placed so that the four land on the same XCD (workgroups are dealt to
// the 8 XCDs round-robin) and share the chunk records through its L2.
__device__ __forceinline__ void scan_block(int bid, int& pair, int& vb) {
  pair = (bid & 7) + 8 * (bid >> 5);
  vb = (bid >> 3) & 3;
}

// Both state scans keep every MFMA operand in LDS with its contracted index
// contiguous ("rows of K", 16-byte reads feeding four FP32 MFMAs), transposing
// where a record's stored order differs, and the state itself transposed
// ([value][key]).  The next chunk's records are loaded into registers while
// the second product of the current chunk runs, then written to LDS.
constexpr int SL_LONG = 132;  // padded row of 128
constexpr int SL_SHORT = 68;  // padded row of 64

// Eight consecutive dout values of one row, scaled.
__device__ __forceinline__ void load8_scaled(const bf16* p, float s, float (&o)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = s * (float)v[e];
}
__device__ __forceinline__ void load8_scaled(const float* p, float s, float (&o)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o[e] = s * a[e]; o[4 + e] = s * b[e]; }
}

// Four consecutive dout values of one row, scaled.
__device__ __forceinline__ void load4_scaled(const bf16* p, float s, float (&o)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = s * (float)v[e];
}
__device__ __forceinline__ void load4_scaled(const float* p, float s, float (&o)[4]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = s * a[e];
}

// ------------------------------------------------------------ 2. forward scan
// Per chunk: snapshot S0; D = U - W S0; S_next = Diag(Gam) S0 + Kb^T D.
// LDS: W [64][128] (rows of K over keys), Kb^T [128][64] (over tokens),
// U^T block [32][64], S^T block [32 value][128 key], D^T [32][64], Gam.
// Eight waves (two per SIMD, so one wave's LDS and barrier waits overlap the
// other's matrix work): D tiles (16 tokens x 16 values) one per wave, state
// tiles (16 keys x 16 values) two per wave.
constexpr int SCAN_THREADS = 512;
__global__ __launch_bounds__(SCAN_THREADS) void kda_bwd_fscan_kernel(BwdArgs p) {
  constexpr int LL = SL_LONG, LS = SL_SHORT, NT = SCAN_THREADS;
  __shared__ __attribute__((aligned(16))) float sW[CHUNK * LL];
  __shared__ __attribute__((aligned(16))) float sKbT[DH * LS];
  __shared__ __attribute__((aligned(16))) float sUT[32 * LS];
  __shared__ __attribute__((aligned(16))) float sST[32 * LL];
  __shared__ __attribute__((aligned(16))) float sDT[32 * LS];
  __shared__ __attribute__((aligned(16))) float sGam[DH];
  int pair, vb;
  scan_block(blockIdx.x + 32 * blockIdx.y, pair, vb);  // grid (32, pairs / 8)
  if (pair >= p.N * p.H) return;
  const int n = pair / p.H, h = pair - n * p.H;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int v0 = 32 * vb;
  const int c_lo = p.cfirst[n], c_hi = p.cfirst[n + 1];
  // the state entering each chunk is snapshotted from registers as it is
  // formed; the first one here
  for (int x = tid; x < DH * 32; x += NT) {
    const int i = x >> 5, j = x & 31;
    const float s0 = p.init ? p.init[((size_t)pair * DH + i) * DH + v0 + j] : 0.0f;
    sST[j * LL + i] = s0;
    if (c_lo < c_hi) p.s0[((size_t)c_lo * p.H + h) * STM + i * DH + v0 + j] = s0;
  }
  // register staging of one chunk's records: W 4, Kb^T 4, U^T 1 f32x4 per thread, Gam
  constexpr int NR = CHUNK * DH / 4 / NT;  // f32x4 of a 64 x 128 matrix per thread
  f32x4 rW[NR], rK[NR], rU, rG;
  auto fetch = [&](int c) {
    const size_t ch = (size_t)c * p.H + h;
    const float* rec = p.rec + ch * REC;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int x = tid + NT * u;
      rW[u] = *reinterpret_cast<const f32x4*>(rec + OFF_W + 4 * x);   // row x/32, cols 4(x%32)
      rK[u] = *reinterpret_cast<const f32x4*>(rec + OFF_KBT + 4 * x); // row x/16, cols 4(x%16)
    }
    // U^T row v0 + tid/16, tokens 4(tid%16)
    rU = *reinterpret_cast<const f32x4*>(rec + OFF_UT + (v0 + (tid >> 4)) * CHUNK + 4 * (tid & 15));
    if (tid < 32) rG = *reinterpret_cast<const f32x4*>(p.gam + ch * DH + 4 * tid);
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int x = tid + NT * u;
      *reinterpret_cast<f32x4*>(sW + (x >> 5) * LL + 4 * (x & 31)) = rW[u];
      *reinterpret_cast<f32x4*>(sKbT + (x >> 4) * LS + 4 * (x & 15)) = rK[u];
    }
    *reinterpret_cast<f32x4*>(sUT + (tid >> 4) * LS + 4 * (tid & 15)) = rU;
    if (tid < 32) *reinterpret_cast<f32x4*>(sGam + 4 * tid) = rG;
  };
  if (c_lo < c_hi) {
    fetch(c_lo);
    stage();
  }
  __syncthreads();
  const int rb = w & 3, cbw = w >> 2;  // this wave's D tile
  for (int c = c_lo; c < c_hi; ++c) {
    const size_t ch = (size_t)c * p.H + h;
    // D[r][j] = U[r][j] - sum_c W[r][c] S[c][j]: rows 16 rb.., values 16 cbw..
    {
      f32x4 acc = {0, 0, 0, 0};
      acc = mma16_rows<float, DH>(sW + 16 * rb * LL, LL, sST + 16 * cbw * LL, LL, acc, l);
      const int j = 16 * cbw + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * (l >> 4) + e;
        const float d = sUT[j * LS + r] - acc[e];
        sDT[j * LS + r] = d;
        p.dmat[ch * MAT + r * DH + v0 + j] = d;
      }
    }
    __syncthreads();
    const bool more = c + 1 < c_hi;
    if (more) fetch(c + 1);
    // S_next[i][j] = Gam_i S[i][j] + sum_r KbT[i][r] D[r][j]: key rows 16w..16w+15
    f32x4 ns[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x4 acc;
      const int j = 16 * cb + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * (l >> 4) + e;
        acc[e] = sGam[i] * sST[j * LL + i];
      }
      ns[cb] = mma16_rows<float, CHUNK>(sKbT + 16 * w * LS, LS, sDT + 16 * cb * LS, LS, acc, l);
      if (more) {
        float* snap = p.s0 + (ch + p.H) * STM;  // state entering chunk c + 1
#pragma unroll
        for (int e = 0; e < 4; ++e) snap[(16 * w + 4 * (l >> 4) + e) * DH + v0 + j] = ns[cb][e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sST[(16 * cb + (l & 15)) * LL + 16 * w + 4 * (l >> 4) + e] = ns[cb][e];
    if (more) stage();
    __syncthreads();
  }
}

// ------------------------------------------------------------ 3. reverse scan
// Chunks in reverse order: snapshot dSn; dD = scale P^T dO + Kb dSn;
// dS0 = Diag(Gam) dSn + scale Qt^T dO - W^T dD.  Ends with dS_init.
// LDS (rows of K): P^T [64 r][64 i], Kb [64 r][128 c], Qt^T [128 i][64 r],
// W^T [128][64], (scale dO)^T block [32 j][64 r], dS^T block [32][128],
// dD^T [32][64], Gam.  Eight waves as in the forward scan: dD tiles one per
// wave, dS0 tiles two per wave.
template <typename TG>
__global__ __launch_bounds__(SCAN_THREADS) void kda_bwd_bscan_kernel(BwdArgs p) {
  constexpr int LL = SL_LONG, LS = SL_SHORT, NT = SCAN_THREADS;
  __shared__ __attribute__((aligned(16))) float sPT[CHUNK * LS];
  __shared__ __attribute__((aligned(16))) float sKb[CHUNK * LL];
  __shared__ __attribute__((aligned(16))) float sQtT[DH * LS];
  __shared__ __attribute__((aligned(16))) float sWT[DH * LS];
  __shared__ __attribute__((aligned(16))) float sOT[32 * LS];
  __shared__ __attribute__((aligned(16))) float sST[32 * LL];
  __shared__ __attribute__((aligned(16))) float sDT[32 * LS];
  __shared__ __attribute__((aligned(16))) float sGam[DH];
  int pair, vb;
  scan_block(blockIdx.x + 32 * blockIdx.y, pair, vb);  // grid (32, pairs / 8)
  if (pair >= p.N * p.H) return;
  const int n = pair / p.H, h = pair - n * p.H;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int v0 = 32 * vb;
  const TG* __restrict__ gO = reinterpret_cast<const TG*>(p.dout);
  const int c_lo = p.cfirst[n], c_hi = p.cfirst[n + 1];
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  // dSn of each chunk is snapshotted from registers as it is formed; the
  // last chunk's (= dS_final) here
  for (int x = tid; x < DH * 32; x += NT) {
    const int i = x >> 5, j = x & 31;
    const float d = p.dfin ? p.dfin[((size_t)pair * DH + i) * DH + v0 + j] : 0.0f;
    sST[j * LL + i] = d;
    if (c_lo < c_hi) p.dsn[((size_t)(c_hi - 1) * p.H + h) * STM + i * DH + v0 + j] = d;
  }
  // register staging: P^T 2, Kb 4, Qt^T 4, W^T 4 f32x4, dO 4 values, Gam
  constexpr int NR = CHUNK * DH / 4 / NT;  // f32x4 of a 64 x 128 matrix per thread
  constexpr int NRP = CHUNK * CHUNK / 4 / NT;
  f32x4 rP[NRP], rK[NR], rQ[NR], rW[NR], rG;
  float rO[4];
  auto fetch = [&](int c) {
    const size_t ch = (size_t)c * p.H + h;
    const float* rec = p.rec + ch * REC;
#pragma unroll
    for (int u = 0; u < NRP; ++u)  // P^T [64 r][64 i]
      rP[u] = *reinterpret_cast<const f32x4*>(rec + OFF_P + 4 * (tid + NT * u));
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int x = tid + NT * u;
      rK[u] = *reinterpret_cast<const f32x4*>(p.kbr + ch * MAT + 4 * x);        // Kb [64][128]
      rQ[u] = *reinterpret_cast<const f32x4*>(rec + OFF_QT + 4 * x);            // Qt^T [128][64]
      rW[u] = *reinterpret_cast<const f32x4*>(p.wt + ch * DH * CHUNK + 4 * x);  // W^T [128][64]
    }
    const int t0 = tseq + (c - c_lo) * CHUNK, len = min(CHUNK, tend - t0);
    const int r = tid >> 3, j4 = 4 * (tid & 7);
    if (r < len) {
      load4_scaled(gO + ((size_t)(t0 + r) * p.H + h) * DH + v0 + j4, p.scale, rO);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) rO[e] = 0.0f;
    }
    if (tid < 32) rG = *reinterpret_cast<const f32x4*>(p.gam + ch * DH + 4 * tid);
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < NRP; ++u) {
      const int x = tid + NT * u;
      *reinterpret_cast<f32x4*>(sPT + (x >> 4) * LS + 4 * (x & 15)) = rP[u];
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int x = tid + NT * u;
      *reinterpret_cast<f32x4*>(sKb + (x >> 5) * LL + 4 * (x & 31)) = rK[u];
      *reinterpret_cast<f32x4*>(sQtT + (x >> 4) * LS + 4 * (x & 15)) = rQ[u];
      *reinterpret_cast<f32x4*>(sWT + (x >> 4) * LS + 4 * (x & 15)) = rW[u];
    }
    {
      const int r = tid >> 3, j4 = 4 * (tid & 7);
#pragma unroll
      for (int e = 0; e < 4; ++e) sOT[(j4 + e) * LS + r] = rO[e];
    }
    if (tid < 32) *reinterpret_cast<f32x4*>(sGam + 4 * tid) = rG;
  };
  if (c_lo < c_hi) {
    fetch(c_hi - 1);
    stage();
  }
  __syncthreads();
  const int rb = w & 3, cbw = w >> 2;  // this wave's dD tile
  for (int c = c_hi - 1; c >= c_lo; --c) {
    const size_t ch = (size_t)c * p.H + h;
    // dD[r][j] = sum_i P^T[r][i] dO^T[j][i] + sum_c Kb[r][c] dS^T[j][c]: rows 16 rb.., values 16 cbw..
    {
      f32x4 acc = {0, 0, 0, 0};
      acc = mma16_rows<float, CHUNK>(sPT + 16 * rb * LS, LS, sOT + 16 * cbw * LS, LS, acc, l);
      acc = mma16_rows<float, DH>(sKb + 16 * rb * LL, LL, sST + 16 * cbw * LL, LL, acc, l);
      const int j = 16 * cbw + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + 4 * (l >> 4) + e;
        sDT[j * LS + r] = acc[e];
        p.ddmat[ch * MAT + r * DH + v0 + j] = acc[e];
      }
    }
    __syncthreads();
    const bool more = c > c_lo;
    if (more) fetch(c - 1);
    // dS0[i][j] = Gam_i dSn[i][j] + sum_r Qt^T[i][r] dO^T[j][r] - sum_r W^T[i][r] dD^T[j][r]:
    // key rows 16w..16w+15
    f32x4 ns[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x4 acc, neg = {0, 0, 0, 0};
      const int j = 16 * cb + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * (l >> 4) + e;
        acc[e] = sGam[i] * sST[j * LL + i];
      }
      acc = mma16_rows<float, CHUNK>(sQtT + 16 * w * LS, LS, sOT + 16 * cb * LS, LS, acc, l);
      neg = mma16_rows<float, CHUNK>(sWT + 16 * w * LS, LS, sDT + 16 * cb * LS, LS, neg, l);
      ns[cb] = acc - neg;
      if (more) {
        float* snap = p.dsn + (ch - p.H) * STM;  // dSn of chunk c - 1
#pragma unroll
        for (int e = 0; e < 4; ++e) snap[(16 * w + 4 * (l >> 4) + e) * DH + v0 + j] = ns[cb][e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sST[(16 * cb + (l & 15)) * LL + 16 * w + 4 * (l >> 4) + e] = ns[cb][e];
    if (more) stage();
    __syncthreads();
  }
  if (p.dinit) {
    for (int x = tid; x < DH * 32; x += NT) {
      const int i = x >> 5, j = x & 31;
      p.dinit[((size_t)pair * DH + i) * DH + v0 + j] = sST[j * LL + i];
    }
  }
}

// Chunk -> (first token, length) for the per-(chunk, head) kernels.
__device__ __forceinline__ bool bwd_chunk(const BwdArgs& p, int c, int& t0, int& len) {
  int tseq;
  return locate_chunk(p.cu, p.cfirst, p.N, c, t0, len, tseq);
}

// ------------------------------------------------------------ 4. products over values
// dQt = scale dO S0^T, dP = scale dO D^T (i <= r), dKb = D dSn^T, dW = -dD S0^T,
// dGam = rowsum(dSn * S0); contracted over the 128 value channels in four
// slabs of 32.  Wave w owns token rows 16w..16w+15 of every output.
template <typename TG>
__global__ __launch_bounds__(256, 2) void kda_bwd_jprod_kernel(BwdArgs p) {
  constexpr int LS = 36;
  __shared__ __attribute__((aligned(16))) float sO[CHUNK * LS];
  __shared__ __attribute__((aligned(16))) float sDm[CHUNK * LS];
  __shared__ __attribute__((aligned(16))) float sDD[CHUNK * LS];
  __shared__ __attribute__((aligned(16))) float sS0[DH * LS];
  __shared__ __attribute__((aligned(16))) float sDS[DH * LS];
  const int c = blockIdx.x, h = blockIdx.y;
  int t0, len;
  if (!bwd_chunk(p, c, t0, len)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const size_t ch = (size_t)c * p.H + h;
  const TG* __restrict__ gO = reinterpret_cast<const TG*>(p.dout);
  f32x4 aq[8], ak[8], aw[8], ap[4];
#pragma unroll
  for (int x = 0; x < 8; ++x) aq[x] = ak[x] = aw[x] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int x = 0; x < 4; ++x) ap[x] = f32x4{0, 0, 0, 0};
  float gacc = 0.0f;
  // slab sl + 1 is loaded into registers while slab sl is multiplied; dout
  // stays in its own dtype (raw 16 or 32 bytes) until it is written to LDS
  constexpr int OW = sizeof(TG) == 2 ? 1 : 2;
  f32x4 rO[OW];
  f32x4 rD[2], rDD[2], rS0[4], rDS[4];
  auto fetch = [&](int sl) {
    const int v0 = 32 * sl;
    const int r = tid >> 2, j8 = 8 * (tid & 3);
    const f32x4* src = reinterpret_cast<const f32x4*>(gO + ((size_t)(t0 + (r < len ? r : 0)) * p.H + h) * DH + v0 + j8);
#pragma unroll
    for (int u = 0; u < OW; ++u) rO[u] = r < len ? src[u] : f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int x = tid + 256 * u, rr = x >> 3, j4 = 4 * (x & 7);
      rD[u] = *reinterpret_cast<const f32x4*>(p.dmat + ch * MAT + rr * DH + v0 + j4);
      rDD[u] = *reinterpret_cast<const f32x4*>(p.ddmat + ch * MAT + rr * DH + v0 + j4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = tid + 256 * u, i = x >> 3, j4 = 4 * (x & 7);
      rS0[u] = *reinterpret_cast<const f32x4*>(p.s0 + ch * STM + i * DH + v0 + j4);
      rDS[u] = *reinterpret_cast<const f32x4*>(p.dsn + ch * STM + i * DH + v0 + j4);
    }
  };
  auto stage = [&]() {
    const int r = tid >> 2, j8 = 8 * (tid & 3);
    float o[8];
    load8_scaled(reinterpret_cast<const TG*>(rO), p.scale, o);  // from registers
    store4(sO + r * LS + j8, f32x4{o[0], o[1], o[2], o[3]});
    store4(sO + r * LS + j8 + 4, f32x4{o[4], o[5], o[6], o[7]});
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int x = tid + 256 * u, rr = x >> 3, j4 = 4 * (x & 7);
      store4(sDm + rr * LS + j4, rD[u]);
      store4(sDD + rr * LS + j4, rDD[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = tid + 256 * u, i = x >> 3, j4 = 4 * (x & 7);
      store4(sS0 + i * LS + j4, rS0[u]);
      store4(sDS + i * LS + j4, rDS[u]);
    }
  };
  fetch(0);
  stage();
  __syncthreads();
  for (int sl = 0; sl < 4; ++sl) {
    if (sl < 3) fetch(sl + 1);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      aq[cb] = mma16_rows<float, 32>(sO + 16 * w * LS, LS, sS0 + 16 * cb * LS, LS, aq[cb], l);
      ak[cb] = mma16_rows<float, 32>(sDm + 16 * w * LS, LS, sDS + 16 * cb * LS, LS, ak[cb], l);
      aw[cb] = mma16_rows<float, 32>(sDD + 16 * w * LS, LS, sS0 + 16 * cb * LS, LS, aw[cb], l);
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
      ap[ib] = mma16_rows<float, 32>(sO + 16 * w * LS, LS, sDm + 16 * ib * LS, LS, ap[ib], l);
    if (tid < DH) {
#pragma unroll 8
      for (int j = 0; j < 32; ++j) gacc = fmaf(sDS[tid * LS + j], sS0[tid * LS + j], gacc);
    }
    __syncthreads();
    if (sl < 3) {
      stage();
      __syncthreads();
    }
  }
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int col = 16 * cb + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * (l >> 4) + e;
      p.dqt[ch * MAT + r * DH + col] = aq[cb][e];
      p.dkb[ch * MAT + r * DH + col] = ak[cb][e];
      p.dw[ch * MAT + r * DH + col] = -aw[cb][e];
    }
  }
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int i = 16 * ib + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * (l >> 4) + e;
      p.dpm[ch * SQM + r * CHUNK + i] = i <= r ? ap[ib][e] : 0.0f;
    }
  }
  if (tid < DH) p.dgam[ch * DH + tid] = gacc;
}

// ------------------------------------------------------------ 5. products with T
// dBu = T^T dD -> dv = beta dBu and db1 = v . dBu per row; dBw = T^T dW;
// dT = dD Bu^T + dW Bw^T;  dA = -(T^T dT) T^T, strictly lower.
// LDS holds unpadded matrices whose 16-byte chunks are XOR-swizzled by row
// (T [64][64], two [64][128] operands; 80 KB in all, two workgroups per CU).
template <int LC>
__device__ __forceinline__ int swz(int r, int c) {
  return r * LC + ((((c >> 2) ^ (r & (LC / 4 - 1)))) << 2) + (c & 3);
}
// C[m][n] += sum_k A[m0+m][k] B[n0+n][k], both swizzled rows of K (16-byte reads)
template <int LCA, int LCB, int K>
__device__ __forceinline__ f32x4 mma16_rows_swz(const float* A, int m0, const float* B, int n0,
                                                f32x4 c, int lane) {
  constexpr int KG = K / 4;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < KG / 4; ++s) {
    const int k = g * KG + 4 * s;
    const f32x4 a4 = *reinterpret_cast<const f32x4*>(A + swz<LCA>(m0 + r, k));
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(B + swz<LCB>(n0 + r, k));
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], b4[e], c, 0, 0, 0);
  }
  return c;
}
// C[m][n] += sum_k At[k][m0+m] B[k][n0+n], both swizzled, k-major
template <int LCA, int LCB, int K>
__device__ __forceinline__ f32x4 mma16_tn_swz(const float* At, int m0, const float* B, int n0,
                                              f32x4 c, int lane) {
  constexpr int KG = K / 4;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < KG; ++s) {
    const int k = g * KG + s;
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(At[swz<LCA>(k, m0 + r)], B[swz<LCB>(k, n0 + r)], c, 0,
                                             0, 0);
  }
  return c;
}

template <typename TA, typename TR>
__global__ __launch_bounds__(256, 2) void kda_bwd_tprod_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) float sT[CHUNK * CHUNK];
  __shared__ __attribute__((aligned(16))) float sR1[CHUNK * DH];
  __shared__ __attribute__((aligned(16))) float sR2[CHUNK * DH];
  const int c = blockIdx.x, h = blockIdx.y;
  int t0, len;
  if (!bwd_chunk(p, c, t0, len)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const size_t ch = (size_t)c * p.H + h;
  const TA* __restrict__ gv = reinterpret_cast<const TA*>(p.v);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  TR* __restrict__ gdv = reinterpret_cast<TR*>(p.dv);
  auto beta_of = [&](int i) {
    return i < len ? sigmoid_f(to_f32(gb[(size_t)(t0 + i) * p.H + h])) : 0.0f;
  };
  // phase 1: T, dD, raw v (rows past the end zero)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int x = tid + 256 * u, r = x >> 4, i4 = 4 * (x & 15);
    *reinterpret_cast<f32x4*>(sT + swz<CHUNK>(r, i4)) =
        *reinterpret_cast<const f32x4*>(p.tmat + ch * SQM + 4 * x);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int x = tid + 256 * u, r = x >> 5, c4 = 4 * (x & 31);
    *reinterpret_cast<f32x4*>(sR1 + swz<DH>(r, c4)) =
        *reinterpret_cast<const f32x4*>(p.ddmat + ch * MAT + 4 * x);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int x = tid + 256 * u, r = x >> 4, c8 = 8 * (x & 15);
    float vv[8];
    if (r < len) {
      load8_scaled(gv + ((size_t)(t0 + r) * p.H + h) * DH + c8, 1.0f, vv);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = 0.0f;
    }
    *reinterpret_cast<f32x4*>(sR2 + swz<DH>(r, c8)) = f32x4{vv[0], vv[1], vv[2], vv[3]};
    *reinterpret_cast<f32x4*>(sR2 + swz<DH>(r, c8 + 4)) = f32x4{vv[4], vv[5], vv[6], vv[7]};
  }
  // this lane's rows 16w + 4(l/16) + e (dv scale) and columns 16 ib + l%16 (dT scale)
  float brow[4], bcol[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    brow[e] = beta_of(16 * w + 4 * (l >> 4) + e);
    bcol[e] = beta_of(16 * e + (l & 15));
  }
  __syncthreads();
  // dBu rows i = 16w.. : dv = beta dBu, db1 = sum_j v dBu
  {
    float bsum[4] = {0, 0, 0, 0};
#pragma unroll 2
    for (int cb = 0; cb < 8; ++cb) {
      f32x4 acc = {0, 0, 0, 0};
      acc = mma16_tn_swz<CHUNK, DH, CHUNK>(sT, 16 * w, sR1, 16 * cb, acc, l);
      const int j = 16 * cb + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * (l >> 4) + e;
        bsum[e] = fmaf(acc[e], sR2[swz<DH>(i, j)], bsum[e]);
        if (i < len) gdv[((size_t)(t0 + i) * p.H + h) * DH + j] = from_f32<TR>(brow[e] * acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) bsum[e] += __shfl_xor(bsum[e], m, 64);
    }
    if ((l & 15) == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) p.db1[ch * CHUNK + 16 * w + 4 * (l >> 4) + e] = bsum[e];
    }
  }
  // dT = dD (beta v)^T: rows r = 16w.., columns i (scaled by beta_i afterwards)
  f32x4 dt[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    f32x4 acc = {0, 0, 0, 0};
    acc = mma16_rows_swz<DH, DH, DH>(sR1, 16 * w, sR2, 16 * ib, acc, l);
    dt[ib] = acc * bcol[ib];
  }
  __syncthreads();
  // phase 2: dW -> sR1, Bw -> sR2 (the other workgroup on the CU covers the latency)
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int x = tid + 256 * u, r = x >> 5, c4 = 4 * (x & 31);
    *reinterpret_cast<f32x4*>(sR1 + swz<DH>(r, c4)) =
        *reinterpret_cast<const f32x4*>(p.dw + ch * MAT + 4 * x);
    *reinterpret_cast<f32x4*>(sR2 + swz<DH>(r, c4)) =
        *reinterpret_cast<const f32x4*>(p.bw + ch * MAT + 4 * x);
  }
  __syncthreads();
  // dT += dW Bw^T
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) dt[ib] = mma16_rows_swz<DH, DH, DH>(sR1, 16 * w, sR2, 16 * ib, dt[ib], l);
  // dBw = T^T dW
#pragma unroll 2
  for (int cb = 0; cb < 8; ++cb) {
    f32x4 acc = {0, 0, 0, 0};
    acc = mma16_tn_swz<CHUNK, DH, CHUNK>(sT, 16 * w, sR1, 16 * cb, acc, l);
    const int col = 16 * cb + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) p.dbw[ch * MAT + (16 * w + 4 * (l >> 4) + e) * DH + col] = acc[e];
  }
  __syncthreads();
  // phase 3: X = T^T dT, dA = -X T^T (strictly lower); dT and X in sR2
  float* sDT = sR2;
  float* sX = sR2 + SQM;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int e = 0; e < 4; ++e) sDT[swz<CHUNK>(16 * w + 4 * (l >> 4) + e, 16 * ib + (l & 15))] = dt[ib][e];
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0, 0, 0, 0};
    acc = mma16_tn_swz<CHUNK, CHUNK, CHUNK>(sT, 16 * w, sDT, 16 * mb, acc, l);
#pragma unroll
    for (int e = 0; e < 4; ++e) sX[swz<CHUNK>(16 * w + 4 * (l >> 4) + e, 16 * mb + (l & 15))] = acc[e];
  }
  __syncthreads();
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    f32x4 acc = {0, 0, 0, 0};
    acc = mma16_rows_swz<CHUNK, CHUNK, CHUNK>(sX, 16 * w, sT, 16 * jb, acc, l);
    const int j = 16 * jb + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * (l >> 4) + e;
      p.dam[ch * SQM + i * CHUNK + j] = j < i ? -acc[e] : 0.0f;
    }
  }
}

// Per-token-head prep of the backward, FP32: the log2-unit gate
// g2 = g log2(e) = -exp(A_log) softplus(x) log2(e), x = f + dt_bias.
__device__ __forceinline__ float gate_log2(float x, float lam) {
  const float t = exp2_hw(-fabsf(x) * LOG2E);
  return -lam * (fmaxf(x, 0.0f) * LOG2E + log2_hw(1.0f + t));
}

// ------------------------------------------------------------ 6. decay-weighted sums
// Recomputes q^, k^ and G (stored for kernel 7), then
//   waves 0-3 (one thread per channel): alpha, pi (sums over i <= r per row r)
//   waves 4-7 (one thread per channel): rho (sums over r >= i per column i)
// in 8x8 token blocks: off-diagonal blocks (R > I) factorised about row 8R,
//   e^{G_r - G_i} = e^{G_r - G_8R} e^{G_8R - G_i}  (both exponents <= 0),
// diagonal blocks per element.
template <typename TA>
__global__ __launch_bounds__(512) void kda_bwd_gate_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) float sQ[CHUNK * DH];
  __shared__ __attribute__((aligned(16))) float sK[CHUNK * DH];
  __shared__ __attribute__((aligned(16))) float sG[CHUNK * DH];
  __shared__ __attribute__((aligned(16))) float sA[SQM];
  __shared__ __attribute__((aligned(16))) float sP[SQM];
  __shared__ float sBeta[CHUNK];
  const int cidx = blockIdx.x, h = blockIdx.y;
  int t0, len;
  if (!bwd_chunk(p, cidx, t0, len)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const size_t ch = (size_t)cidx * p.H + h;
  const TA* __restrict__ gq = reinterpret_cast<const TA*>(p.q);
  const TA* __restrict__ gk = reinterpret_cast<const TA*>(p.k);
  const TA* __restrict__ gf = reinterpret_cast<const TA*>(p.f);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  const float lam = expf(p.A_log[h]);
  const int c0 = 2 * l;
  const f32x2 dtb = *reinterpret_cast<const f32x2*>(p.dt_bias + (size_t)h * DH + c0);
  // prep: wave w (of 8) rows 8w..8w+7, lane channels c0, c0+1; rows past the
  // end are zero (q^ = k^ = 0, g = 0).  All row loads are issued before any use.
  f32x2 qv[8], kv[8], fv[8];
  float bv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * w + j;
    const int rr = r < len ? r : 0;
    const size_t o = ((size_t)(t0 + rr) * p.H + h) * DH + c0;
    qv[j] = load2(gq + o);
    kv[j] = load2(gk + o);
    fv[j] = load2(gf + o);
    bv[j] = to_f32(gb[(size_t)(t0 + rr) * p.H + h]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * w + j;
    const bool ok = r < len;
    if (!ok) qv[j] = kv[j] = fv[j] = f32x2{0, 0};
    const float sq = wave_sum(qv[j][0] * qv[j][0] + qv[j][1] * qv[j][1]);
    const float sk = wave_sum(kv[j][0] * kv[j][0] + kv[j][1] * kv[j][1]);
    const float rq = rsqrt_hw(sq + p.eps), rk = rsqrt_hw(sk + p.eps);
    sQ[r * DH + c0] = qv[j][0] * rq; sQ[r * DH + c0 + 1] = qv[j][1] * rq;
    sK[r * DH + c0] = kv[j][0] * rk; sK[r * DH + c0 + 1] = kv[j][1] * rk;
    sG[r * DH + c0] = ok ? gate_log2(fv[j][0] + dtb[0], lam) : 0.0f;
    sG[r * DH + c0 + 1] = ok ? gate_log2(fv[j][1] + dtb[1], lam) : 0.0f;
    if (l == 0) {
      sBeta[r] = ok ? sigmoid_f(bv[j]) : 0.0f;
      p.rqk[ch * 2 * CHUNK + r] = rq;
      p.rqk[ch * 2 * CHUNK + CHUNK + r] = rk;
    }
  }
  __syncthreads();
  if (tid < DH) {
    float acc = 0.0f;
    for (int r = 0; r < CHUNK; ++r) {
      acc += sG[r * DH + tid];
      sG[r * DH + tid] = acc;
    }
  } else {
    for (int x = tid - DH; x < SQM / 4; x += 384) {
      reinterpret_cast<f32x4*>(sA)[x] = reinterpret_cast<const f32x4*>(p.dam + ch * SQM)[x];
      reinterpret_cast<f32x4*>(sP)[x] = reinterpret_cast<const f32x4*>(p.dpm + ch * SQM)[x];
    }
  }
  __syncthreads();
  for (int x = tid; x < MAT / 4; x += 512) {
    reinterpret_cast<f32x4*>(p.qn + ch * MAT)[x] = reinterpret_cast<const f32x4*>(sQ)[x];
    reinterpret_cast<f32x4*>(p.kn + ch * MAT)[x] = reinterpret_cast<const f32x4*>(sK)[x];
    reinterpret_cast<f32x4*>(p.g2 + ch * MAT)[x] = reinterpret_cast<const f32x4*>(sG)[x];
  }
  // Four roles of 128 threads (one per channel): rows of blocks {7,6,1,0},
  // rows of {5,4,3,2}, columns of blocks {0,1,6,7}, columns of {2,3,4,5}
  // (18 of the 36 block pairs each).
  const int c = tid & (DH - 1), role = tid >> 7;
  const int set = role & 1;
  if (role < 2) {
    // rows: alpha_r = sum_{i<r} dA_ri k^_i e^{G_r-G_i}, pi_r = sum_{i<=r} dP_ri k^_i e^{..}
    for (int k4 = 0; k4 < 4; ++k4) {
      const int R = set == 0 ? (k4 < 2 ? 7 - k4 : 3 - k4) : 5 - k4;
      const int m = 8 * R;
      const float gm = sG[m * DH + c];
      float ao[8], po[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) ao[a] = po[a] = 0.0f;
      for (int I = 0; I < R; ++I) {
        float kt[8];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          const int i = 8 * I + bb;
          kt[bb] = sK[i * DH + c] * exp2_hw(gm - sG[i * DH + c]);
        }
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const float* ar = sA + (m + a) * CHUNK + 8 * I;
          const float* pr = sP + (m + a) * CHUNK + 8 * I;
#pragma unroll
          for (int bb = 0; bb < 8; ++bb) {
            ao[a] = fmaf(ar[bb], kt[bb], ao[a]);
            po[a] = fmaf(pr[bb], kt[bb], po[a]);
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int r = m + a;
        const float gr = sG[r * DH + c];
        const float fa = exp2_hw(gr - gm);
        float al = ao[a] * fa, pv = po[a] * fa;
#pragma unroll
        for (int bb = 0; bb <= a; ++bb) {
          const int i = m + bb;
          const float kte = sK[i * DH + c] * exp2_hw(gr - sG[i * DH + c]);
          al = fmaf(sA[r * CHUNK + i], kte, al);
          pv = fmaf(sP[r * CHUNK + i], kte, pv);
        }
        p.al[ch * MAT + r * DH + c] = al;
        p.pi[ch * MAT + r * DH + c] = pv;
      }
    }
  } else {
    // columns: rho_i = sum_{r>=i} (beta_r dA_ri k^_r + dP_ri q^_r) e^{G_r-G_i}
    for (int k4 = 0; k4 < 4; ++k4) {
      const int I = set == 0 ? (k4 < 2 ? k4 : 4 + k4) : 2 + k4;
      float ro[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) ro[bb] = 0.0f;
      for (int R = I + 1; R < 8; ++R) {
        const int m = 8 * R;
        const float gm = sG[m * DH + c];
        float bk[8], qq[8], part[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const int r = m + a;
          const float fa = exp2_hw(sG[r * DH + c] - gm);
          bk[a] = sBeta[r] * sK[r * DH + c] * fa;
          qq[a] = sQ[r * DH + c] * fa;
        }
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) part[bb] = 0.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const float* ar = sA + (m + a) * CHUNK + 8 * I;
          const float* pr = sP + (m + a) * CHUNK + 8 * I;
#pragma unroll
          for (int bb = 0; bb < 8; ++bb) part[bb] = fmaf(ar[bb], bk[a], fmaf(pr[bb], qq[a], part[bb]));
        }
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          const int i = 8 * I + bb;
          ro[bb] = fmaf(exp2_hw(gm - sG[i * DH + c]), part[bb], ro[bb]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int i = 8 * I + bb;
        const float gi = sG[i * DH + c];
        float rv = ro[bb];
#pragma unroll
        for (int a = bb; a < 8; ++a) {
          const int r = 8 * I + a;
          const float e = exp2_hw(sG[r * DH + c] - gi);
          rv = fmaf(fmaf(sA[r * CHUNK + i], sBeta[r] * sK[r * DH + c], sP[r * CHUNK + i] * sQ[r * DH + c]), e, rv);
        }
        p.rho[ch * MAT + i * DH + c] = rv;
      }
    }
  }
}

// ------------------------------------------------------------ 7. elementwise chain
// Wave w: rows 16w..16w+15, lane channels c0, c0+1.  Row-local parts (dq, dk,
// db, dG) row by row; dG goes to LDS.  Then the reverse
// prefix of dG over the chunk: inside the wave over its 16 rows from LDS,
// across waves one carry (column totals of the later waves plus the last
// row's d(G_last) terms), giving df and the per-chunk parameter partials.
template <typename TA, typename TR>
__global__ __launch_bounds__(256) void kda_bwd_final_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(16))) float sDG[CHUNK * DH];
  __shared__ float sTot[4][DH];
  __shared__ float sCol[4][DH];
  __shared__ float sPdt[4][DH];
  __shared__ float sPa[4];
  const int cidx = blockIdx.x, h = blockIdx.y;
  int t0, len;
  if (!bwd_chunk(p, cidx, t0, len)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const size_t ch = (size_t)cidx * p.H + h;
  const TA* __restrict__ gf = reinterpret_cast<const TA*>(p.f);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  TR* __restrict__ gdq = reinterpret_cast<TR*>(p.dq);
  TR* __restrict__ gdk = reinterpret_cast<TR*>(p.dk);
  TR* __restrict__ gdf = reinterpret_cast<TR*>(p.df);
  TR* __restrict__ gdb = reinterpret_cast<TR*>(p.db);
  const int c0 = 2 * l;
  const size_t mb = ch * MAT;
  const float lam = expf(p.A_log[h]);
  const f32x2 dtb = *reinterpret_cast<const f32x2*>(p.dt_bias + (size_t)h * DH + c0);
  const f32x2 gL = load2(p.g2 + mb + (CHUNK - 1) * DH + c0);  // G_last (rows past the end keep it)
  float tot0 = 0.0f, tot1 = 0.0f, col0 = 0.0f, col1 = 0.0f;
#pragma unroll 2
  for (int j = 0; j < 16; ++j) {
    const int r = 16 * w + j;
    const bool ok = r < len;
    const int rr = ok ? r : 0;
    const size_t o = mb + r * DH + c0;
    const f32x2 qn = load2(p.qn + o), kn = load2(p.kn + o), g2 = load2(p.g2 + o);
    const f32x2 al = load2(p.al + o), pv = load2(p.pi + o), rh = load2(p.rho + o);
    const f32x2 dqt = load2(p.dqt + o), dkb = load2(p.dkb + o), dbw = load2(p.dbw + o);
    const float bv = to_f32(gb[(size_t)(t0 + rr) * p.H + h]);
    const float beta = ok ? sigmoid_f(bv) : 0.0f;
    float dqn[2], dkn[2], dG[2], kbf[2], sb = 0.0f;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float E = exp2_hw(g2[x]), F = exp2_hw(gL[x] - g2[x]);
      dqn[x] = pv[x] + dqt[x] * E;
      dkn[x] = beta * al[x] + rh[x] + beta * dbw[x] * E + dkb[x] * F;
      kbf[x] = ok ? dkb[x] * kn[x] * F : 0.0f;
      dG[x] = ok ? beta * kn[x] * al[x] + qn[x] * pv[x] - kn[x] * rh[x] + dqt[x] * qn[x] * E +
                       beta * dbw[x] * kn[x] * E - kbf[x]
                 : 0.0f;
      sb += kn[x] * al[x] + dbw[x] * kn[x] * E;
    }
    tot0 += dG[0]; tot1 += dG[1];
    col0 += kbf[0]; col1 += kbf[1];
    *reinterpret_cast<f32x2*>(sDG + r * DH + c0) = f32x2{dG[0], dG[1]};
    const float s_b = wave_sum(sb);
    const float s_q = wave_sum(qn[0] * dqn[0] + qn[1] * dqn[1]);
    const float s_k = wave_sum(kn[0] * dkn[0] + kn[1] * dkn[1]);
    if (ok) {
      const float rq = p.rqk[ch * 2 * CHUNK + r], rk = p.rqk[ch * 2 * CHUNK + CHUNK + r];
      const size_t go = ((size_t)(t0 + r) * p.H + h) * DH + c0;
      store2(gdq + go, rq * (dqn[0] - qn[0] * s_q), rq * (dqn[1] - qn[1] * s_q));
      store2(gdk + go, rk * (dkn[0] - kn[0] * s_k), rk * (dkn[1] - kn[1] * s_k));
      if (l == 0)
        gdb[(size_t)(t0 + r) * p.H + h] =
            from_f32<TR>((p.db1[ch * CHUNK + r] + s_b) * beta * (1.0f - beta));
    }
  }
  sTot[w][c0] = tot0; sTot[w][c0 + 1] = tot1;
  sCol[w][c0] = col0; sCol[w][c0 + 1] = col1;
  __syncthreads();
  // dg_r = sum_{j >= r} dG_j plus, on every valid row, the last row's extra
  // terms sum_r dKb k^ F + dGam Gam (they belong to G_last)
  float carry[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int c = c0 + x;
    float a = sCol[0][c] + sCol[1][c] + sCol[2][c] + sCol[3][c] + p.dgam[ch * DH + c] * exp2_hw(gL[x]);
    for (int w2 = w + 1; w2 < 4; ++w2) a += sTot[w2][c];
    carry[x] = a;
  }
  float pdt0 = 0.0f, pdt1 = 0.0f, pa = 0.0f;
  // x = f + dt_bias of the wave's 16 rows, loaded together (second read, cached)
  f32x2 xs[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 16 * w + j;
    xs[j] = load2(gf + ((size_t)(t0 + (r < len ? r : 0)) * p.H + h) * DH + c0) + dtb;
  }
#pragma unroll
  for (int j = 15; j >= 0; --j) {
    const int r = 16 * w + j;
    if (r >= len) continue;  // uniform over the wave
    const f32x2 dg = *reinterpret_cast<const f32x2*>(sDG + r * DH + c0);
    const f32x2 xx = xs[j];
    carry[0] += dg[0];
    carry[1] += dg[1];
    const float dx0 = lam == 0.0f ? 0.0f : -lam * sigmoid_f(xx[0]) * carry[0];
    const float dx1 = lam == 0.0f ? 0.0f : -lam * sigmoid_f(xx[1]) * carry[1];
    pdt0 += dx0;
    pdt1 += dx1;
    pa = fmaf(carry[0], gate_log2(xx[0], lam) * (1.0f / LOG2E), pa);
    pa = fmaf(carry[1], gate_log2(xx[1], lam) * (1.0f / LOG2E), pa);
    store2(gdf + ((size_t)(t0 + r) * p.H + h) * DH + c0, dx0, dx1);
  }
  sPdt[w][c0] = pdt0; sPdt[w][c0 + 1] = pdt1;
  pa = wave_sum(pa);
  if (l == 0) sPa[w] = pa;
  __syncthreads();
  if (tid < DH) p.ppart[ch * PPART + tid] = sPdt[0][tid] + sPdt[1][tid] + sPdt[2][tid] + sPdt[3][tid];
  if (tid == 0) p.ppart[ch * PPART + DH] = sPa[0] + sPa[1] + sPa[2] + sPa[3];
}

// ------------------------------------------------------------ 8. parameter gradients
// dt_bias and A_log gradients of head h: per-chunk partials summed in chunk
// order (FP32, deterministic).
__global__ __launch_bounds__(DH) void kda_bwd_param_kernel(BwdArgs p) {
  const int h = blockIdx.x, c = threadIdx.x;
  const int nch = p.cfirst[p.N];
  float sdt = 0.0f, sa = 0.0f;
  for (int k = 0; k < nch; ++k) {
    const float* pp = p.ppart + ((size_t)k * p.H + h) * PPART;
    sdt += pp[c];
    if (c == 0) sa += pp[DH];
  }
  p.ddt_bias[(size_t)h * DH + c] = sdt;
  if (c == 0) p.dA_log[h] = sa;
}

// Gradient outputs of an empty batch: dS_init = dS_final (or zero), dA_log
// and the dt_bias gradient zero.
__global__ __launch_bounds__(256) void kda_bwd_empty_kernel(const float* __restrict__ dfin,
                                                            float* __restrict__ dinit, int64_t n,
                                                            float* __restrict__ dA_log,
                                                            float* __restrict__ ddt, int H) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (dinit)
    for (int64_t i = i0; i < n; i += stride) dinit[i] = dfin ? dfin[i] : 0.0f;
  for (int64_t i = i0; i < (int64_t)H * DH; i += stride) ddt[i] = 0.0f;
  for (int64_t i = i0; i < H; i += stride) dA_log[i] = 0.0f;
}

}  // namespace kda
