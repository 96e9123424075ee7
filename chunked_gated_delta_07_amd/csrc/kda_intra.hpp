// kda_intra.hpp -- per-(chunk, head) kernel: gate/beta/L2-norm prep, the
// decay-weighted intra-chunk blocks, the chunk solve, and the matrices the
// state pass consumes.
//
// Chunk algebra (the token recurrence re-associated over a chunk of n <= 64
// tokens; the chunked operator and its "chunk solve / state intermediates"
// are those of xtuner PR #2301 "[Enhancement] Add opt-in FP32 KDA chunk
// computation", sections Problem and Change):
//   a_r[c]  = exp(g_r[c]) (per-token decay), Gam = prod_r a_r
//   A[r,i]  = beta_r sum_c k^_rc k^_ic prod_{i<j<=r} a_j[c]      (i < r)
//   P[r,i]  = sum_c q^_rc k^_ic prod_{i<j<=r} a_j[c]             (i <= r)
//   T       = (I + A)^{-1}   (unit lower triangular)
//   W       = T Diag(beta) (k^ * E),   E_r = prod_{j<=r} a_j
//   U       = T Diag(beta) v
//   Qt      = q^ * E,   Kb_r = k^_r * prod_{j>r} a_j
// Every decay factor is a product of per-token decays over a token range, so
// it lies in [0, 1] and never overflows, however strong the gate; the pages'
// FP32 gate prefix with a fixed layout (xtuner PR #2153, KDA module section) is
// kept as an FP32 prefix, multiplicative here.
//
// Off-diagonal 16x16 blocks (row block R > column block I) are products
// (k^_r * prod_{16R<j<=r} a_j) . (k^_i * prod_{i<j<=16R} a_j): both factors
// <= 1, one MFMA tile each.  Inside a diagonal block the same split about a
// row between the two covers rows 8..15 x columns 0..7 (about row 8) and, with
// bf16 operands, rows 4..7 x 0..3 and 12..15 x 8..11 (about rows 4 and 12, one
// tile for both); for the remaining pairs the decay is formed per pair and
// channel on the VALU and the channel sum is done by an MFMA (one useful pair
// per output column), or with FP32 operands by a sum over the wave.
//
// Layout choices: one workgroup (4 waves) per (chunk, head).  For the VALU
// work each wave owns 16 token rows and each lane two adjacent channels, so
// prefix/suffix products along tokens are plain register loops.  MFMA
// operands are staged through LDS as rows of contiguous channels.
#pragma once

#include <type_traits>

#include "kda_common.hpp"

namespace kda {

// Per-(chunk, head) record in the workspace, element type MT, holding
//   W [64 tok][128 key ch], Qt [64][128], Kb^T [128 key ch][64 tok],
//   U [64 tok][128 value ch], P [64][64] (its three 32x32 tiles on or below
//   the diagonal)
// plus Gam [128] float in a separate array.  Each matrix is stored in the
// order in which the state pass reads it: one state-pass load instruction
// (64 lanes x 16 bytes) covers 1 KB of contiguous memory (Qt: one 16-byte
// unit per lane from a row-major layout, see qt).  The state pass uses
// 32x32 MFMA tiles; lane L = 32 g + col holds tile row/column col and the
// contracted-index half g (see kda_scan.hpp).  FE = elements per 16 bytes.
constexpr int OFF_W = 0;
constexpr int OFF_QT = CHUNK * DH;
constexpr int OFF_KBT = 2 * CHUNK * DH;
constexpr int OFF_UT = 3 * CHUNK * DH;
constexpr int OFF_P = 4 * CHUNK * DH;
constexpr int REC = 4 * CHUNK * DH + CHUNK * CHUNK;
// P as its three 32x32 tiles on or below the diagonal (the fourth is zero):
// the records of the forward (Frag, FragW)
constexpr int REC_LP = 4 * CHUNK * DH + 3 * CHUNK * CHUNK / 4;

template <typename MT> struct Frag {
  static constexpr int FE = 16 / (int)sizeof(MT);
  static constexpr bool TRANSPOSED_QT_P = false;
  // P without its zero tile, and the token-contracted operands (Kb^T, P) in
  // steps of 16 consecutive tokens (see kb).
  static constexpr bool P_LOWER_TILES = true;
  static constexpr int REC_ELEMS = REC_LP;
  // W / Qt element (token r, key channel c): A operand of [W;Qt] S0, contracted
  // over key channels, half g = c/64.
  __host__ __device__ static constexpr int a(int r, int c) {
    return (((r >> 5) * (64 / FE) + (c & 63) / FE) * 64 + 32 * (c >> 6) + (r & 31)) * FE + (c & 63) % FE;
  }
  // Qt element (token r, key channel c): row-major, the 16-byte chunks of row
  // r permuted by chunk ^ (r % 16), so that the intra kernel writes whole rows
  // per store (two or four lanes per chunk; as W's order a chunk would hold
  // values of lanes 1 KB apart) and the state pass reads the values of a W
  // fragment (lane: token, 8 or 4 channels) from 16 rows per 16 lanes with no
  // bank conflicts.
  __host__ __device__ static constexpr int qt(int r, int c) {
    return r * DH + FE * ((c / FE) ^ (r & 15)) + c % FE;
  }
  // Kb^T element (key channel c, token t): A operand of Kb^T D, contracted over
  // tokens in steps of 16: the 8 tokens 16 s + 8 g .. + 7 of step s sit in
  // lane half g (one 16-byte unit in bf16, the units of fragments 2 s and
  // 2 s + 1 in FP32).
  __host__ __device__ static constexpr int kb(int c, int t) {
    return (((c >> 5) * (32 / FE) + (t >> 4) * (8 / FE) + (t & 7) / FE) * 64 + 32 * ((t >> 3) & 1) +
            (c & 31)) * FE + t % FE;
  }
  // P element (token r, token i): A operand of P D, contracted over i in the
  // order of Kb^T's tokens.  Only i < 32 (r / 32 + 1) is stored: rows 0..31
  // in the first 16 / FE fragments (i < 32), rows 32..63 in the next 32 / FE.
  __host__ __device__ static constexpr int pm(int r, int i) {
    return ((((r >> 5) == 0 ? 0 : 16 / FE) + (i >> 4) * (8 / FE) + (i & 7) / FE) * 64 +
            32 * ((i >> 3) & 1) + (r & 31)) * FE + i % FE;
  }
  // column i of element q of lane half g in P fragment u of its row tile
  __host__ __device__ static constexpr int pcol(int u, int g, int q) {
    return 16 * (u / (8 / FE)) + 8 * g + FE * (u % (8 / FE)) + q;
  }
  // U element (token t, value channel v): lane (g, col = v%32) of wave t/32 in
  // value block v/32 holds the 16 tokens 32w + 8e + 4g + i as q = 4e + i.
  __host__ __device__ static constexpr int u(int t, int v) {
    return ((((v >> 5) * 2 + (t >> 5)) * (16 / FE) + (4 * ((t & 31) >> 3) + (t & 3)) / FE) * 64 +
            32 * ((t >> 2) & 1) + (v & 31)) * FE + (4 * ((t & 31) >> 3) + (t & 3)) % FE;
  }
};

// The same record as whole matrices for the backward pass, each in the
// orientation its consumer contracts over: W [64 tok][128 key], Qt^T
// [128 key][64 tok], Kb^T [128][64], U^T [128 value][64 tok], P^T [64 i][64 r].
// (The forward's own layout is Frag; there the Qt and P stores are vectors.)
template <typename MT> struct PlainRec {
  static constexpr int FE = 16 / (int)sizeof(MT);
  static constexpr bool TRANSPOSED_QT_P = true;
  static constexpr bool P_LOWER_TILES = false;
  static constexpr int REC_ELEMS = REC;
  __host__ __device__ static constexpr int a(int r, int c) { return r * DH + c; }
  __host__ __device__ static constexpr int qt(int r, int c) { return c * CHUNK + r; }
  __host__ __device__ static constexpr int kb(int c, int t) { return c * CHUNK + t; }
  __host__ __device__ static constexpr int pm(int r, int i) { return i * CHUNK + r; }
  __host__ __device__ static constexpr int u(int t, int v) { return v * CHUNK + t; }
};

// The record in the order of the windowed state pass (kda_window.hpp), bf16
// only.  There every matrix is a 32x32x16 bf16 MFMA operand fragment read by
// one wave: 64 lanes x 8 elements, 1 KB contiguous.  The contracted index is
// permuted inside each step of 16: lane group g (lanes 32g..32g+31) element p
// holds index kappa(g, p) = 4g + (p & 3) + 8 (p >> 2).  With that order the
// rows held by one lane of a 32x32 accumulator (rows 8j + 4g + i of lane
// group g) are, two j at a time, exactly one operand fragment, so the state
// and the corrected values D feed the next products straight from their
// accumulators.  Fragments:
//   W, Qt  (token r, key c):    (key step c/16, token tile r/32), lane r%32 + 32 g
//   Kb^T   (key c, token t):    (token step t/16, key tile c/32), lane c%32 + 32 g
//   P      (row r, column i):   only the tiles on or below the diagonal at
//                               32-token granularity: (0,0) (0,1) (1,0) .. (1,3)
//   U      (token t, value v):  accumulator order, 16 values per lane:
//                               (value block v/32, token tile t/32), lane v%32 + 32 g
//                               element 4 (m/8) + m%4, m = t%32, g = (m/4)%2
constexpr int OFFW_P = 4 * CHUNK * DH;  // = OFF_P
constexpr int RECW = REC_LP;  // 35,840 elements
template <typename MT> struct FragW {
  static_assert(sizeof(MT) == 2, "bf16 records only");
  static constexpr int FE = 8;
  static constexpr bool TRANSPOSED_QT_P = false;
  static constexpr bool P_LOWER_TILES = true;
  static constexpr int REC_ELEMS = RECW;
  // element p of lane group g for contracted index k (within its step of 16)
  __host__ __device__ static constexpr int kg(int k) { return (k >> 2) & 1; }
  __host__ __device__ static constexpr int kp(int k) { return 4 * ((k & 15) >> 3) + (k & 3); }
  __host__ __device__ static constexpr int a(int r, int c) {
    return (((c >> 4) * 2 + (r >> 5)) * 64 + (r & 31) + 32 * kg(c)) * 8 + kp(c);
  }
  __host__ __device__ static constexpr int qt(int r, int c) { return a(r, c); }
  __host__ __device__ static constexpr int kb(int c, int t) {
    return (((t >> 4) * 4 + (c >> 5)) * 64 + (c & 31) + 32 * kg(t)) * 8 + kp(t);
  }
  // P (row r, column i), i < 32 (r / 32 + 1); the record holds these only.
  // Offset inside the P region, which starts at OFF_P (= OFFW_P).
  __host__ __device__ static constexpr int pm(int r, int i) {
    return ((((r >> 5) == 0 ? 0 : 2) + (i >> 4)) * 64 + (r & 31) + 32 * kg(i)) * 8 + kp(i);
  }
  // column i of element q of lane half g in P fragment step s
  __host__ __device__ static constexpr int pcol(int s, int g, int q) { return 16 * s + 4 * g + (q & 3) + 8 * (q >> 2); }
  __host__ __device__ static constexpr int u(int t, int v) {
    return ((((v >> 5) * 2 + (t >> 5)) * 64 + (v & 31) + 32 * (((t & 31) >> 2) & 1)) * 16 +
            4 * ((t & 31) >> 3) + (t & 3));
  }
};

struct IntraArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* f;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  const int32_t* cu;
  const int32_t* cfirst;  // [N+1] first chunk of each sequence; cfirst[N] = chunk count; null for N = 1
  int N;
  int H;
  float eps;
  float* gam;  // [chunks][H][128]
  void* rec;   // [chunks][H][LY::REC_ELEMS] of MT (or [ring][H][..])
  int ring;    // > 0: records and gam of chunk c live in slot c % ring
  int c0;      // forward kernel: first chunk of this launch's grid rows
  // optional short causal convolution on q, k, v (used when the kernel's
  // CONV parameter is set): weights [3][H*128][4] (tap 3 = current token),
  // bias [3][H*128] or null, SiLU after it when conv_silu != 0
  const float* conv_w;
  const float* conv_b;
  int conv_silu;
  // backward recomputation only (kernel parameter BWD): T = (I + A)^{-1}
  // [chunks][H][64][64] and Bw = Diag(beta) (k^ * E) [chunks][H][64][128], FP32
  float* tmat;
  float* bw;
  // and W^T [128][64], Kb [64][128] (the backward's reverse state scan)
  float* wt;
  float* kbr;
  // key and value widths of the inputs when the kernel's RECT parameter is
  // set (q, k, f_raw [T][H][dk], dt_bias [H][dk], v [T][H][dv], each <= 128);
  // the chunk algebra runs at 128 with the missing channels taken as zero
  int dk, dv;
};

// Chunks [cbeg, cend) of sequence n.  A null cfirst means a single sequence
// (N = 1): its chunks are 0 .. ceil(length / 64) - 1 and no table is built.
__device__ __forceinline__ void chunk_range(const int32_t* __restrict__ cu,
                                            const int32_t* __restrict__ cfirst, int n, int& cbeg,
                                            int& cend) {
  if (cfirst == nullptr) {
    cbeg = 0;
    cend = (cu[1] - cu[0] + CHUNK - 1) / CHUNK;
  } else {
    cbeg = cfirst[n];
    cend = cfirst[n + 1];
  }
}

// Chunk c -> (first token, length, first token of its sequence).  cfirst is
// non-decreasing with cfirst[0]=0, or null for a single sequence.
__device__ __forceinline__ bool locate_chunk(const int32_t* __restrict__ cu,
                                             const int32_t* __restrict__ cfirst, int N, int c,
                                             int& t0, int& len, int& tseq) {
  if (cfirst == nullptr) {
    tseq = cu[0];
    t0 = tseq + c * CHUNK;
    len = min(CHUNK, cu[1] - t0);
    return len > 0;
  }
  if (c >= cfirst[N]) return false;
  int lo = 0, hi = N;  // cfirst[lo] <= c < cfirst[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cfirst[mid] <= c) lo = mid; else hi = mid;
  }
  tseq = cu[lo];
  t0 = tseq + (c - cfirst[lo]) * CHUNK;
  len = min(CHUNK, cu[lo + 1] - t0);
  return true;
}

// Pairs (u, i), i < u, inside one 8-row half of a 16-row diagonal block,
// ordered by half, then i, then u (u, i are rows within the 16-row block).
__host__ __device__ constexpr int pair8_first(int i) { return 7 * i - (i * (i - 1)) / 2; }
__host__ __device__ constexpr int pair8_i(int q) {
  int i = 0;
  while (i < 6 && pair8_first(i + 1) <= q) ++i;
  return i;
}
__host__ __device__ constexpr int pair_i(int p) { return 8 * (p / 28) + pair8_i(p % 28); }
__host__ __device__ constexpr int pair_u(int p) {
  return 8 * (p / 28) + pair8_i(p % 28) + 1 + (p % 28 - pair8_first(pair8_i(p % 28)));
}
constexpr int NPAIR = 56;
constexpr int NBATCH = 4;  // ceil(56 / 16)
// Pairs (u, i), i < u, inside one 4-row group of a 16-row diagonal block,
// ordered by group, then i, then u (six per group: (0,1) (0,2) (0,3) (1,2)
// (1,3) (2,3) relative to the group's first row).
__host__ __device__ constexpr int pair4_i(int p) {
  return 4 * (p / 6) + (p % 6 < 3 ? 0 : p % 6 < 5 ? 1 : 2);
}
__host__ __device__ constexpr int pair4_u(int p) {
  return 4 * (p / 6) + (p % 6 < 3 ? p % 6 + 1 : p % 6 < 5 ? p % 6 - 1 : 3);
}
constexpr int NPAIR4 = 24;
constexpr int NBATCH4 = 2;  // ceil(24 / 16)

template <typename MT> struct IntraLds {
  static constexpr int ROWL = sizeof(MT) == 2 ? 136 : 132;  // padded row of 128 channels
  static constexpr int TL = sizeof(MT) == 2 ? 72 : 68;      // padded row of 64 tokens
  static constexpr int AL = 68;                              // fp32 64x64 row
  // FP32 operands take twice the bytes: their 128-channel contractions run as
  // NP = 2 passes over 64-channel halves (lanes 32p..32p+31 hold channels
  // 64p..64p+63) through half-width buffers of row stride ROWP, so the kernel
  // fits two workgroups per CU like the bf16 one.
  static constexpr int NP = sizeof(MT) == 2 ? 1 : 2;
  static constexpr int ROWP = NP == 1 ? ROWL : 68;
  static constexpr bool TS_ALIAS = sizeof(MT) == 4;  // FP32: the "scaled" T is T itself
  // fixed part
  static constexpr int O_BETA = 0;                  // float[64]
  static constexpr int O_RK = O_BETA + 256;         // float[64]
  static constexpr int O_RQ = O_RK + 256;           // float[64]
  static constexpr int O_TOT = O_RQ + 256;          // float[4][128] block decay products
  static constexpr int O_A0 = O_TOT + 2048;         // float[4][128] first-row decay of each block
  static constexpr int O_A = O_A0 + 2048;           // float[64][AL] strictly-lower A
  static constexpr int O_U = O_A + 64 * AL * 4;     // union region
  // union, phase 1: per wave private rows: raw k [16], raw q [16], pair vectors [16]
  static constexpr int PRIV_ROWS = 48;
  static constexpr int PRIV_BYTES = PRIV_ROWS * ROWP * (int)sizeof(MT);
  // union, phase 2: cross-block operands: A-side rows (kL,qL for R=1..3) 96, B-side 96
  static constexpr int X_ROWS = 192;
  // union, phase 3: T (float [64][AL]), T-scaled operand (MT [64][TL], or T itself),
  // transposed operand (MT [128 / NP][TL])
  static constexpr int O_T = 0;
  static constexpr int O_TS = TS_ALIAS ? O_T : O_T + 64 * AL * 4;
  static constexpr int O_XT = TS_ALIAS ? O_T + 64 * AL * 4 : O_TS + 64 * TL * (int)sizeof(MT);
  static constexpr int U_P1 = 4 * PRIV_BYTES;
  static constexpr int U_P2 = X_ROWS * ROWP * (int)sizeof(MT);
  static constexpr int U_P3 = O_XT + (128 / NP) * TL * (int)sizeof(MT);
  // scratch of the 16x16 block substitution (phase 3, before W/U use O_XT)
  static constexpr int O_SCR = TS_ALIAS ? O_XT : O_TS;
  static constexpr int U_BYTES = U_P1 > U_P2 ? (U_P1 > U_P3 ? U_P1 : U_P3) : (U_P2 > U_P3 ? U_P2 : U_P3);
  static constexpr int BYTES = O_U + U_BYTES;
};

// A pointer that is the same in every lane of the wave, moved to scalar
// registers so that addressing from it is scalar arithmetic.
template <typename T> __device__ __forceinline__ const T* wave_uniform(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Short causal convolution (width 4) of a wave's 16 rows, channels c0 and
// c0+1, in place: x[j] <- act(b + sum_i w[i] x[j-3+i]), rows before j = 0
// taken from hist[0..2] (zero outside the sequence).  Computed from the last
// row backwards so every row still reads raw inputs.  Weights and bias are
// rounded to the activation dtype, products accumulate in FP32, the result is
// rounded to the activation dtype (the convolution's forward keeps it).
template <typename TA>
__device__ __forceinline__ void conv16(f32x2 (&x)[16], const f32x2 (&hist)[3], const float* wt,
                                       const float* bs, int c0, bool silu) {
  float w[2][4], b[2];
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[ch][i] = to_f32(from_f32<TA>(wt[(c0 + ch) * 4 + i]));
    b[ch] = bs ? to_f32(from_f32<TA>(bs[c0 + ch])) : 0.0f;
  }
#pragma unroll
  for (int j = 15; j >= 0; --j) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float acc = b[ch];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = j - 3 + i;
        acc = fmaf(w[ch][i], src >= 0 ? x[src][ch] : hist[src + 3][ch], acc);
      }
      if (silu) acc *= sigmoid_f(acc);
      x[j][ch] = to_f32(from_f32<TA>(acc));
    }
  }
}

// Sums over the 64 lanes of a wave of N (32 or 64) values, each lane holding
// one partial of every value.  Exchanges between the lane halves
// (v_permlane32_swap) and between rows of 16 lanes (v_permlane16_swap) halve
// the values twice; DPP steps inside a row (mirror, half mirror, quad xor 2)
// halve them further, each pairing lanes that hold the same values so far.
// Lane l ends with the total of value
//   N = 64: 32 h32 + 16 h16 + (l & 15)
//   N = 32: 16 h32 + 8 h16 + ((l & 15) >> 1)   (lanes l and l^1 alike)
// where h32, h16 (wave_swap_sides) tell which of the two values each swap
// left in this lane.
struct SwapSides { int h32, h16; };
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ SwapSides wave_swap_sides() {
  // a tag goes through the same exchanges as the values
  const auto t32 = __builtin_amdgcn_permlane32_swap(f2u(0.0f), f2u(1.0f), false, false);
  const auto t16 = __builtin_amdgcn_permlane16_swap(f2u(0.0f), f2u(1.0f), false, false);
  return SwapSides{u2f(t32[0]) + u2f(t32[1]) > 0.5f, u2f(t16[0]) + u2f(t16[1]) > 0.5f};
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(x), CTRL, 0xF, 0xF, false));
}
// one DPP halving step: keep value hi (bit set) or lo, add the partner's copy
template <int CTRL> __device__ __forceinline__ float dpp_halve(float lo, float hi, bool bit) {
  return (bit ? hi : lo) + dpp_f<CTRL>(bit ? lo : hi);
}
template <int N> __device__ __forceinline__ float wave_sum_many(const float (&v)[N], int l) {
  static_assert(N == 32 || N == 64, "32 or 64 values");
  constexpr int DPP_MIRROR = 0x140, DPP_HALF_MIRROR = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1;
  float v1[N / 2], v2[N / 4], v3[N / 8], v4[N / 16];
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(f2u(v[k]), f2u(v[k + N / 2]), false, false);
    v1[k] = u2f(r[0]) + u2f(r[1]);
  }
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(f2u(v1[k]), f2u(v1[k + N / 4]), false, false);
    v2[k] = u2f(r[0]) + u2f(r[1]);
  }
  const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1, b1 = (l >> 1) & 1, b0 = l & 1;
#pragma unroll
  for (int k = 0; k < N / 8; ++k) v3[k] = dpp_halve<DPP_MIRROR>(v2[k], v2[k + N / 8], b3);
#pragma unroll
  for (int k = 0; k < N / 16; ++k) v4[k] = dpp_halve<DPP_HALF_MIRROR>(v3[k], v3[k + N / 16], b2);
  if constexpr (N == 64) {
    const float v5[2] = {dpp_halve<DPP_XOR2>(v4[0], v4[2], b1), dpp_halve<DPP_XOR2>(v4[1], v4[3], b1)};
    return dpp_halve<DPP_XOR1>(v5[0], v5[1], b0);
  } else {
    const float t = dpp_halve<DPP_XOR2>(v4[0], v4[1], b1);
    return t + dpp_f<DPP_XOR1>(t);
  }
}

// Index of cross-block combination (R, I), R > I, in 0..5.
__device__ __forceinline__ constexpr int combo(int R, int I) { return (R * (R - 1)) / 2 + I; }

// The work of one (chunk, head): a workgroup of 256 threads; smem is the
// workgroup's LDS buffer of IntraLds<MT>::BYTES bytes, 16-byte aligned.
// Template parameters as for kda_intra_kernel below.
template <typename TA, typename MT, bool CONV, typename LY, bool BWD, bool RECT = false>
__device__ __forceinline__ void intra_chunk(const IntraArgs& p, int chunk, int h, char* smem) {
  static_assert(!(RECT && (CONV || BWD)), "rectangular widths: forward without convolution only");
  typedef IntraLds<MT> L;
  constexpr int ROWL = L::ROWL, TL = L::TL, AL = L::AL;
  float* sBeta = reinterpret_cast<float*>(smem + L::O_BETA);
  float* sRk = reinterpret_cast<float*>(smem + L::O_RK);
  float* sRq = reinterpret_cast<float*>(smem + L::O_RQ);
  float* sTot = reinterpret_cast<float*>(smem + L::O_TOT);
  float* sA0 = reinterpret_cast<float*>(smem + L::O_A0);
  float* sA = reinterpret_cast<float*>(smem + L::O_A);
  char* sU = smem + L::O_U;

  int t0, len, tseq;
  if (!locate_chunk(p.cu, p.cfirst, p.N, chunk, t0, len, tseq)) return;  // uniform over the block

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int H = p.H;
  const int c0 = 2 * l;  // this lane's two channels: c0, c0 + 1
  const TA* __restrict__ gq = reinterpret_cast<const TA*>(p.q);
  const TA* __restrict__ gk = reinterpret_cast<const TA*>(p.k);
  const TA* __restrict__ gv = reinterpret_cast<const TA*>(p.v);
  const TA* __restrict__ gf = reinterpret_cast<const TA*>(p.f);
  const TA* __restrict__ gb = reinterpret_cast<const TA*>(p.b);
  // record slot: chunk modulo the ring length when the records live in a ring
  const int slot = p.ring > 0 ? chunk % p.ring : chunk;
  const size_t rec_off = ((size_t)slot * H + h) * LY::REC_ELEMS;
  MT* __restrict__ gW = reinterpret_cast<MT*>(p.rec) + rec_off + OFF_W;
  MT* __restrict__ gQt = reinterpret_cast<MT*>(p.rec) + rec_off + OFF_QT;
  MT* __restrict__ gKbT = reinterpret_cast<MT*>(p.rec) + rec_off + OFF_KBT;
  MT* __restrict__ gUT = reinterpret_cast<MT*>(p.rec) + rec_off + OFF_UT;
  MT* __restrict__ gP = reinterpret_cast<MT*>(p.rec) + rec_off + OFF_P;

  // ------------------------------------------------------------ phase 1: prep
  // Per lane: rows 16w..16w+15, channels c0, c0+1.  Rows past the chunk end
  // hold q = k = v = 0 and decay 1, which makes every formula exact without
  // special cases (they add nothing to any sum and do not decay the state).
  // All row loads are issued before any use (rows past the end re-read the
  // chunk's first row and are masked), so their latencies overlap.
  const float lam = expf(p.A_log[h]);  // exp(-inf) = 0 gives g = 0 exactly
  // RECT: channel c of a row of width dim; missing channels (c >= dim) read as
  // zero, which leaves q, k, v zero there (and the decay finite)
  auto ld2 = [&](const TA* __restrict__ gx, int tok, int dim) -> f32x2 {
    const TA* row = gx + ((size_t)tok * p.H + h) * dim;
    return f32x2{c0 < dim ? to_f32(row[c0]) : 0.0f, c0 + 1 < dim ? to_f32(row[c0 + 1]) : 0.0f};
  };
  f32x2 dtb;
  if constexpr (RECT) {
    const float* db = p.dt_bias + (size_t)h * p.dk;
    dtb = f32x2{c0 < p.dk ? db[c0] : 0.0f, c0 + 1 < p.dk ? db[c0 + 1] : 0.0f};
  } else {
    dtb = *reinterpret_cast<const f32x2*>(p.dt_bias + (size_t)h * DH + c0);
  }
  float qa[16][2], ka[16][2], aa[16][2];
  // Full chunks (all but a sequence's last) load their rows from one
  // wave-uniform base with scalar row offsets and need no masks.
  const bool full = !RECT && len == CHUNK;  // uniform over the block
  const size_t rstride = (size_t)H * DH;  // elements from one token to the next
  // the three tokens before this wave's first row, for the convolution: zero
  // before the sequence start (and past the chunk's end, where every row of
  // this wave is masked anyway); reads stay inside the chunk or the sequence
  auto conv_hist = [&](const TA* __restrict__ gx, f32x2 (&hx)[3]) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int tok = t0 + 16 * w - 3 + i;
      const bool ok = tok >= tseq && tok < t0 + len;
      const f32x2 x = load2(gx + ((size_t)(ok ? tok : t0) * H + h) * DH + c0);
      hx[i] = ok ? x : f32x2{0.0f, 0.0f};
    }
  };
  const size_t HDt = (size_t)H * DH;  // channels of one tensor
  auto conv_w_of = [&](int tensor) { return p.conv_w + (tensor * HDt + (size_t)h * DH) * 4; };
  auto conv_b_of = [&](int tensor) {
    return p.conv_b ? p.conv_b + tensor * HDt + (size_t)h * DH : (const float*)nullptr;
  };
  {
    f32x2 xq[16], xk[16], xf[16];
    if (full) {
      const size_t wb = ((size_t)(t0 + 16 * w) * H + h) * DH;
      const TA* bq = wave_uniform(gq + wb);
      const TA* bk = wave_uniform(gk + wb);
      const TA* bf = wave_uniform(gf + wb);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        xq[j] = load2(bq + j * rstride + c0);
        xk[j] = load2(bk + j * rstride + c0);
        xf[j] = load2(bf + j * rstride + c0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 16 * w + j;
        if constexpr (RECT) {
          const int tok = t0 + (r < len ? r : 0);
          xq[j] = ld2(gq, tok, p.dk); xk[j] = ld2(gk, tok, p.dk); xf[j] = ld2(gf, tok, p.dk);
        } else {
          const size_t o = ((size_t)(t0 + (r < len ? r : 0)) * H + h) * DH + c0;
          xq[j] = load2(gq + o); xk[j] = load2(gk + o); xf[j] = load2(gf + o);
        }
      }
    }
    if constexpr (CONV) {
      f32x2 hq[3], hk[3];
      conv_hist(gq, hq);
      conv_hist(gk, hk);
      conv16<TA>(xq, hq, conv_w_of(0), conv_b_of(0), c0, p.conv_silu != 0);
      conv16<TA>(xk, hk, conv_w_of(1), conv_b_of(1), c0, p.conv_silu != 0);
    }
    float bl = 0.0f;
    if (l < 16) bl = to_f32(gb[(size_t)(t0 + (16 * w + l < len ? 16 * w + l : 0)) * H + h]);
    if (full) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        qa[j][0] = xq[j][0]; qa[j][1] = xq[j][1];
        ka[j][0] = xk[j][0]; ka[j][1] = xk[j][1];
        aa[j][0] = decay_from_gate(xf[j][0] + dtb[0], lam);
        aa[j][1] = decay_from_gate(xf[j][1] + dtb[1], lam);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool ok = 16 * w + j < len;
        qa[j][0] = ok ? xq[j][0] : 0.0f; qa[j][1] = ok ? xq[j][1] : 0.0f;
        ka[j][0] = ok ? xk[j][0] : 0.0f; ka[j][1] = ok ? xk[j][1] : 0.0f;
        aa[j][0] = ok ? decay_from_gate(xf[j][0] + dtb[0], lam) : 1.0f;
        aa[j][1] = ok ? decay_from_gate(xf[j][1] + dtb[1], lam) : 1.0f;
      }
    }
    if (l < 16) sBeta[16 * w + l] = (16 * w + l < len) ? sigmoid_f(bl) : 0.0f;
  }
  if constexpr (L::NP == 2) {
    // FP32: the norms, the q.k diagonal and the pairs inside each 8-row half
    // are channel sums on the VALU (each lane holds two channels of every row
    // of its wave), summed over the wave; FP32 matrix tiles there would use one
    // entry in sixteen.  The 8 x 8 cross-half block stays on the matrix cores,
    // in two passes over 64-channel halves: the first pass parks its raw
    // partial sums in sA (A entries in place, P entries in the unused upper
    // triangle, transposed); the second adds its own, applies the norms and
    // writes the final entries.  Every entry is read back by the lane that
    // parked it.
    constexpr int RP = L::ROWP;
    MT* priv = reinterpret_cast<MT*>(sU + w * L::PRIV_BYTES);
    MT* pD = priv + 32 * RP;   // rows 32..47 (factor rows of the 8 x 8 block)
    {
      float t0c = 1.0f, t1c = 1.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) { t0c *= aa[j][0]; t1c *= aa[j][1]; }
      sTot[w * DH + c0] = t0c; sTot[w * DH + c0 + 1] = t1c;
      sA0[w * DH + c0] = aa[0][0]; sA0[w * DH + c0 + 1] = aa[0][1];
    }
    const int cl = c0 - 64 * (l >> 5);  // this lane's first channel inside its half
    // each wave touches only its own rows: a compiler-level fence orders its LDS traffic
    auto wsync = [] {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    };
    // entry (ru, ri), ri < ru, of A (va) and P (vp) in pass ps
    auto entry = [&](int ps, int ru, int ri, float va, float vp) {
      float* sa = sA + ru * AL + ri;
      float* sp = sA + ri * AL + ru;
      if (ps == 0) {
        *sa = va;
        *sp = vp;
      } else {
        va += *sa;
        vp += *sp;
        *sa = sBeta[ru] * sRk[ru] * sRk[ri] * va;
        *sp = sRq[ru] * sRk[ri] * vp;
      }
    };
    // norms (sums of squares) and the plain q.k diagonal on the VALU: 48
    // channel sums over this wave's rows, value 16 t + row for t = 0 (k.k),
    // 1 (q.q), 2 (q.k); the raw sums go to sRk, sRq and the diagonal of sA
    {
      float v[64];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = fmaf(ka[j][0], ka[j][0], ka[j][1] * ka[j][1]);
        v[16 + j] = fmaf(qa[j][0], qa[j][0], qa[j][1] * qa[j][1]);
        v[32 + j] = fmaf(qa[j][0], ka[j][0], qa[j][1] * ka[j][1]);
        v[48 + j] = 0.0f;
      }
      const float tot = wave_sum_many<64>(v, l);
      const SwapSides sd = wave_swap_sides();
      const int t = 2 * sd.h32 + sd.h16, r = 16 * w + (l & 15);
      if (t == 0) sRk[r] = tot;
      else if (t == 1) sRq[r] = tot;
      else if (t == 2) sA[r * AL + r] = tot;
      wsync();
      if (l < 16) {
        const float rk = rsqrt_hw(sRk[r] + p.eps);
        const float rq = rsqrt_hw(sRq[r] + p.eps);
        sRk[r] = rk;
        sRq[r] = rq;
        sA[r * AL + r] = rq * rk * sA[r * AL + r];  // P[r][r], decay 1
      }
      wsync();
    }
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const bool mine = (l >> 5) == ps;
      // the decays pass through an empty asm per pass, so the compiler cannot
      // form the products of both passes once and keep them all live
      float la[16][2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        la[j][0] = aa[j][0]; la[j][1] = aa[j][1];
        asm volatile("" : "+v"(la[j][0]), "+v"(la[j][1]));
      }
      // diagonal block rows 8..15 x columns 0..7, factorised about row 8:
      // k row factors (rows 8..15) and column factors (rows 0..7), then q row factors
      float ra0[8], ra1[8];
      if (mine) {
        float x0 = 1.0f, x1 = 1.0f;
#pragma unroll
        for (int j = 8; j < 16; ++j) {
          if (j > 8) { x0 *= la[j][0]; x1 *= la[j][1]; }
          ra0[j - 8] = x0; ra1[j - 8] = x1;
          store2(pD + j * RP + cl, ka[j][0] * x0, ka[j][1] * x1);
        }
        float y0 = la[8][0], y1 = la[8][1];
#pragma unroll
        for (int j = 7; j >= 0; --j) {
          store2(pD + j * RP + cl, ka[j][0] * y0, ka[j][1] * y1);
          y0 *= la[j][0]; y1 *= la[j][1];
        }
      }
      wsync();
      f32x4 c8a = {0, 0, 0, 0};
      c8a = mma16_rows<MT, CHUNK>(pD, RP, pD, RP, c8a, l);
      wsync();
      if (mine) {
#pragma unroll
        for (int j = 8; j < 16; ++j) store2(pD + j * RP + cl, qa[j][0] * ra0[j - 8], qa[j][1] * ra1[j - 8]);
      }
      wsync();
      f32x4 c8p = {0, 0, 0, 0};
      c8p = mma16_rows<MT, CHUNK>(pD, RP, pD, RP, c8p, l);
      {
        const int n = l & 15, m0 = 4 * (l >> 4);
        if (m0 >= 8 && n < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) entry(ps, 16 * w + m0 + e, 16 * w + n, c8a[e], c8p[e]);
        }
      }
      wsync();
    }
    // Pairs (u, i), i < u, inside each 8-row half: the channel sums on the
    // VALU.  Each lane forms its two channels' share of
    //   A[u][i] ~ k_u . (k_i prod_{i<j<=u} a_j),   P[u][i] ~ q_u . (same),
    // 16 pairs (32 values) per batch, and the wave sums them.  The norms are
    // complete by now, so the entries are written in their final form.
    {
      const SwapSides sd = wave_swap_sides();
      const int b3 = (l >> 3) & 1, b2 = (l >> 2) & 1, b1 = (l >> 1) & 1;
      float kd0 = 0.0f, kd1 = 0.0f;
#pragma unroll
      for (int bt = 0; bt < NBATCH; ++bt) {
        float v[32];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int pp = 16 * bt + n;
          if (pp < NPAIR) {
            const int i = pair_i(pp), u = pair_u(pp);
            if (u == i + 1) { kd0 = ka[i][0] * aa[u][0]; kd1 = ka[i][1] * aa[u][1]; }
            else { kd0 *= aa[u][0]; kd1 *= aa[u][1]; }
            v[2 * n] = fmaf(ka[u][0], kd0, ka[u][1] * kd1);
            v[2 * n + 1] = fmaf(qa[u][0], kd0, qa[u][1] * kd1);
          } else {
            v[2 * n] = 0.0f;
            v[2 * n + 1] = 0.0f;
          }
        }
        const float tot = wave_sum_many<32>(v, l);
        // value 2n + ap, n = 8 h32 + 4 h16 + 2 b3 + b2, ap = b1 (0: A, 1: P)
        if ((l & 1) == 0) {
          const int pp = 16 * bt + 8 * sd.h32 + 4 * sd.h16 + 2 * b3 + b2;
          if (pp < NPAIR) {
            const int ru = 16 * w + pair_u(pp), ri = 16 * w + pair_i(pp);
            if (b1) sA[ri * AL + ru] = sRq[ru] * sRk[ri] * tot;
            else sA[ru * AL + ri] = sBeta[ru] * sRk[ru] * sRk[ri] * tot;
          }
        }
      }
    }
    wsync();
  } else {
    // raw rows for the MFMA work inside the diagonal block (wave-private)
    MT* priv = reinterpret_cast<MT*>(sU + w * L::PRIV_BYTES);
    MT* pK = priv;               // rows 0..15
    MT* pQ = priv + 16 * ROWL;   // rows 16..31
    MT* pD = priv + 32 * ROWL;   // rows 32..47 (pair vectors)
  #pragma unroll
    for (int j = 0; j < 16; ++j) {
      store2(pK + j * ROWL + c0, ka[j][0], ka[j][1]);
      store2(pQ + j * ROWL + c0, qa[j][0], qa[j][1]);
    }
    {
      float t0c = 1.0f, t1c = 1.0f;
  #pragma unroll
      for (int j = 0; j < 16; ++j) { t0c *= aa[j][0]; t1c *= aa[j][1]; }
      sTot[w * DH + c0] = t0c; sTot[w * DH + c0 + 1] = t1c;
      sA0[w * DH + c0] = aa[0][0]; sA0[w * DH + c0 + 1] = aa[0][1];
    }
    // From here to the end of the diagonal-block work each wave touches only
    // its own rows: LDS traffic of one wave is processed in program order, so a
    // compiler-level fence is all the ordering needed.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // Norms (sum of squares) and the plain q.k diagonal via MFMA on the raw rows.
    {
      f32x4 ckk = {0, 0, 0, 0}, cqq = {0, 0, 0, 0}, cqk = {0, 0, 0, 0};
      ckk = mma16_rows<MT, DH>(pK, ROWL, pK, ROWL, ckk, l);
      cqq = mma16_rows<MT, DH>(pQ, ROWL, pQ, ROWL, cqq, l);
      cqk = mma16_rows<MT, DH>(pQ, ROWL, pK, ROWL, cqk, l);
      const int n = l & 15, m0 = 4 * (l >> 4);
      if (n >= m0 && n < m0 + 4) {
        const int e = n - m0;
        const int r = 16 * w + n;
        const float rk = rsqrt_hw(ckk[e] + p.eps);
        const float rq = rsqrt_hw(cqq[e] + p.eps);
        sRk[r] = rk;
        sRq[r] = rq;
        sA[r * AL + r] = rq * rk * cqk[e];  // P[r][r], decay 1
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // Diagonal block, rows 8..15 x columns 0..7: factorised about row 8,
    //   A[u][i] ~ (k_u prod_{8<j<=u} a_j) . (k_i prod_{i<j<=8} a_j),
    // both factors <= 1.  X8 rows 0..7 hold the column factors, rows 8..15 the
    // row factors of k (then of q for P); one MFMA tile each, block [8..15][0..7].
    {
      float x0 = 1.0f, x1 = 1.0f;
      float ra0[8], ra1[8];
  #pragma unroll
      for (int j = 8; j < 16; ++j) {
        if (j > 8) { x0 *= aa[j][0]; x1 *= aa[j][1]; }
        ra0[j - 8] = x0; ra1[j - 8] = x1;
        store2(pD + j * ROWL + c0, ka[j][0] * x0, ka[j][1] * x1);
      }
      float y0 = aa[8][0], y1 = aa[8][1];
  #pragma unroll
      for (int j = 7; j >= 0; --j) {
        store2(pD + j * ROWL + c0, ka[j][0] * y0, ka[j][1] * y1);
        y0 *= aa[j][0]; y1 *= aa[j][1];
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 ca = {0, 0, 0, 0};
      ca = mma16_rows<MT, DH>(pD, ROWL, pD, ROWL, ca, l);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
  #pragma unroll
      for (int j = 8; j < 16; ++j) store2(pD + j * ROWL + c0, qa[j][0] * ra0[j - 8], qa[j][1] * ra1[j - 8]);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 cp = {0, 0, 0, 0};
      cp = mma16_rows<MT, DH>(pD, ROWL, pD, ROWL, cp, l);
      const int n = l & 15, m0 = 4 * (l >> 4);
      if (m0 >= 8 && n < 8) {
        const int ri = 16 * w + n;
        const float rki = sRk[ri];
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ru = 16 * w + m0 + e;
          sA[ru * AL + ri] = sBeta[ru] * sRk[ru] * rki * ca[e];
          sA[ri * AL + ru] = sRq[ru] * rki * cp[e];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    // Rows 4..7 x columns 0..3 and rows 12..15 x columns 8..11: factorised
    // about rows 4 and 12 in the same way, both blocks from one tile: X8 rows
    // 0..3 and 8..11 hold the column factors, rows 4..7 and 12..15 the row
    // factors of k (then of q for P).
    {
      float ra0[8], ra1[8];
  #pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int m = 8 * hf + 4;  // reference row
        float x0 = 1.0f, x1 = 1.0f;
  #pragma unroll
        for (int j = m; j < m + 4; ++j) {
          if (j > m) { x0 *= aa[j][0]; x1 *= aa[j][1]; }
          ra0[4 * hf + j - m] = x0; ra1[4 * hf + j - m] = x1;
          store2(pD + j * ROWL + c0, ka[j][0] * x0, ka[j][1] * x1);
        }
        float y0 = aa[m][0], y1 = aa[m][1];
  #pragma unroll
        for (int j = m - 1; j >= m - 4; --j) {
          store2(pD + j * ROWL + c0, ka[j][0] * y0, ka[j][1] * y1);
          y0 *= aa[j][0]; y1 *= aa[j][1];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 ca = {0, 0, 0, 0};
      ca = mma16_rows<MT, DH>(pD, ROWL, pD, ROWL, ca, l);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
  #pragma unroll
      for (int hf = 0; hf < 2; ++hf)
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 8 * hf + 4 + j;
          store2(pD + r * ROWL + c0, qa[r][0] * ra0[4 * hf + j], qa[r][1] * ra1[4 * hf + j]);
        }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 cp = {0, 0, 0, 0};
      cp = mma16_rows<MT, DH>(pD, ROWL, pD, ROWL, cp, l);
      const int n = l & 15, g = l >> 4;
      if ((g == 1 && n < 4) || (g == 3 && n >= 8 && n < 12)) {
        const int ri = 16 * w + n;
        const float rki = sRk[ri];
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ru = 16 * w + 4 * g + e;
          sA[ru * AL + ri] = sBeta[ru] * sRk[ru] * rki * ca[e];
          sA[ri * AL + ru] = sRq[ru] * rki * cp[e];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    // Inside each 4-row group: pair vectors kd_(u,i)[c] = k_i[c] prod_{i<j<=u} a_j[c],
    // 16 per batch; MFMA k.kd and q.kd; keep the (u, column) entry.
    {
      float d0 = 1.0f, d1 = 1.0f;
  #pragma unroll
      for (int bt = 0; bt < NBATCH4; ++bt) {
  #pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int pp = 16 * bt + n;
          if (pp < NPAIR4) {
            const int i = pair4_i(pp), u = pair4_u(pp);
            if (u == i + 1) { d0 = aa[u][0]; d1 = aa[u][1]; }
            else { d0 *= aa[u][0]; d1 *= aa[u][1]; }
            store2(pD + n * ROWL + c0, ka[i][0] * d0, ka[i][1] * d1);
          } else {
            store2(pD + n * ROWL + c0, 0.0f, 0.0f);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        f32x4 ca = {0, 0, 0, 0}, cp = {0, 0, 0, 0};
        ca = mma16_rows<MT, DH>(pK, ROWL, pD, ROWL, ca, l);
        cp = mma16_rows<MT, DH>(pQ, ROWL, pD, ROWL, cp, l);
        {
          const int n = l & 15, pp = 16 * bt + n;
          if (pp < NPAIR4) {
            const int i = pair4_i(pp), u = pair4_u(pp);
            const int m0 = 4 * (l >> 4);
            if (u >= m0 && u < m0 + 4) {
              const int e = u - m0;
              const float va = e == 0 ? ca[0] : e == 1 ? ca[1] : e == 2 ? ca[2] : ca[3];
              const float vp = e == 0 ? cp[0] : e == 1 ? cp[1] : e == 2 ? cp[2] : cp[3];
              const int ru = 16 * w + u, ri = 16 * w + i;
              sA[ru * AL + ri] = sBeta[ru] * sRk[ru] * sRk[ri] * va;
              sA[ri * AL + ru] = sRq[ru] * sRk[ri] * vp;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------- phase 2: cross-block
  // Per channel: product of decays of the blocks before / after mine.
  float pb[2] = {1.0f, 1.0f}, sa[2] = {1.0f, 1.0f};
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    if (x < w) { pb[0] *= sTot[x * DH + c0]; pb[1] *= sTot[x * DH + c0 + 1]; }
    if (x > w) { sa[0] *= sTot[x * DH + c0]; sa[1] *= sTot[x * DH + c0 + 1]; }
  }
  {
    // Qt = q^ * prod_{j<=r} a_j ;  KbT = (k^ * prod_{j>r} a_j)^T ; Gam
    float e0 = pb[0], e1 = pb[1];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * w + j;
      e0 *= aa[j][0]; e1 *= aa[j][1];
      const float rq = sRq[r];
      if constexpr (LY::TRANSPOSED_QT_P) {
        gQt[LY::qt(r, c0)] = from_f32<MT>(qa[j][0] * rq * e0);
        gQt[LY::qt(r, c0 + 1)] = from_f32<MT>(qa[j][1] * rq * e1);
      } else {
        store2(gQt + LY::qt(r, c0), qa[j][0] * rq * e0, qa[j][1] * rq * e1);
      }
    }
    float s0 = sa[0], s1 = sa[1];
    float kb0[16], kb1[16];
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      const float rk = sRk[16 * w + j];
      kb0[j] = ka[j][0] * rk * s0;
      kb1[j] = ka[j][1] * rk * s1;
      s0 *= aa[j][0]; s1 *= aa[j][1];
    }
    if constexpr (sizeof(MT) == 2 && std::is_same<LY, Frag<MT>>::value) {
      // a 16-byte unit of Kb^T is 8 consecutive tokens of one channel: this
      // lane holds four whole units (channels c0, c0 + 1; tokens 16w .. 16w+7
      // and 16w+8 .. 16w+15), written with one 16-byte store each (8-byte
      // half-unit stores took about 1 % longer over the kernel)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 x0, x1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x0[i] = cvt_pair(f32x2{kb0[8 * hh + 2 * i], kb0[8 * hh + 2 * i + 1]});
          x1[i] = cvt_pair(f32x2{kb1[8 * hh + 2 * i], kb1[8 * hh + 2 * i + 1]});
        }
        *reinterpret_cast<u32x4*>(gKbT + LY::kb(c0, 16 * w + 8 * hh)) = x0;
        *reinterpret_cast<u32x4*>(gKbT + LY::kb(c0 + 1, 16 * w + 8 * hh)) = x1;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        store4(gKbT + LY::kb(c0, 16 * w + j), f32x4{kb0[j], kb0[j + 1], kb0[j + 2], kb0[j + 3]});
        store4(gKbT + LY::kb(c0 + 1, 16 * w + j),
               f32x4{kb1[j], kb1[j + 1], kb1[j + 2], kb1[j + 3]});
        if constexpr (BWD) {
          float* gk = p.kbr + ((size_t)chunk * H + h) * CHUNK * DH;
#pragma unroll
          for (int e = 0; e < 4; ++e) store2(gk + (16 * w + j + e) * DH + c0, kb0[j + e], kb1[j + e]);
        }
      }
    }
    if (w == 0) {
      float g0 = 1.0f, g1 = 1.0f;
#pragma unroll
      for (int x = 0; x < 4; ++x) { g0 *= sTot[x * DH + c0]; g1 *= sTot[x * DH + c0 + 1]; }
      *reinterpret_cast<f32x2*>(p.gam + ((size_t)slot * H + h) * DH + c0) = f32x2{g0, g1};
    }
  }
  // Cross-block operands.  A-side (rows of block R = w >= 1, reference = the
  // block's first row): kL = k * prod_{16R<j<=r} a_j, qL likewise.  B-side
  // (rows of block I = w for every R > w): kR = k * prod_{i<j<=16R} a_j.
  if constexpr (L::NP == 2) {
    // FP32: the same operands and products in two 64-channel passes
    constexpr int RP = L::ROWP;
    MT* xA = reinterpret_cast<MT*>(sU);            // [3][32] rows: kL then qL of R=1..3
    MT* xB = reinterpret_cast<MT*>(sU) + 96 * RP;  // [6][16] rows
    const int cl = c0 - 64 * (l >> 5);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      if ((l >> 5) == ps) {
        if (w >= 1) {
          float x0 = 1.0f, x1 = 1.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (j > 0) { x0 *= aa[j][0]; x1 *= aa[j][1]; }
            store2(xA + ((w - 1) * 32 + j) * RP + cl, ka[j][0] * x0, ka[j][1] * x1);
            store2(xA + ((w - 1) * 32 + 16 + j) * RP + cl, qa[j][0] * x0, qa[j][1] * x1);
          }
        }
        if (w <= 2) {
          float ks0[16], ks1[16];
          float s0 = 1.0f, s1 = 1.0f;
#pragma unroll
          for (int j = 15; j >= 0; --j) {
            ks0[j] = ka[j][0] * s0; ks1[j] = ka[j][1] * s1;
            s0 *= aa[j][0]; s1 *= aa[j][1];
          }
#pragma unroll
          for (int R = 1; R < 4; ++R) {
            if (R > w) {
              float k0 = sA0[R * DH + c0], k1 = sA0[R * DH + c0 + 1];
#pragma unroll
              for (int x = 1; x < 4; ++x)
                if (x > w && x < R) { k0 *= sTot[x * DH + c0]; k1 *= sTot[x * DH + c0 + 1]; }
              MT* dst = xB + combo(R, w) * 16 * RP;
#pragma unroll
              for (int j = 0; j < 16; ++j) store2(dst + j * RP + cl, ks0[j] * k0, ks1[j] * k1);
            }
          }
        }
      }
      __syncthreads();
      // the first pass parks its partial sums (A in place, P transposed into
      // the upper triangle of sA); the second adds its own and finalises
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int tp = 3 * w + t;  // 0..11
        const int cmb = tp >> 1, isq = tp & 1;
        const int R = cmb == 0 ? 1 : cmb <= 2 ? 2 : 3;
        const int I = cmb - (R * (R - 1)) / 2;
        f32x4 cx = {0, 0, 0, 0};
        cx = mma16_rows<MT, CHUNK>(xA + ((R - 1) * 32 + 16 * isq) * RP, RP, xB + cmb * 16 * RP, RP,
                                   cx, l);
        const int n = l & 15, m0 = 4 * (l >> 4);
        const int ri = 16 * I + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ru = 16 * R + m0 + e;
          float* slot = isq ? sA + ri * AL + ru : sA + ru * AL + ri;
          if (ps == 0) {
            *slot = cx[e];
          } else {
            const float v = *slot + cx[e];
            *slot = isq ? sRq[ru] * sRk[ri] * v : sBeta[ru] * sRk[ru] * sRk[ri] * v;
          }
        }
      }
      __syncthreads();
    }
  } else {
    MT* xA = reinterpret_cast<MT*>(sU);              // [3][32] rows: kL then qL of R=1..3
    MT* xB = reinterpret_cast<MT*>(sU) + 96 * ROWL;  // [6][16] rows
    if (w >= 1) {
      float x0 = 1.0f, x1 = 1.0f;
  #pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j > 0) { x0 *= aa[j][0]; x1 *= aa[j][1]; }
        store2(xA + ((w - 1) * 32 + j) * ROWL + c0, ka[j][0] * x0, ka[j][1] * x1);
        store2(xA + ((w - 1) * 32 + 16 + j) * ROWL + c0, qa[j][0] * x0, qa[j][1] * x1);
      }
    }
    if (w <= 2) {
      // suffix within my block, excluding the row itself
      float ks0[16], ks1[16];
      float s0 = 1.0f, s1 = 1.0f;
  #pragma unroll
      for (int j = 15; j >= 0; --j) {
        ks0[j] = ka[j][0] * s0; ks1[j] = ka[j][1] * s1;
        s0 *= aa[j][0]; s1 *= aa[j][1];
      }
  #pragma unroll
      for (int R = 1; R < 4; ++R) {
        if (R > w) {
          // kappa = prod of whole blocks strictly between w and R, times the
          // decay of the reference row 16R
          float k0 = sA0[R * DH + c0], k1 = sA0[R * DH + c0 + 1];
  #pragma unroll
          for (int x = 1; x < 4; ++x)
            if (x > w && x < R) { k0 *= sTot[x * DH + c0]; k1 *= sTot[x * DH + c0 + 1]; }
          MT* dst = xB + combo(R, w) * 16 * ROWL;
  #pragma unroll
          for (int j = 0; j < 16; ++j) store2(dst + j * ROWL + c0, ks0[j] * k0, ks1[j] * k1);
        }
      }
    }
    __syncthreads();
    // 12 tile products (R, I, k|q), three per wave.
  #pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int tp = 3 * w + t;  // 0..11
      const int cmb = tp >> 1, isq = tp & 1;
      const int R = cmb == 0 ? 1 : cmb <= 2 ? 2 : 3;
      const int I = cmb - (R * (R - 1)) / 2;
      f32x4 c = {0, 0, 0, 0};
      c = mma16_rows<MT, DH>(xA + ((R - 1) * 32 + 16 * isq) * ROWL, ROWL, xB + cmb * 16 * ROWL, ROWL,
                             c, l);
      const int n = l & 15, m0 = 4 * (l >> 4);
      const int ri = 16 * I + n;
  #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ru = 16 * R + m0 + e;
        if (isq) sA[ri * AL + ru] = sRq[ru] * sRk[ri] * c[e];
        else sA[ru * AL + ri] = sBeta[ru] * sRk[ru] * sRk[ri] * c[e];
      }
    }
  }
  if constexpr (L::NP == 1) __syncthreads();  // (the two-pass FP32 loop ends with one)
  // P to the record.  Every entry P[r][i] (i <= r) was left in LDS at
  // sA[i][r], the upper triangle of the A buffer (A is strictly lower); here
  // it is written in the layout's order (its tiles on or below the diagonal;
  // zeros above the diagonal inside them), 16-byte stores, one fragment per 64 (consecutive lanes: consecutive rows r, so the LDS reads
  // fall in consecutive banks).  The T solve below reads only A's lower part.
  {
    auto pval = [&](int r, int i) { return i <= r ? sA[i * AL + r] : 0.0f; };
    if constexpr (LY::TRANSPOSED_QT_P) {
      // P^T [i][r] (FP32 records): four consecutive rows r per store
      static_assert(sizeof(MT) == 4, "transposed records are FP32");
      for (int f = tid; f < CHUNK * CHUNK / 4; f += 256) {
        const int i = f >> 4, r0 = 4 * (f & 15);
        store4(gP + LY::pm(r0, i), f32x4{pval(r0, i), pval(r0 + 1, i), pval(r0 + 2, i), pval(r0 + 3, i)});
      }
    } else {
      static_assert(LY::P_LOWER_TILES, "forward records hold P's lower tiles");
      // the stored fragments (16 / FE for rows 0..31, then 32 / FE for rows
      // 32..63): lane (r % 32, g) of fragment u of its row tile
      constexpr int FE = LY::FE, F0 = 16 / FE;
      typedef typename std::conditional<sizeof(MT) == 2, bf16x8, f32x4>::type v16;
      for (int f = tid; f < 3 * F0 * 64; f += 256) {
        const int idx = f >> 6, lane = f & 63, g = lane >> 5;
        const int r = (idx >= F0 ? 32 : 0) + (lane & 31), u = idx >= F0 ? idx - F0 : idx;
        v16 x;
#pragma unroll
        for (int q = 0; q < FE; ++q) x[q] = from_f32<MT>(pval(r, LY::pcol(u, g, q)));
        *reinterpret_cast<v16*>(gP + LY::pm(r, LY::pcol(u, g, 0))) = x;
      }
    }
  }

  // ------------------------------------------------- phase 3: T = (I + A)^{-1}
  // Forward substitution, blocked: 4x4 diagonal blocks explicitly, then
  // 4x4-block substitution to the 16x16 diagonal blocks (one wave each), then
  // 16x16-block substitution across waves with FP32 MFMA:
  //   T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI.
  float* sT = reinterpret_cast<float*>(sU + L::O_T);
  // values for the U product, loaded early so their latency hides under the solve
  float v0[16], v1[16];
  if constexpr (CONV) {
    f32x2 xv[16], hv[3];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * w + j;
      xv[j] = load2(gv + ((size_t)(t0 + (r < len ? r : 0)) * H + h) * DH + c0);
    }
    conv_hist(gv, hv);
    conv16<TA>(xv, hv, conv_w_of(2), conv_b_of(2), c0, p.conv_silu != 0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool ok = 16 * w + j < len;
      v0[j] = ok ? xv[j][0] : 0.0f;
      v1[j] = ok ? xv[j][1] : 0.0f;
    }
  } else if (full) {
    const TA* bv = wave_uniform(gv + ((size_t)(t0 + 16 * w) * H + h) * DH);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const f32x2 xv = load2(bv + j * rstride + c0);
      v0[j] = xv[0];
      v1[j] = xv[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * w + j;
      const f32x2 xv = RECT ? ld2(gv, t0 + (r < len ? r : 0), p.dv)
                            : load2(gv + ((size_t)(t0 + (r < len ? r : 0)) * H + h) * DH + c0);
      v0[j] = r < len ? xv[0] : 0.0f;
      v1[j] = r < len ? xv[1] : 0.0f;
    }
  }
  {
    // (a) 4x4 diagonal blocks.  Lane: sub-block sb, row r4, column c4.
    const int sb = l >> 4, r4 = (l >> 2) & 3, c4 = l & 3;
    const int base = 16 * w + 4 * sb;
    const float* ab = sA + base * AL + base;
    const float n10 = ab[1 * AL + 0], n20 = ab[2 * AL + 0], n21 = ab[2 * AL + 1];
    const float n30 = ab[3 * AL + 0], n31 = ab[3 * AL + 1], n32 = ab[3 * AL + 2];
    // column c4 of the inverse: t_c = 1, t_i = -sum_{c<=j<i} n_ij t_j
    float t0v = c4 == 0 ? 1.0f : 0.0f;
    float t1v = c4 == 1 ? 1.0f : (c4 < 1 ? -n10 * t0v : 0.0f);
    float t2v = c4 == 2 ? 1.0f : (c4 < 2 ? -(n20 * t0v + n21 * t1v) : 0.0f);
    float t3v = c4 == 3 ? 1.0f : -(n30 * t0v + n31 * t1v + n32 * t2v);
    const float mine = r4 == 0 ? t0v : r4 == 1 ? t1v : r4 == 2 ? t2v : t3v;
    sT[(base + r4) * AL + base + c4] = mine;
    // zero the rest of this wave's 16x16 diagonal block above the 4x4 diagonal,
    // and with FP32 operands (T is then the W/U operand itself) every block
    // above the 16x16 diagonal; a bf16 operand is converted with those blocks
    // masked instead
    for (int x = l; x < 16 * 16; x += 64) {
      const int rr = x >> 4, cc = x & 15;
      if ((cc >> 2) > (rr >> 2)) sT[(16 * w + rr) * AL + 16 * w + cc] = 0.0f;
    }
    if constexpr (L::TS_ALIAS) {
      for (int x = tid; x < CHUNK * CHUNK; x += 256) {
        const int rr = x >> 6, cc = x & 63;
        if ((cc >> 4) > (rr >> 4)) sT[rr * AL + cc] = 0.0f;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // (b) 4x4-block substitution inside the 16x16 block, by block distance d.
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (l < 16 * (4 - d)) {
        const int I4 = l >> 4, R4 = I4 + d, rr = (l >> 2) & 3, cc = l & 3;
        const int rb = 16 * w + 4 * R4, cb = 16 * w + 4 * I4;
        float y[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float acc = 0.0f;
          for (int J = I4; J < R4; ++J) {
            const float* arow = sA + (rb + m) * AL + 16 * w + 4 * J;
            const float* tcol = sT + (16 * w + 4 * J) * AL + cb + cc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc += arow[j] * tcol[j * AL];
          }
          y[m] = acc;
        }
        const float* trr = sT + (rb + rr) * AL + rb;
        sT[(rb + rr) * AL + cb + cc] = -(trr[0] * y[0] + trr[1] * y[1] + trr[2] * y[2] + trr[3] * y[3]);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  {
    // (c) 16x16 blocks across waves, FP32 MFMA.  Y goes through a per-wave
    // scratch tile so it can feed the second product as its B operand.
    float* sY = reinterpret_cast<float*>(sU + L::O_SCR) + w * 16 * 20;
    const int nn = l & 15, m0 = 4 * (l >> 4);
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      if (w < 4 - dist) {
        const int I = w, R = w + dist;
        f32x4 y = {0, 0, 0, 0};
        const float* a = sA + (16 * R) * AL + 16 * I;
        const float* b = sT + (16 * I) * AL + 16 * I;
        if (dist == 1) y = mma16_f32_kn<16>(a, AL, b, AL, y, l);
        else if (dist == 2) y = mma16_f32_kn<32>(a, AL, b, AL, y, l);
        else y = mma16_f32_kn<48>(a, AL, b, AL, y, l);
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[(m0 + e) * 20 + nn] = y[e];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        f32x4 t = {0, 0, 0, 0};
        t = mma16_f32_kn<16>(sT + (16 * R) * AL + 16 * R, AL, sY, 20, t, l);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * R + m0 + e) * AL + 16 * I + nn] = -t[e];
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------------ phase 4: W and U
  if constexpr (sizeof(MT) == 4) {
    // FP32 operands on bf16 matrix cores: W = T' (Diag(rk) (k * E)) and
    // U = T' v with T' = T Diag(beta), each product from three-piece splits
    // (bf16x6; v from bf16 activations is exact in one piece and takes three
    // terms).  T' and one 64-channel half of the right-hand operand,
    // transposed to [channel][token], are bf16 planes of 64-element rows
    // whose 16-byte chunks are XOR-swizzled by row.
    constexpr int PP = CHUNK * CHUNK;                         // plane stride
    bf16* pX = reinterpret_cast<bf16*>(sU);                   // right-hand planes
    bf16* pT = reinterpret_cast<bf16*>(sU + 3 * PP * 2);      // T' planes
    static_assert(6 * PP * 2 <= L::U_BYTES, "W/U planes fit the union region");
    static_assert(CHUNK * AL * 4 <= 3 * PP * 2, "the FP32 T lies below the T' planes");
    auto sw64 = [](int r, int k) { return r * 64 + ((((k >> 3) ^ r) & 7) << 3) + (k & 7); };
    // (T is lower triangular, its blocks above the 16x16 diagonal zeroed)
    for (int x4 = tid; x4 < PP / 4; x4 += 256) {
      const int r = x4 >> 4, i4 = 4 * (x4 & 15);
      const f32x4 tv = *reinterpret_cast<const f32x4*>(sT + r * AL + i4);
      if constexpr (BWD)
        *reinterpret_cast<f32x4*>(p.tmat + ((size_t)chunk * H + h) * PP + r * CHUNK + i4) = tv;
      f32x4 tb;
#pragma unroll
      for (int e = 0; e < 4; ++e) tb[e] = tv[e] * sBeta[i4 + e];
      store_pieces4(pT + sw64(r, i4), PP, tb);
    }
    __syncthreads();  // the FP32 T is no longer read; the right-hand planes may overwrite it
    // one product: tiles of 16 x 16 over the 64 tokens (two steps of 32),
    // rows ra of the planes at A, rows rb at B; B in one piece when exact
    auto tile = [&](const bf16* A, int ra, const bf16* B, int rb, bool b_exact) {
      f32x4 c = {0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int k = 32 * st + 8 * (l >> 4);
        bf16x8 a[3], bb[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) a[q] = *reinterpret_cast<const bf16x8*>(A + q * PP + sw64(ra, k));
        bb[0] = *reinterpret_cast<const bf16x8*>(B + sw64(rb, k));
        if (b_exact) {
          c = mma_x3b(a, bb[0], c);
        } else {
          bb[1] = *reinterpret_cast<const bf16x8*>(B + PP + sw64(rb, k));
          bb[2] = *reinterpret_cast<const bf16x8*>(B + 2 * PP + sw64(rb, k));
          c = mma_x6_16(a, bb, c);
        }
      }
      return c;
    };
    // W, per channel half: the lanes owning the half store (rk k E) transposed
#pragma unroll 1
    for (int ps = 0; ps < 2; ++ps) {
      const int cl = c0 - 64 * ps;
      if ((l >> 5) == ps) {
        float kg0[16], kg1[16];
        float e0 = pb[0], e1 = pb[1];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          e0 *= aa[j][0]; e1 *= aa[j][1];
          const float rk = sRk[16 * w + j];
          kg0[j] = ka[j][0] * e0 * rk; kg1[j] = ka[j][1] * e1 * rk;
        }
        if constexpr (BWD) {
          float* gb = p.bw + ((size_t)chunk * H + h) * CHUNK * DH;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float bj = sBeta[16 * w + j];
            store2(gb + (16 * w + j) * DH + c0, kg0[j] * bj, kg1[j] * bj);
          }
        }
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          store_pieces4(pX + sw64(cl, 16 * w + j), PP, f32x4{kg0[j], kg0[j + 1], kg0[j + 2], kg0[j + 3]});
          store_pieces4(pX + sw64(cl + 1, 16 * w + j), PP, f32x4{kg1[j], kg1[j + 1], kg1[j + 2], kg1[j + 3]});
        }
      }
      __syncthreads();
      // W^T tiles (channel block mtl of the half, token block nt), four per wave
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tl = 4 * w + t, mtl = tl >> 2, nt = tl & 3, mt = 4 * ps + mtl;
        const f32x4 c = tile(pX, 16 * mtl + (l & 15), pT, 16 * nt + (l & 15), false);
        // c[e] = W^T[16mt + 4(l/16) + e][16nt + l%16] = W[tok][ch..ch+3]
        const int tok = 16 * nt + (l & 15), ch = 16 * mt + 4 * (l >> 4);
        store4(gW + LY::a(tok, ch), c);
        if constexpr (BWD) {
          float* gwt = p.wt + ((size_t)chunk * H + h) * DH * CHUNK;
#pragma unroll
          for (int e = 0; e < 4; ++e) gwt[(ch + e) * CHUNK + tok] = c[e];
        }
      }
      __syncthreads();
    }
    // U = T' v, per value half (beta is in T')
    constexpr bool V_EXACT = sizeof(TA) == 2;  // v from bf16 activations (or their convolution)
#pragma unroll 1
    for (int ps = 0; ps < 2; ++ps) {
      const int cl = c0 - 64 * ps;
      if ((l >> 5) == ps) {
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const f32x4 a0 = f32x4{v0[j], v0[j + 1], v0[j + 2], v0[j + 3]};
          const f32x4 a1 = f32x4{v1[j], v1[j + 1], v1[j + 2], v1[j + 3]};
          if constexpr (V_EXACT) {
            *reinterpret_cast<u32x2*>(pX + sw64(cl, 16 * w + j)) =
                u32x2{cvt_pair(f32x2{a0[0], a0[1]}), cvt_pair(f32x2{a0[2], a0[3]})};
            *reinterpret_cast<u32x2*>(pX + sw64(cl + 1, 16 * w + j)) =
                u32x2{cvt_pair(f32x2{a1[0], a1[1]}), cvt_pair(f32x2{a1[2], a1[3]})};
          } else {
            store_pieces4(pX + sw64(cl, 16 * w + j), PP, a0);
            store_pieces4(pX + sw64(cl + 1, 16 * w + j), PP, a1);
          }
        }
      }
      __syncthreads();
      // U tiles (token block w, value block t of the half)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int nt = 4 * ps + t;
        const f32x4 c = tile(pT, 16 * w + (l & 15), pX, 16 * t + (l & 15), V_EXACT);
        // c[e] = U[16w + 4(l/16) + e][16nt + l%16]: four consecutive tokens
        const int dv = 16 * nt + (l & 15), tok = 16 * w + 4 * (l >> 4);
        store4(gUT + LY::u(tok, dv), c);
      }
      if (ps == 0) __syncthreads();
    }
  } else {
    MT* sTs = reinterpret_cast<MT*>(sU + L::O_TS);  // scaled T, row-major [64][TL]
    MT* sXt = reinterpret_cast<MT*>(sU + L::O_XT);  // transposed operand [128 / NP][TL]
    // W = T (Diag(beta rk) (k * E)),  U = T (Diag(beta) v): the row scales go
    // on the right-hand operands, T is converted once (FP32: T is used as is).
    // (T is lower triangular: entries above the 16x16 block diagonal were not
    // written and read as zero here)
    for (int x = tid; x < CHUNK * CHUNK; x += 256) {
      const int r = x >> 6, i = x & 63;
      const float tv = (i >> 4) > (r >> 4) ? 0.0f : sT[r * AL + i];
      if constexpr (!L::TS_ALIAS) sTs[r * TL + i] = from_f32<MT>(tv);
      if constexpr (BWD) p.tmat[((size_t)chunk * H + h) * CHUNK * CHUNK + x] = tv;
    }
  #pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float bj = sBeta[16 * w + j];
      v0[j] *= bj; v1[j] *= bj;
    }
    // Each product in NP passes over channel halves (NP = 1 for bf16): the
    // transposed operand holds 128 / NP channels; lanes whose channels fall in
    // the pass form and write them.
    constexpr int NP = L::NP, CB = 8 / NP;  // channel blocks of 16 per pass
  #pragma unroll 1
    for (int ps = 0; ps < NP; ++ps) {
      const int cl = c0 - 64 * ps;
      if (NP == 1 || (l >> 5) == ps) {
        float kg0[16], kg1[16];
        float e0 = pb[0], e1 = pb[1];
  #pragma unroll
        for (int j = 0; j < 16; ++j) {
          e0 *= aa[j][0]; e1 *= aa[j][1];
          const float sc = sBeta[16 * w + j] * sRk[16 * w + j];
          kg0[j] = ka[j][0] * e0 * sc; kg1[j] = ka[j][1] * e1 * sc;
        }
        if constexpr (BWD) {
          float* gb = p.bw + ((size_t)chunk * H + h) * CHUNK * DH;
  #pragma unroll
          for (int j = 0; j < 16; ++j) store2(gb + (16 * w + j) * DH + c0, kg0[j], kg1[j]);
        }
  #pragma unroll
        for (int j = 0; j < 16; j += 4) {
          store4(sXt + cl * TL + 16 * w + j, f32x4{kg0[j], kg0[j + 1], kg0[j + 2], kg0[j + 3]});
          store4(sXt + (cl + 1) * TL + 16 * w + j, f32x4{kg1[j], kg1[j + 1], kg1[j + 2], kg1[j + 3]});
        }
      }
      __syncthreads();
      // output tiles of W^T: (channel block mt) x (token block nt 0..3); 8 / NP per wave
  #pragma unroll
      for (int t = 0; t < 2 * CB / 2; ++t) {
        const int tile = CB * w + t, mtl = tile >> 2, nt = tile & 3, mt = CB * ps + mtl;
        f32x4 c = {0, 0, 0, 0};
        c = mma16_rows<MT, CHUNK>(sXt + 16 * mtl * TL, TL, sTs + 16 * nt * TL, TL, c, l);
        // c[e] = W^T[16mt + 4(l/16) + e][16nt + l%16] = W[tok][ch..ch+3]
        const int tok = 16 * nt + (l & 15), ch = 16 * mt + 4 * (l >> 4);
        store4(gW + LY::a(tok, ch), c);
        if constexpr (BWD) {
          float* gwt = p.wt + ((size_t)chunk * H + h) * DH * CHUNK;
  #pragma unroll
          for (int e = 0; e < 4; ++e) gwt[(ch + e) * CHUNK + tok] = c[e];
        }
      }
      __syncthreads();
    }
    // U = T (Diag(beta) v)
  #pragma unroll 1
    for (int ps = 0; ps < NP; ++ps) {
      const int cl = c0 - 64 * ps;
      if (NP == 1 || (l >> 5) == ps) {
  #pragma unroll
        for (int j = 0; j < 16; j += 4) {
          store4(sXt + cl * TL + 16 * w + j, f32x4{v0[j], v0[j + 1], v0[j + 2], v0[j + 3]});
          store4(sXt + (cl + 1) * TL + 16 * w + j, f32x4{v1[j], v1[j + 1], v1[j + 2], v1[j + 3]});
        }
      }
      __syncthreads();
      // output tiles of U: (token block mt 0..3) x (value block nt); 8 / NP per wave
  #pragma unroll
      for (int t = 0; t < CB; ++t) {
        const int tile = CB * w + t, mt = tile / CB, ntl = tile % CB, nt = CB * ps + ntl;
        f32x4 c = {0, 0, 0, 0};
        c = mma16_rows<MT, CHUNK>(sTs + 16 * mt * TL, TL, sXt + 16 * ntl * TL, TL, c, l);
        // c[e] = U[16mt + 4(l/16) + e][16nt + l%16]: four consecutive tokens
        const int dv = 16 * nt + (l & 15), tok = 16 * mt + 4 * (l >> 4);
        store4(gUT + LY::u(tok, dv), c);
      }
      if (ps + 1 < NP) __syncthreads();
    }
  }
}

// LY: record layout (Frag for the two-pass forward's state pass, FragW for the
// windowed one, PlainRec for the backward).  BWD: also store T and the W
// product's right-hand operand.  RECT: inputs of key / value widths p.dk,
// p.dv below 128 (zero-padded on load).
//   Forward: a grid of heads x chunks, chunk-major with the last chunk first,
//   so that the records the state pass reads first (every head's first
//   chunks) are the most recently written ones, still in the memory-side
//   cache; consecutive workgroups read neighbouring heads of the same tokens.
//   Backward recomputation: the (chunk, head) grid of the other kernels.
template <typename TA, typename MT, bool CONV, typename LY = Frag<MT>, bool BWD = false,
          bool RECT = false>
__global__ __launch_bounds__(256, 2) void kda_intra_kernel(IntraArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[IntraLds<MT>::BYTES];
  if constexpr (BWD)
    intra_chunk<TA, MT, CONV, LY, BWD, RECT>(p, (int)blockIdx.x, (int)blockIdx.y, smem);
  else  // grid (H, chunks): x = head, y = chunk counted from the last one of the launch
    intra_chunk<TA, MT, CONV, LY, BWD, RECT>(p, p.c0 + (int)gridDim.y - 1 - (int)blockIdx.y,
                                             (int)blockIdx.x, smem);
}

}  // namespace kda
