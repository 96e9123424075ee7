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

#include <type_traits>

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
  const float* init; // [N][H][128 key][128 value] start states, or null (zero)
  float* fin;        // [N][H][128][128] end states, or null (not written)
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

// Per-chunk operands of one lane, loaded one chunk ahead of their use.  The
// record is stored in this kernel's read order (Frag in kda_intra.hpp), so
// every load below is one contiguous 16-byte piece per lane and 1 KB per wave.
// ROLE 0 (waves 0,1): W rows and U values; ROLE 1 (waves 2,3): Qt and P rows.
template <typename MT, int ROLE> struct ScanOps {
  static constexpr int FE = 16 / (int)sizeof(MT);
  typedef typename std::conditional<sizeof(MT) == 2, bf16x8, f32x4>::type v16;
  static constexpr int NX = ROLE == 0 ? 16 / FE : 32 / FE;
  v16 a[64 / FE];   // W or Qt row: 64 key channels
  v16 kb[32 / FE];  // Kb^T row: 32 tokens
  v16 x[NX];        // U values (role 0) or P row (role 1)
  f32x4 gm[4];      // Gam at the wave's 16 state rows
};

template <typename MT, int ROLE>
__device__ __forceinline__ void scan_load(ScanOps<MT, ROLE>& o, const MT* __restrict__ R,
                                          const float* __restrict__ gm, int wp, int w, int l,
                                          int g, int vb) {
  typedef ScanOps<MT, ROLE> O;
  constexpr int FE = O::FE;
  typedef typename O::v16 v16;
  // The loads keep this order everywhere (the scheduling barriers stop the
  // compiler from permuting them differently in the prologue and in the loop,
  // which would make its memory-counter waits at the loop head conservative).
  const MT* A = R + (ROLE == 0 ? OFF_W : OFF_QT) + wp * (64 / FE) * 64 * FE + l * FE;
#pragma unroll
  for (int s = 0; s < 64 / FE; ++s) {
    o.a[s] = *reinterpret_cast<const v16*>(A + s * 64 * FE);
    __builtin_amdgcn_sched_barrier(0);
  }
  const MT* kb = R + OFF_KBT + w * (32 / FE) * 64 * FE + l * FE;
#pragma unroll
  for (int s = 0; s < 32 / FE; ++s) {
    o.kb[s] = *reinterpret_cast<const v16*>(kb + s * 64 * FE);
    __builtin_amdgcn_sched_barrier(0);
  }
  const MT* x = ROLE == 0 ? R + OFF_UT + (vb * 2 + wp) * (16 / FE) * 64 * FE + l * FE
                          : R + OFF_P + wp * (32 / FE) * 64 * FE + l * FE;
#pragma unroll
  for (int s = 0; s < O::NX; ++s) {
    o.x[s] = *reinterpret_cast<const v16*>(x + s * 64 * FE);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    o.gm[e4] = *reinterpret_cast<const f32x4*>(gm + 32 * w + 8 * e4 + 4 * g);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// C += A B over NK contracted values per lane: A from register fragments, B
// from LDS (contiguous NK values at pb), 16-byte LDS reads in both precisions.
template <typename MT, int NK, typename V>
__device__ __forceinline__ f32x16 mma32_frags(const V* afr, const MT* pb, f32x16 c) {
  typedef Mma32<MT> M;
  if constexpr (sizeof(MT) == 2) {
#pragma unroll
    for (int s = 0; s < NK / 8; ++s) c = M::mma(afr[s], *reinterpret_cast<const bf16x8*>(pb + 8 * s), c);
  } else {
#pragma unroll
    for (int s = 0; s < NK / 4; ++s) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(pb + 4 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) c = M::mma(afr[s][e], b4[e], c);
    }
  }
  return c;
}
// C += A B with A read from LDS (contiguous NK values at pa) and B from
// register fragments: the same MFMAs as mma32_frags with the operands
// exchanged, so C comes out transposed.
template <typename MT, int NK, typename V>
__device__ __forceinline__ f32x16 mma32_lds_frags(const MT* pa, const V* bfr, f32x16 c) {
  typedef Mma32<MT> M;
  if constexpr (sizeof(MT) == 2) {
#pragma unroll
    for (int s = 0; s < NK / 8; ++s) c = M::mma(*reinterpret_cast<const bf16x8*>(pa + 8 * s), bfr[s], c);
  } else {
#pragma unroll
    for (int s = 0; s < NK / 4; ++s) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(pa + 4 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) c = M::mma(a4[e], bfr[s][e], c);
    }
  }
  return c;
}
// C += A B, both operands from register fragments (NK values per lane).
template <typename MT, int NK, typename V>
__device__ __forceinline__ f32x16 mma32_rr(const V* afr, const V* bfr, f32x16 c) {
  typedef Mma32<MT> M;
  if constexpr (sizeof(MT) == 2) {
#pragma unroll
    for (int s = 0; s < NK / 8; ++s) c = M::mma(afr[s], bfr[s], c);
  } else {
#pragma unroll
    for (int s = 0; s < NK / 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) c = M::mma(afr[s][e], bfr[s][e], c);
  }
  return c;
}
template <typename V> __device__ __forceinline__ float val_at(const V* f, int q) {
  constexpr int FE = sizeof(f[0][0]) == 2 ? 8 : 4;
  return (float)f[q / FE][q % FE];
}

// One chunk of the state pass for one wave.  ROLE 0 forms D = U - W S0 (and
// publishes it); ROLE 1 forms the output rows.  Both update their 32 rows of
// the running state S.  Two barriers per chunk, the same for every wave.
// `issue` sends the loads of a later chunk; each role issues them where it
// would otherwise wait at a barrier (role 1 while role 0 forms D, role 0
// while role 1 forms the output), so that the in-order load issue stays off
// the step's dependency chain.  With fp32 operands only one chunk is loaded
// ahead, and role 0 issues at the start of the step so that the loads have a
// whole step to arrive.
template <typename MT, typename TO, int ROLE, bool FULL, typename Issue>
__device__ __forceinline__ void scan_step(const ScanArgs& p, const ScanOps<MT, ROLE>& cur, f32x16& S,
                                          MT* sS, MT* sD, int h, int ctok, int len, int vb, int w,
                                          int l, Issue&& issue) {
  typedef ScanLds<MT> L;
  constexpr int SL = L::SL, DL = L::DL;
  const int col = l & 31, g = l >> 5, wp = w & 1;
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
  // Role 0: X = W S0 (rows = 32 tokens, columns = 32 values).  Role 1: the
  // transposed product X = S0^T Qt^T (rows = values, columns = tokens), so
  // that each lane ends up holding one token's run of value columns for the
  // output store.  128 key channels contracted; lane group g covers channels
  // [64g, 64g+64) in both forms.
  f32x16 X;
#pragma unroll
  for (int e = 0; e < 16; ++e) X[e] = 0.0f;
  constexpr bool EARLY = ROLE == 0 && sizeof(MT) == 4;
  if constexpr (EARLY) {
    issue();
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (ROLE == 0) {
    X = mma32_frags<MT, 64>(cur.a, sS + col * SL + 64 * g, X);
    // D = U - W S0 at tokens 32wp + row32(e), value column col
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = val_at(cur.x, 4 * e4 + i) - X[4 * e4 + i];
      store4(sD + col * DL + 32 * wp + 8 * e4 + 4 * g, d);
    }
  } else {
    X = mma32_lds_frags<MT, 64>(sS + col * SL + 64 * g, cur.a, X);
    // X is next used after the barrier; without this the compiler sinks the
    // products below the load issue and the barrier, onto the critical path.
    asm volatile("" : "+a"(X));
    __builtin_amdgcn_sched_barrier(0);
    issue();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // D complete; every wave is done reading S0
  // D^T fragments (lane: value column col, tokens 32g..32g+31): the A operand
  // of the transposed P D product and the B operand of the state update.
  typedef typename ScanOps<MT, ROLE>::v16 v16;
  constexpr int FE = ScanOps<MT, ROLE>::FE;
  v16 dfr[32 / FE];
#pragma unroll
  for (int s = 0; s < 32 / FE; ++s) dfr[s] = *reinterpret_cast<const v16*>(sD + col * DL + 32 * g + FE * s);
  if constexpr (ROLE == 1) {
    // out^T = scale (S0^T Qt^T + D^T P^T): P rows 32wp.. are the columns
    X = mma32_rr<MT, 32>(dfr, cur.x, X);
    // Lane (col, g) holds token 32wp + col at values 8 e4 + 4g + (0..3).  One
    // exchange between the lane halves per pair of e4 gives each lane the
    // eight consecutive values 16 pr + 8g + (0..7), pr = 0, 1: 16-byte
    // (bf16) or 32-byte (fp32) stores of whole 32-byte pieces.
    typedef unsigned u32;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NW = (int)sizeof(TO);  // 32-bit words per four output values
    u32 wd[4][NW];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      if constexpr (sizeof(TO) == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wd[e4][j] = __builtin_bit_cast(u32, bf16x2{(bf16)(p.scale * X[4 * e4 + 2 * j]),
                                                     (bf16)(p.scale * X[4 * e4 + 2 * j + 1])});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wd[e4][j] = __builtin_bit_cast(u32, p.scale * X[4 * e4 + j]);
      }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(wd[2 * pr][j], wd[2 * pr + 1][j], false, false);
        wd[2 * pr][j] = r[0];
        wd[2 * pr + 1][j] = r[1];
      }
    const int tk = 32 * wp + col;
    // full chunks store without a branch, which keeps the memory-counter
    // waits of the loop exact; only a sequence's last chunk is masked
    if (FULL || tk < len) {
      u32x4* o = reinterpret_cast<u32x4*>(out + ((size_t)(ctok + tk) * p.H + h) * DH + DVB * vb + 8 * g);
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        if constexpr (sizeof(TO) == 2) {
          o[2 * pr] = u32x4{wd[2 * pr][0], wd[2 * pr][1], wd[2 * pr + 1][0], wd[2 * pr + 1][1]};
        } else {
          o[4 * pr] = u32x4{wd[2 * pr][0], wd[2 * pr][1], wd[2 * pr][2], wd[2 * pr][3]};
          o[4 * pr + 1] = u32x4{wd[2 * pr + 1][0], wd[2 * pr + 1][1], wd[2 * pr + 1][2], wd[2 * pr + 1][3]};
        }
      }
    }
  }
  // S_next = Diag(Gam) S0 + Kb^T D, rows 32w.. of Kb^T, 64 tokens contracted
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] *= cur.gm[e >> 2][e & 3];
  S = mma32_rr<MT, 32>(cur.kb, dfr, S);
  // operand copy of the new state, transposed: sS[value][key]
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store4(sS + col * SL + 32 * w + 8 * e4 + 4 * g,
           f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  if constexpr (ROLE == 0 && !EARLY) {
    __builtin_amdgcn_sched_barrier(0);
    issue();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // new S0 complete; D may be overwritten
}

// The chunk loop of one wave: operands are loaded ahead into rotating register
// sets (bf16: two chunks ahead, three sets; fp32: one chunk ahead, two sets).
// S (in/out): the wave's 32 state rows 32w.. (key) at value columns vb*32..
// of this sequence, FP32; the LDS operand copy of its start value is in sS.
template <typename MT, typename TO, int ROLE>
__device__ __forceinline__ void scan_chunks(const ScanArgs& p, MT* sS, MT* sD, int h, int cbeg,
                                            int cend, int tseq, int tend, int vb, int w, int l,
                                            f32x16& S) {
  const int g = l >> 5, wp = w & 1;
  const int H = p.H;
  const MT* __restrict__ rec = reinterpret_cast<const MT*>(p.rec);
  auto load = [&](ScanOps<MT, ROLE>& o, int c) {
    scan_load(o, rec + ((size_t)c * H + h) * REC, p.gam + ((size_t)c * H + h) * DH, wp, w, l, g, vb);
  };
  auto step = [&](const ScanOps<MT, ROLE>& o, f32x16& S, int c, auto&& issue) {
    const int ctok = tseq + (c - cbeg) * CHUNK;
    scan_step<MT, TO, ROLE, true>(p, o, S, sS, sD, h, ctok, CHUNK, vb, w, l, issue);
  };
  auto tail = [&](const ScanOps<MT, ROLE>& o, f32x16& S, int c, auto&& issue) {
    const int ctok = tseq + (c - cbeg) * CHUNK;
    scan_step<MT, TO, ROLE, false>(p, o, S, sS, sD, h, ctok, tend - ctok, vb, w, l, issue);
  };
  auto none = [] {};
  // Full chunks run in the main loop; a partial last chunk runs after it.
  // Prefetch loads are unconditional (indices clamped to the last chunk), so
  // every iteration issues the same memory operations and the compiler's
  // memory-counter waits only cover the chunk being consumed.
  const int cfull = cbeg + (tend - tseq) / CHUNK;  // chunks [cbeg, cfull) are full
  const int clast = cend - 1;
  ScanOps<MT, ROLE> o0, o1, o2;
  load(o0, cbeg);
  if constexpr (sizeof(MT) == 2) load(o1, min(cbeg + 1, clast));
  __syncthreads();  // start-state operand visible
  int c = cbeg;
  if constexpr (sizeof(MT) == 2) {
    // o0 holds chunk c, o1 chunk c+1; step c sends the loads of chunk c+2
    for (; c + 3 <= cfull; c += 3) {
      step(o0, S, c, [&] { load(o2, min(c + 2, clast)); });
      step(o1, S, c + 1, [&] { load(o0, min(c + 3, clast)); });
      step(o2, S, c + 2, [&] { load(o1, min(c + 4, clast)); });
    }
    // at most two full chunks and the partial chunk remain
    if (c < cend) {
      auto nx = [&] { load(o2, min(c + 2, clast)); };
      if (c < cfull) step(o0, S, c, nx); else tail(o0, S, c, nx);
      ++c;
    }
    if (c < cend) {
      if (c < cfull) step(o1, S, c, none); else tail(o1, S, c, none);
      ++c;
    }
    if (c < cend) tail(o2, S, c, none);
  } else {
    // FP32 operands are twice as large: two sets; step c sends chunk c+1
    for (; c + 2 <= cfull; c += 2) {
      step(o0, S, c, [&] { load(o1, min(c + 1, clast)); });
      step(o1, S, c + 1, [&] { load(o0, min(c + 2, clast)); });
    }
    if (c < cend) {
      auto nx = [&] { load(o1, min(c + 1, clast)); };
      if (c < cfull) step(o0, S, c, nx); else tail(o0, S, c, nx);
      ++c;
    }
    if (c < cend) tail(o1, S, c, none);
  }
}

template <typename MT, typename TO>
__global__ __launch_bounds__(256) void kda_scan_kernel(ScanArgs p) {
  typedef ScanLds<MT> L;
  constexpr int SL = L::SL;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  MT* sS = reinterpret_cast<MT*>(smem + L::O_S);  // S0^T [32 dv][SL]
  MT* sD = reinterpret_cast<MT*>(smem + L::O_D);  // D^T  [32 dv][DL]

  int pair, vb;
  scan_unit(blockIdx.x, pair, vb);
  if (pair >= p.N * p.H) return;
  const int n = pair / p.H, h = pair - n * p.H;
  const int cbeg = p.cfirst[n], cend = p.cfirst[n + 1];
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 31, g = l >> 5;
  // Lane (col, g) of wave w holds state entries (key 32w + row32(e), value
  // 32vb + col); for each e the 32 lanes of a group touch 128 contiguous bytes.
  const size_t sbase = (size_t)pair * DH * DH + (size_t)(32 * w) * DH + DVB * vb + col;
  f32x16 S;
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] = p.init ? p.init[sbase + (size_t)row32(e, l) * DH] : 0.0f;
  if (cbeg == cend) {  // empty sequence: the end state is the start state
    if (p.fin) {
#pragma unroll
      for (int e = 0; e < 16; ++e) p.fin[sbase + (size_t)row32(e, l) * DH] = S[e];
    }
    return;
  }
  // operand copy of the start state, transposed: sS[value][key]
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store4(sS + col * SL + 32 * w + 8 * e4 + 4 * g,
           f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  if (w < 2) scan_chunks<MT, TO, 0>(p, sS, sD, h, cbeg, cend, tseq, tend, vb, w, l, S);
  else scan_chunks<MT, TO, 1>(p, sS, sD, h, cbeg, cend, tseq, tend, vb, w, l, S);
  if (p.fin) {
#pragma unroll
    for (int e = 0; e < 16; ++e) p.fin[sbase + (size_t)row32(e, l) * DH] = S[e];
  }
}

// ===========================================================================
// State pass with loader waves (bf16 intermediates).
//
// The state pass is bound by how fast one CU can bring in each chunk's
// operands (about 60 KB per workgroup) while the compute waves also have to
// issue those loads in order with their matrix work.  Here four extra waves do
// nothing but copy each chunk's operands straight from global memory into a
// two-slot LDS ring with 16-byte direct-to-LDS loads; the four compute waves
// read their fragments from LDS.  The records are already in fragment order,
// so every copy is 1 KB contiguous on both sides.
//
// Slot layout (bytes): W [0,16K) | Qt [16K,32K) | Kb^T [32K,48K) | U of this
// value block [48K,52K) | P [52K,60K) | Gam [60K, 60K+512).  "Early" operands
// (W, Qt, U) are read before the first barrier of a step, "late" ones (Kb^T,
// P, Gam) after it.  In step c the loaders copy chunk c+1's early operands at
// the start and its late operands after the first barrier, each into the slot
// that chunk c-1 used; a loader waits for its own copies (memory counter)
// right before the barrier that publishes them.  The barriers here are plain
// s_barrier with explicit waits: a workgroup-scope fence would make every
// loader wait for all of its copies in flight.
constexpr int RG_W = 0, RG_QT = 16384, RG_KBT = 32768, RG_U = 49152, RG_P = 53248, RG_GM = 61440;
constexpr int RG_SLOT = 61952;
struct RingLds {
  static constexpr int SL = 136, DL = 72;  // bf16 row lengths of S0^T and D^T
  static constexpr int O_RING = 0;
  static constexpr int O_S = 2 * RG_SLOT;
  static constexpr int O_D = O_S + DVB * SL * 2;
  static constexpr int BYTES = O_D + DVB * DL * 2;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// One wave copies 1 KB: lane l's 16 bytes from src_wave + 16 l to
// lds_wave + 16 l (lds_wave is uniform across the wave).
__device__ __forceinline__ void copy_1k(const char* src_wave, char* lds_wave, int l) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)(src_wave + 16 * l), (lds_void_t*)lds_wave, 16, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations of this wave are outstanding / until LDS operations are done.
template <int n> __device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Workgroup barrier without a workgroup-scope fence.  Callers wait for what
// they must publish (compute waves: their LDS writes; loaders: their copies).
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Loader wave lw (0..3): copies of chunk record rc (bytes) and gamma gc.
constexpr int RG_EARLY_PER_LOADER = 9;  // 32 KB of W, Qt + 4 KB of U over 4 loaders
constexpr int RG_LATE_MIN = 6;          // 24 KB of Kb^T, P over 4 loaders (+ Gam on loader 0)
__device__ __forceinline__ void ring_copy_early(const char* rc, char* slot, int vb, int lw, int l) {
#pragma unroll
  for (int k = 0; k < 8; ++k) copy_1k(rc + (lw + 4 * k) * 1024, slot + RG_W + (lw + 4 * k) * 1024, l);
  copy_1k(rc + 2 * OFF_UT + vb * 4096 + lw * 1024, slot + RG_U + lw * 1024, l);
}
__device__ __forceinline__ void ring_copy_late(const char* rc, const char* gc, char* slot, int lw, int l) {
#pragma unroll
  for (int k = 0; k < 4; ++k) copy_1k(rc + 2 * OFF_KBT + (lw + 4 * k) * 1024, slot + RG_KBT + (lw + 4 * k) * 1024, l);
#pragma unroll
  for (int k = 0; k < 2; ++k) copy_1k(rc + 2 * OFF_P + (lw + 4 * k) * 1024, slot + RG_P + (lw + 4 * k) * 1024, l);
  if (lw == 0 && l < 32) copy_1k(gc, slot + RG_GM, l);  // 512 bytes of Gam
}

// One chunk for one compute wave; operands come from ring slot `slot`.
template <typename TO, int ROLE, bool FULL>
__device__ __forceinline__ void ring_step(const ScanArgs& p, const char* slot, f32x16& S, bf16* sS,
                                          bf16* sD, int h, int ctok, int len, int vb, int w, int l) {
  typedef RingLds L;
  constexpr int SL = L::SL, DL = L::DL;
  const int col = l & 31, g = l >> 5, wp = w & 1;
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
  auto frag = [&](int off) { return *reinterpret_cast<const bf16x8*>(slot + off + 16 * l); };
  bf16x8 a[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) a[s] = frag((ROLE == 0 ? RG_W : RG_QT) + wp * 8192 + s * 1024);
  f32x16 X;
#pragma unroll
  for (int e = 0; e < 16; ++e) X[e] = 0.0f;
  if constexpr (ROLE == 0) {
    bf16x8 u[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) u[s] = frag(RG_U + wp * 2048 + s * 1024);
    X = mma32_frags<bf16, 64>(a, sS + col * SL + 64 * g, X);
    // D = U - W S0 at tokens 32wp + row32(e), value column col
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = val_at(u, 4 * e4 + i) - X[4 * e4 + i];
      store4(sD + col * DL + 32 * wp + 8 * e4 + 4 * g, d);
    }
  } else {
    // transposed product S0^T Qt^T: rows = values, columns = tokens
    X = mma32_lds_frags<bf16, 64>(sS + col * SL + 64 * g, a, X);
  }
  wait_lds();
  ring_barrier();  // D complete; every wave is done reading S0
  bf16x8 kb[4], dfr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kb[s] = frag(RG_KBT + w * 4096 + s * 1024);
  const f32x4* gmp = reinterpret_cast<const f32x4*>(slot + RG_GM);
  f32x4 gm[4];
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) gm[e4] = gmp[(32 * w + 8 * e4 + 4 * g) / 4];
#pragma unroll
  for (int s = 0; s < 4; ++s) dfr[s] = *reinterpret_cast<const bf16x8*>(sD + col * DL + 32 * g + 8 * s);
  if constexpr (ROLE == 1) {
    bf16x8 pr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) pr[s] = frag(RG_P + wp * 4096 + s * 1024);
    X = mma32_rr<bf16, 32>(dfr, pr, X);
    // lane (col, g): token 32wp + col, values 8 e4 + 4g + (0..3); one exchange
    // between the lane halves per pair of e4 gives 8 consecutive values
    typedef unsigned u32;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NW = (int)sizeof(TO);
    u32 wd[4][NW];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      if constexpr (sizeof(TO) == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wd[e4][j] = __builtin_bit_cast(u32, bf16x2{(bf16)(p.scale * X[4 * e4 + 2 * j]),
                                                     (bf16)(p.scale * X[4 * e4 + 2 * j + 1])});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wd[e4][j] = __builtin_bit_cast(u32, p.scale * X[4 * e4 + j]);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(wd[2 * q][j], wd[2 * q + 1][j], false, false);
        wd[2 * q][j] = r[0];
        wd[2 * q + 1][j] = r[1];
      }
    const int tk = 32 * wp + col;
    if (FULL || tk < len) {
      u32x4* o = reinterpret_cast<u32x4*>(out + ((size_t)(ctok + tk) * p.H + h) * DH + DVB * vb + 8 * g);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if constexpr (sizeof(TO) == 2) {
          o[2 * q] = u32x4{wd[2 * q][0], wd[2 * q][1], wd[2 * q + 1][0], wd[2 * q + 1][1]};
        } else {
          o[4 * q] = u32x4{wd[2 * q][0], wd[2 * q][1], wd[2 * q][2], wd[2 * q][3]};
          o[4 * q + 1] = u32x4{wd[2 * q + 1][0], wd[2 * q + 1][1], wd[2 * q + 1][2], wd[2 * q + 1][3]};
        }
      }
    }
  }
  // S_next = Diag(Gam) S0 + Kb^T D
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] *= gm[e >> 2][e & 3];
  S = mma32_rr<bf16, 32>(kb, dfr, S);
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store4(sS + col * SL + 32 * w + 8 * e4 + 4 * g,
           f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  wait_lds();
  ring_barrier();  // new S0 complete; D may be overwritten
}

template <typename TO>
__global__ __launch_bounds__(512) void kda_scan_ring_kernel(ScanArgs p) {
  typedef RingLds L;
  constexpr int SL = L::SL;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* ring = smem + L::O_RING;
  bf16* sS = reinterpret_cast<bf16*>(smem + L::O_S);
  bf16* sD = reinterpret_cast<bf16*>(smem + L::O_D);

  int pair, vb;
  scan_unit(blockIdx.x, pair, vb);
  if (pair >= p.N * p.H) return;
  const int n = pair / p.H, h = pair - n * p.H;
  const int cbeg = p.cfirst[n], cend = p.cfirst[n + 1];
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 31, g = l >> 5;
  const size_t sbase = (size_t)pair * DH * DH + (size_t)(32 * (w & 3)) * DH + DVB * vb + col;
  const int H = p.H;
  const char* recb = reinterpret_cast<const char*>(p.rec);
  const char* gamb = reinterpret_cast<const char*>(p.gam);
  auto rec_of = [&](int c) { return recb + ((size_t)c * H + h) * (size_t)REC * 2; };
  auto gam_of = [&](int c) { return gamb + ((size_t)c * H + h) * DH * 4; };

  if (w >= 4) {
    // ------------------------------------------------------------ loaders
    if (cbeg == cend) return;
    const int lw = w - 4, clast = cend - 1;
    ring_copy_early(rec_of(cbeg), ring, vb, lw, l);
    ring_copy_late(rec_of(cbeg), gam_of(cbeg), ring, lw, l);
    wait_vm<0>();
    ring_barrier();  // chunk cbeg in slot 0; start state in sS
    for (int c = cbeg; c < cend; ++c) {
      const int nx = min(c + 1, clast);
      char* nslot = ring + ((c - cbeg + 1) & 1) * RG_SLOT;
      ring_copy_early(rec_of(nx), nslot, vb, lw, l);
      wait_vm<RG_EARLY_PER_LOADER>();  // late operands of chunk c are in
      ring_barrier();
      ring_copy_late(rec_of(nx), gam_of(nx), nslot, lw, l);
      wait_vm<RG_LATE_MIN>();  // early operands of chunk c+1 are in
      ring_barrier();
    }
    wait_vm<0>();  // nothing left in flight when the wave ends
    return;
  }
  // -------------------------------------------------------------- compute
  f32x16 S;
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] = p.init ? p.init[sbase + (size_t)row32(e, l) * DH] : 0.0f;
  if (cbeg == cend) {
    if (p.fin) {
#pragma unroll
      for (int e = 0; e < 16; ++e) p.fin[sbase + (size_t)row32(e, l) * DH] = S[e];
    }
    return;
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store4(sS + col * SL + 32 * w + 8 * e4 + 4 * g,
           f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  wait_lds();
  ring_barrier();
  const int cfull = cbeg + (tend - tseq) / CHUNK;
  for (int c = cbeg; c < cend; ++c) {
    const char* slot = ring + ((c - cbeg) & 1) * RG_SLOT;
    const int ctok = tseq + (c - cbeg) * CHUNK;
    if (c < cfull) {
      if (w < 2) ring_step<TO, 0, true>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l);
      else ring_step<TO, 1, true>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l);
    } else {
      if (w < 2) ring_step<TO, 0, false>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l);
      else ring_step<TO, 1, false>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l);
    }
  }
  if (p.fin) {
#pragma unroll
    for (int e = 0; e < 16; ++e) p.fin[sbase + (size_t)row32(e, l) * DH] = S[e];
  }
}

}  // namespace kda
