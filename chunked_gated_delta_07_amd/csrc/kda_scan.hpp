// kda_scan.hpp -- chunk-to-chunk state pass fused with the output combine.
//
// For each chunk of a sequence, with S0 the state entering it (d_k x d_v,
// zero at the sequence start unless a start state is given):
//   D      = U - W S0                       (corrected values)
//   out    = scale (Qt S0 + P D)            (inter- plus intra-chunk terms)
//   S_next = Diag(Gam) S0 + Kb^T D
// (the inter-chunk part of the chunked operator of xtuner PR #2301, sections
// Problem and Change; the algebra is written out in kda_intra.hpp).  Columns
// of S are independent, so one workgroup owns a 32-wide block of value
// channels of one (sequence, head) and walks its chunks in order.  The running state stays FP32 in MFMA
// accumulators for the whole sequence.
//
// Work split inside a workgroup (4 compute waves, 32x32 MFMA tiles): wave w
// owns state rows 32w..32w+31 (key channels).  X = [W; Qt] S0 is 128 x 32:
// waves 0,1 form W S0 (-> D), waves 2,3 form Qt S0 (-> output).  Four more
// waves copy each chunk's operands into LDS.  Two kernels:
//   kda_scan_ring_kernel    bf16 intermediates, two LDS slots;
//   kda_scan_ring32_kernel  FP32 intermediates, one LDS slot refilled in
//                           halves, products on bf16 matrix cores from
//                           three-piece splits of the FP32 operands.
#pragma once

#include "kda_common.hpp"
#include "kda_intra.hpp"

namespace kda {

struct ScanArgs {
  const int32_t* cu;
  const int32_t* cfirst;  // [N+1] first chunk of each sequence, or null for N = 1
  int N;
  int H;
  float scale;
  const float* gam;  // [chunks][H][128]
  const void* rec;   // [chunks][H][record elements] (Frag layout)
  void* out;         // [T][H][128]
  const float* init; // [N][H][128 key][128 value] start states, or null (zero)
  float* fin;        // [N][H][128][128] end states, or null (not written)
  // with the kernels' RECT parameter: key / value widths (<= 128) of out
  // [T][H][dv] and of the states [N][H][dk][dv]
  int dk, dv;
  // Segmented schedule (BF16 intermediates): this launch walks the chunks in
  // [c0, c1) only; records and Gam of chunk c sit in slot c % ring (ring = 0:
  // slot c).  A sequence that starts before c0 takes its state from carry_in,
  // one that continues past c1 leaves it in carry_out ([H][128][128] each; at
  // most one sequence crosses a segment boundary).  Whole-sequence launches
  // use c0 = 0, c1 = INT_MAX.  Only kda_scan_ring_kernel reads these.
  int c0, c1, ring;
  const float* carry_in;
  float* carry_out;
};

constexpr int SEG_CHUNKS = 32;  // chunks per segment of the segmented schedule

// State entry (key, value) of (sequence, head) pair `pair` in a [..][dk][dv]
// array, or -1 when the pair of widths leaves it out.
template <bool RECT>
__device__ __forceinline__ int64_t state_index(const ScanArgs& p, int pair, int key, int value) {
  if constexpr (RECT) {
    if (key >= p.dk || value >= p.dv) return -1;
    return ((int64_t)pair * p.dk + key) * p.dv + value;
  } else {
    return ((int64_t)pair * DH + key) * DH + value;
  }
}

constexpr int DVB = 32;  // value channels per workgroup


// Output of one lane after the lane-half exchange: for q = 0, 1 the words
// wd[2q][..] hold values rowp[16q .. 16q+3] and wd[2q+1][..] values
// rowp[16q+4 .. 16q+7] (packed pairs for bf16); rowp is value column v0 of
// the token's output row.  RECT: values at or past column dv are not written
// (element stores).
template <typename TO, bool RECT>
__device__ __forceinline__ void store_out8(TO* rowp, int v0, int dv, const u32 (&wd)[4][sizeof(TO)]) {
  constexpr int NW = (int)sizeof(TO);
  if constexpr (!RECT) {
    u32x4* o = reinterpret_cast<u32x4*>(rowp);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (NW == 2) {
        o[2 * q] = u32x4{wd[2 * q][0], wd[2 * q][1], wd[2 * q + 1][0], wd[2 * q + 1][1]};
      } else {
        o[4 * q] = u32x4{wd[2 * q][0], wd[2 * q][1], wd[2 * q][2], wd[2 * q][3]};
        o[4 * q + 1] = u32x4{wd[2 * q + 1][0], wd[2 * q + 1][1], wd[2 * q + 1][2], wd[2 * q + 1][3]};
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 16 * q + 4 * half + i;  // offset from v0
          if (v0 + v < dv) {
            const u32 word = wd[2 * q + half][NW == 2 ? i / 2 : i];
            if constexpr (NW == 2)
              reinterpret_cast<uint16_t*>(rowp)[v] = (uint16_t)(i & 1 ? word >> 16 : word & 0xffff);
            else
              reinterpret_cast<u32*>(rowp)[v] = word;
          }
        }
  }
}

// C += A B over 16 contracted values from their pieces (smallest terms first)
__device__ __forceinline__ f32x16 mma_x6(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c, 0, 0, 0);
  return c;
}

// Operand copies of S0 (S0^T, [value][key]) and of D (D^T, [value][token])
// in the FP32-intermediate state pass, each as three bf16 planes (pieces h,
// m, l) of row lengths SL and DL.
struct ScanLds {
  static constexpr int SL = 136;      // S0^T row: 128 key channels (+8 pad)
  static constexpr int DL = 72;       // D^T row: 64 tokens (+8 pad)
  static constexpr int PS = DVB * SL; // plane strides, elements
  static constexpr int PD = DVB * DL;
  static constexpr int O_S = 0;
  static constexpr int O_D = O_S + 3 * PS * 2;
  static constexpr int BYTES = O_D + 3 * PD * 2;
};
__device__ __forceinline__ void load_pieces8(const bf16* p, int stride, bf16x8 (&o)[3]) {
#pragma unroll
  for (int q = 0; q < 3; ++q) o[q] = *reinterpret_cast<const bf16x8*>(p + q * stride);
}

// Workgroup id -> (sequence*H + head, value block).  The four value blocks of
// one (sequence, head) get ids that are equal mod 8, i.e. land on one XCD and
// share its L2 for the per-chunk matrices they all read.
__device__ __forceinline__ void scan_unit(int bid, int& pair, int& vb) {
  const int xcd = bid & 7, slot = bid >> 3;
  vb = slot & 3;
  pair = (slot >> 2) * 8 + xcd;
}

// bf16 32x32 tiles over NK contracted values per lane (NK/8 instructions).
// C += A B: A from register fragments, B from LDS (NK contiguous values at pb).
template <int NK>
__device__ __forceinline__ f32x16 mma32_frags(const bf16x8* afr, const bf16* pb, f32x16 c) {
#pragma unroll
  for (int s = 0; s < NK / 8; ++s)
    c = Mma32<bf16>::mma(afr[s], *reinterpret_cast<const bf16x8*>(pb + 8 * s), c);
  return c;
}
// C += A B with A read from LDS (NK contiguous values at pa) and B from
// register fragments: the same instructions as mma32_frags with the operands
// exchanged, so C comes out transposed.
template <int NK>
__device__ __forceinline__ f32x16 mma32_lds_frags(const bf16* pa, const bf16x8* bfr, f32x16 c) {
#pragma unroll
  for (int s = 0; s < NK / 8; ++s)
    c = Mma32<bf16>::mma(*reinterpret_cast<const bf16x8*>(pa + 8 * s), bfr[s], c);
  return c;
}
// C += A B, both operands from register fragments.
template <int NK>
__device__ __forceinline__ f32x16 mma32_rr(const bf16x8* afr, const bf16x8* bfr, f32x16 c) {
#pragma unroll
  for (int s = 0; s < NK / 8; ++s) c = Mma32<bf16>::mma(afr[s], bfr[s], c);
  return c;
}
template <typename V> __device__ __forceinline__ float val_at(const V* f, int q) {
  constexpr int FE = sizeof(f[0][0]) == 2 ? 8 : 4;
  return (float)f[q / FE][q % FE];
}

// ===========================================================================
// State pass with loader waves (bf16 intermediates).
//
// The state pass is bound by how fast one CU can bring in each chunk's
// operands (about 58 KB per workgroup) while the compute waves also have to
// issue those loads in order with their matrix work.  Here four extra waves do
// nothing but copy each chunk's operands straight from global memory into a
// two-slot LDS ring with 16-byte direct-to-LDS loads; the four compute waves
// read their fragments from LDS.  The records are already in fragment order,
// so every copy is 1 KB contiguous on both sides.
//
// Slot layout (bytes): W [0,16K) | Qt [16K,32K) | Kb^T [32K,48K) | U of this
// value block [48K,52K) | P's lower tiles [52K,58K) | Gam [58K, 58K+512).
// "Early" operands
// (W, Qt, U) are read before the first barrier of a step, "late" ones (Kb^T,
// P, Gam) after it.  In step c the loaders copy chunk c+1's early operands at
// the start and its late operands after the first barrier, each into the slot
// that chunk c-1 used; a loader waits for its own copies (memory counter)
// right before the barrier that publishes them.  The barriers here are plain
// s_barrier with explicit waits: a workgroup-scope fence would make every
// loader wait for all of its copies in flight.
constexpr int RG_W = 0, RG_QT = 16384, RG_KBT = 32768, RG_U = 49152, RG_P = 53248, RG_GM = 59392;
constexpr int RG_SLOT = 59904;
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
// 22 KB of Kb^T, P and Gam over 4 loaders: 5 copies on loader 0, 6 on the others
template <int LW> constexpr int rg_late_copies() { return LW == 0 ? 5 : 6; }
__device__ __forceinline__ void ring_copy_early(const char* rc, char* slot, int vb, int lw, int l) {
#pragma unroll
  for (int k = 0; k < 8; ++k) copy_1k(rc + (lw + 4 * k) * 1024, slot + RG_W + (lw + 4 * k) * 1024, l);
  copy_1k(rc + 2 * OFF_UT + vb * 4096 + lw * 1024, slot + RG_U + lw * 1024, l);
}
__device__ __forceinline__ void ring_copy_late(const char* rc, const char* gc, char* slot, int lw, int l) {
#pragma unroll
  for (int k = 0; k < 4; ++k) copy_1k(rc + 2 * OFF_KBT + (lw + 4 * k) * 1024, slot + RG_KBT + (lw + 4 * k) * 1024, l);
  copy_1k(rc + 2 * OFF_P + lw * 1024, slot + RG_P + lw * 1024, l);  // P: six fragments
  if (lw >= 2) copy_1k(rc + 2 * OFF_P + (lw + 2) * 1024, slot + RG_P + (lw + 2) * 1024, l);
  if (lw == 1 && l < 32) copy_1k(gc, slot + RG_GM, l);  // 512 bytes of Gam
}
// Wait until only this loader's late copies are in flight.
__device__ __forceinline__ void ring_wait_early(int lw) {
  if (lw == 0) wait_vm<rg_late_copies<0>()>();
  else wait_vm<rg_late_copies<1>()>();
}

// Output of one chunk from an output wave's accumulator X (lane (col, g):
// token 32 wp + col, values 8 e4 + 4 g + (0..3)): scaled, converted, one
// exchange between the lane halves per pair of e4 (8 consecutive values per
// lane), 16-byte stores of the tokens below len.
template <typename TO, bool RECT>
__device__ __forceinline__ void ring_out_store(const ScanArgs& p, const f32x16& X, int ctok, int len,
                                               int h, int vb, int w, int l) {
  const int col = l & 31, g = l >> 5, wp = w & 1;
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
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
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const auto r = __builtin_amdgcn_permlane32_swap(wd[2 * q][j], wd[2 * q + 1][j], false, false);
      wd[2 * q][j] = r[0];
      wd[2 * q + 1][j] = r[1];
    }
  const int tk = 32 * wp + col;
  if (tk < len) {
    const int dvo = RECT ? p.dv : DH;  // output row width
    store_out8<TO, RECT>(out + ((size_t)(ctok + tk) * p.H + h) * dvo + DVB * vb + 8 * g,
                         DVB * vb + 8 * g, dvo, wd);
  }
}

// One chunk for one compute wave; operands come from ring slot `slot`.
template <typename TO, int ROLE, bool FULL, bool RECT>
__device__ __forceinline__ void ring_step(const ScanArgs& p, const char* slot, f32x16& S, bf16* sS,
                                          bf16* sD, int h, int ctok, int len, int vb, int w, int l) {
  typedef RingLds L;
  constexpr int SL = L::SL, DL = L::DL;
  const int col = l & 31, g = l >> 5, wp = w & 1;
  auto frag = [&](int off) { return *reinterpret_cast<const bf16x8*>(slot + off + 16 * l); };
  bf16x8 a[8];
  if constexpr (ROLE == 0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = frag(RG_W + wp * 8192 + s * 1024);
  } else {
    // Qt in its own order (Frag::qt): token 32 wp + col, channels 64 g + 8 s
    // .. + 7, the same values as a W fragment
#pragma unroll
    for (int s = 0; s < 8; ++s)
      a[s] = *reinterpret_cast<const bf16x8*>(slot + RG_QT + 2 * Frag<bf16>::qt(32 * wp + col, 64 * g + 8 * s));
  }
  f32x16 X;
#pragma unroll
  for (int e = 0; e < 16; ++e) X[e] = 0.0f;
  if constexpr (ROLE == 0) {
    bf16x8 u[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) u[s] = frag(RG_U + wp * 2048 + s * 1024);
    X = mma32_frags<64>(a, sS + col * SL + 64 * g, X);
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
    X = mma32_lds_frags<64>(sS + col * SL + 64 * g, a, X);
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
  // D^T fragments, tokens 16 s + 8 g .. + 7 (the records' token order)
#pragma unroll
  for (int s = 0; s < 4; ++s) dfr[s] = *reinterpret_cast<const bf16x8*>(sD + col * DL + 16 * s + 8 * g);
  if constexpr (ROLE == 1) {
    bf16x8 pr[4];
    if (wp == 0) {  // tokens 0..31: P's columns below 32 only
#pragma unroll
      for (int s = 0; s < 2; ++s) pr[s] = frag(RG_P + s * 1024);
      X = mma32_rr<16>(dfr, pr, X);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) pr[s] = frag(RG_P + 2048 + s * 1024);
      X = mma32_rr<32>(dfr, pr, X);
    }
    ring_out_store<TO, RECT>(p, X, ctok, FULL ? CHUNK : len, h, vb, w, l);
  }
  // S_next = Diag(Gam) S0 + Kb^T D
#pragma unroll
  for (int e = 0; e < 16; ++e) S[e] *= gm[e >> 2][e & 3];
  S = mma32_rr<32>(kb, dfr, S);
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store4(sS + col * SL + 32 * w + 8 * e4 + 4 * g,
           f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  wait_lds();
  ring_barrier();  // new S0 complete; D may be overwritten
}

template <typename TO, bool RECT = false>
__global__ __launch_bounds__(512) void kda_scan_ring_kernel(ScanArgs p) {
  typedef RingLds L;
  constexpr int SL = L::SL;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* ring = smem + L::O_RING;
  bf16* sS = reinterpret_cast<bf16*>(smem + L::O_S);
  bf16* sD = reinterpret_cast<bf16*>(smem + L::O_D);

  int pair, vb;
  scan_unit(blockIdx.x + 32 * blockIdx.y, pair, vb);  // grid (32, pairs / 8)
  if (pair >= p.N * p.H) return;
  if (RECT && DVB * vb >= p.dv) return;  // a value block past the value width
  const int n = pair / p.H, h = pair - n * p.H;
  int cbeg, cend;
  chunk_range(p.cu, p.cfirst, n, cbeg, cend);
  // this launch's chunks of the sequence; an empty sequence is handled by the
  // launch whose range holds its position
  const int lo = max(cbeg, p.c0), hi = min(cend, p.c1);
  if (cbeg < cend ? lo >= hi : (cbeg < p.c0 || cbeg >= p.c1)) return;  // uniform over the block
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 31, g = l >> 5;
  // state entry e of this lane: key 32 (w & 3) + row32(e, l), value 32 vb + col
  auto sidx = [&](int e) { return state_index<RECT>(p, pair, 32 * (w & 3) + row32(e, l), DVB * vb + col); };
  // the same entry in a per-head carry buffer [H][128][128]
  auto cidx = [&](int e) { return ((size_t)h * DH + 32 * (w & 3) + row32(e, l)) * DH + DVB * vb + col; };
  const int H = p.H;
  const char* recb = reinterpret_cast<const char*>(p.rec);
  const char* gamb = reinterpret_cast<const char*>(p.gam);
  auto slot_of = [&](int c) { return (size_t)(p.ring ? c % p.ring : c); };
  auto rec_of = [&](int c) { return recb + (slot_of(c) * H + h) * (size_t)Frag<bf16>::REC_ELEMS * 2; };
  auto gam_of = [&](int c) { return gamb + (slot_of(c) * H + h) * DH * 4; };

  if (w >= 4) {
    // ------------------------------------------------------------ loaders
    if (cbeg == cend) return;
    const int lw = w - 4, clast = hi - 1;
    ring_copy_early(rec_of(lo), ring, vb, lw, l);
    ring_copy_late(rec_of(lo), gam_of(lo), ring, lw, l);
    wait_vm<0>();
    ring_barrier();  // chunk lo in slot 0; start state in sS
    for (int c = lo; c < hi; ++c) {
      const int nx = min(c + 1, clast);
      char* nslot = ring + ((c - lo + 1) & 1) * RG_SLOT;
      ring_copy_early(rec_of(nx), nslot, vb, lw, l);
      wait_vm<RG_EARLY_PER_LOADER>();  // late operands of chunk c are in
      ring_barrier();
      ring_copy_late(rec_of(nx), gam_of(nx), nslot, lw, l);
      ring_wait_early(lw);  // early operands of chunk c+1 are in
      ring_barrier();
    }
    wait_vm<0>();  // nothing left in flight when the wave ends
    return;
  }
  // -------------------------------------------------------------- compute
  f32x16 S;
  if (lo > cbeg) {  // continued from the previous segment
#pragma unroll
    for (int e = 0; e < 16; ++e) S[e] = p.carry_in[cidx(e)];
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t i = sidx(e);
      S[e] = (p.init && i >= 0) ? p.init[i] : 0.0f;
    }
  }
  if (cbeg == cend) {
    if (p.fin) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (sidx(e) >= 0) p.fin[sidx(e)] = S[e];
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
  for (int c = lo; c < hi; ++c) {
    const char* slot = ring + ((c - lo) & 1) * RG_SLOT;
    const int ctok = tseq + (c - cbeg) * CHUNK;
    if (c < cfull) {
      if (w < 2) ring_step<TO, 0, true, RECT>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l);
      else ring_step<TO, 1, true, RECT>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l);
    } else {
      if (w < 2) ring_step<TO, 0, false, RECT>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l);
      else ring_step<TO, 1, false, RECT>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l);
    }
  }
  if (hi < cend) {  // the sequence continues in the next segment
#pragma unroll
    for (int e = 0; e < 16; ++e) p.carry_out[cidx(e)] = S[e];
  } else if (p.fin) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (sidx(e) >= 0) p.fin[sidx(e)] = S[e];
  }
}

// ===========================================================================
// State pass with loader waves, FP32 intermediates.
//
// The same division of labour as above, with one LDS slot: a chunk's FP32
// operands (116.5 KB) and the pieces of S0 and D (39 KB) fill the 160 KB of a
// CU, so there is no second slot.  The slot is refilled in halves instead:
// the early operands (W, Qt, U; read before the first barrier of a step) of
// chunk c+1 are copied while the compute waves work on chunk c's late
// operands (Kb^T, P, Gam), and those of chunk c+1 while the compute waves
// work on chunk c+1's early ones.  Each copy has half a step to land and each
// loader waits for all of its copies before the barrier that publishes them.
// The compute waves hold no prefetched operands in registers, which leaves
// the register file to the splitting of the operands into bf16 pieces.
//
// Slot layout (bytes): W [0,32K) | Qt [32K,64K) | Kb^T [64K,96K) | U of this
// value block [96K,104K) | P's lower tiles [104K,116K) | Gam [116K, 116K+512).
constexpr int RF_W = 0, RF_QT = 32768, RF_KBT = 65536, RF_U = 98304, RF_P = 106496, RF_GM = 118784;
constexpr int RF_SLOT = 119296;
struct Ring32Lds {
  static constexpr int SL = ScanLds::SL, DL = ScanLds::DL, PS = ScanLds::PS, PD = ScanLds::PD;
  static constexpr int O_SLOT = 0;
  static constexpr int O_S = RF_SLOT;               // S0^T pieces [3][32][SL]
  static constexpr int O_D = O_S + 3 * PS * 2;      // D^T pieces  [3][32][DL]
  static constexpr int O_Z = O_D + 3 * PD * 2;      // 1 KB of zeros: P of rows 0..31, columns 32..63
  static constexpr int BYTES = O_Z + 1024;
};
static_assert(Ring32Lds::BYTES <= 160 * 1024, "one slot plus the pieces fit in a CU's LDS");

// Loader wave lw (0..3).  rc: chunk record (bytes, FP32 elements), gc: Gam.
__device__ __forceinline__ void ring32_copy_early(const char* rc, char* slot, int vb, int lw, int l) {
#pragma unroll
  for (int k = 0; k < 16; ++k)  // W and Qt: 64 KB, adjacent in the record and in the slot
    copy_1k(rc + (lw + 4 * k) * 1024, slot + RF_W + (lw + 4 * k) * 1024, l);
#pragma unroll
  for (int k = 0; k < 2; ++k)  // U columns of value block vb: 8 KB
    copy_1k(rc + 4 * OFF_UT + vb * 8192 + (lw + 4 * k) * 1024, slot + RF_U + (lw + 4 * k) * 1024, l);
}
__device__ __forceinline__ void ring32_copy_late(const char* rc, const char* gc, char* slot, int lw,
                                                 int l) {
#pragma unroll
  for (int k = 0; k < 8; ++k)  // Kb^T: 32 KB
    copy_1k(rc + 4 * OFF_KBT + (lw + 4 * k) * 1024, slot + RF_KBT + (lw + 4 * k) * 1024, l);
#pragma unroll
  for (int k = 0; k < 3; ++k)  // P: 12 KB
    copy_1k(rc + 4 * OFF_P + (lw + 4 * k) * 1024, slot + RF_P + (lw + 4 * k) * 1024, l);
  if (lw == 0 && l < 32) copy_1k(gc, slot + RF_GM, l);  // 512 bytes of Gam
}

// Software-pipelined six-product step: C += (record operand) x (other operand)
// over 16 contracted values from their pieces r and o, while the split of the
// next step's record fragments (na, nb -> nr) runs on the VALU between the six
// matrix-core products.  The products of one step accumulate into one tile, so
// each waits for the previous; the wave issues the independent split
// instructions in those gaps instead of after the sixth product.  The
// scheduling barriers pin that order.  REC_A: the record operand is A (rows of
// the product), else B.  Terms are summed smallest first, as in mma_x6.
template <bool REC_A>
__device__ __forceinline__ f32x16 mma_x6_pipe(const bf16x8 (&r)[3], const bf16x8 (&o)[3], f32x16 c,
                                              bool next, const f32x4& na, const f32x4& nb,
                                              bf16x8 (&nr)[3]) {
  auto mm = [&](const bf16x8& x, const bf16x8& y) {
    c = REC_A ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0)
              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c, 0, 0, 0);
  };
  Pieces2 p0{}, p1{}, p2{}, p3{};
  mm(r[2], o[0]);
  if (next) p0 = split2(f32x2{na[0], na[1]});
  __builtin_amdgcn_sched_barrier(0);
  mm(r[1], o[1]);
  if (next) p1 = split2(f32x2{na[2], na[3]});
  __builtin_amdgcn_sched_barrier(0);
  mm(r[0], o[2]);
  if (next) p2 = split2(f32x2{nb[0], nb[1]});
  __builtin_amdgcn_sched_barrier(0);
  mm(r[1], o[0]);
  if (next) p3 = split2(f32x2{nb[2], nb[3]});
  __builtin_amdgcn_sched_barrier(0);
  mm(r[0], o[1]);
  if (next) {
    nr[0] = __builtin_bit_cast(bf16x8, u32x4{p0.h, p1.h, p2.h, p3.h});
    nr[1] = __builtin_bit_cast(bf16x8, u32x4{p0.m, p1.m, p2.m, p3.m});
    nr[2] = __builtin_bit_cast(bf16x8, u32x4{p0.l, p1.l, p2.l, p3.l});
  }
  __builtin_amdgcn_sched_barrier(0);
  mm(r[0], o[0]);
  return c;
}

// One chunk for one compute wave of the FP32 ring.  Every FP32 record fragment
// is one 16-byte LDS read per lane from the slot, issued two steps before its
// products, and split into pieces during the previous step's products.
// A finished output tile waiting for its store (FP32 state pass): the output
// waves store it at the start of the next step, in the first phase, where
// they wait for the other waves' D anyway, instead of at the end of the
// second phase, which ends the step.
struct Ring32Out {
  f32x16 X;
  int ctok, len;
  bool valid;
};

template <typename TO, int ROLE, bool FULL, bool RECT>
__device__ __forceinline__ void ring32_step(const ScanArgs& p, const char* slot, f32x16& S,
                                            bf16* sS, bf16* sD, int h, int ctok, int len, int vb,
                                            int w, int l, Ring32Out& ro) {
  if constexpr (ROLE == 1) {
    if (ro.valid) ring_out_store<TO, RECT>(p, ro.X, ro.ctok, ro.len, h, vb, w, l);
  }
  typedef Ring32Lds L;
  constexpr int SL = L::SL, DL = L::DL, PS = L::PS, PD = L::PD;
  const int col = l & 31, g = l >> 5, wp = w & 1;
  auto frag = [&](int off) { return *reinterpret_cast<const f32x4*>(slot + off + 16 * l); };
  f32x16 X;
#pragma unroll
  for (int e = 0; e < 16; ++e) X[e] = 0.0f;
  // X = W S0 (role 0) or S0^T Qt^T (role 1); fragments 2s, 2s+1 of the row
  // pair with S0^T entries 64g + 8s .. 64g + 8s + 7 (Qt in its own row-major
  // order, Frag::qt: the same values, token 32 wp + col)
  {
    const int abase = RF_W + wp * 16384;
    auto afrag = [&](int s, int d) {
      if constexpr (ROLE == 0) return frag(abase + (2 * s + d) * 1024);
      else
        return *reinterpret_cast<const f32x4*>(
            slot + RF_QT + 4 * Frag<float>::qt(32 * wp + col, 64 * g + 8 * s + 4 * d));
    };
    const bf16* ps = sS + col * SL + 64 * g;
    f32x4 raw[8][2];
    bf16x8 rr[8][3], oo[8][3];
    raw[0][0] = afrag(0, 0);
    raw[0][1] = afrag(0, 1);
    raw[1][0] = afrag(1, 0);
    raw[1][1] = afrag(1, 1);
    load_pieces8(ps, PS, oo[0]);
    f32x4 u[4];
    if constexpr (ROLE == 0) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) u[e4] = frag(RF_U + wp * 4096 + e4 * 1024);
    }
    split8(raw[0][0], raw[0][1], rr[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 2 < 8) {
        raw[s + 2][0] = afrag(s + 2, 0);
        raw[s + 2][1] = afrag(s + 2, 1);
      }
      if (s + 1 < 8) load_pieces8(ps + 8 * (s + 1), PS, oo[s + 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int sn = s + 1 < 8 ? s + 1 : s;
      X = mma_x6_pipe<ROLE == 0>(rr[s], oo[s], X, s + 1 < 8, raw[sn][0], raw[sn][1], rr[sn]);
    }
    if constexpr (ROLE == 0) {
      // D = U - W S0 at tokens 32wp + row32(e), value column col
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        store_pieces4(sD + col * DL + 32 * wp + 8 * e4 + 4 * g, PD,
                      f32x4{u[e4][0] - X[4 * e4], u[e4][1] - X[4 * e4 + 1],
                            u[e4][2] - X[4 * e4 + 2], u[e4][3] - X[4 * e4 + 3]});
    }
  }
  wait_lds();
  ring_barrier();  // D complete; every wave is done reading S0 and the early operands
  // Phase 2, one pipelined sequence of steps: role 1 runs D^T P^T into X
  // (4 steps of 16 tokens; for tokens 0..31, whose P columns stop at 31, the
  // last two read a zero fragment) and then Kb^T D into S (4 steps); role 0
  // only the latter.
  constexpr int NPS = ROLE == 1 ? 4 : 0, NST = NPS + 4;
  bf16x8 dp[4][3];
  f32x4 raw[NST][2];
  bf16x8 rr[NST][3];
  auto rec_off = [&](int j, int half) {
    if (j < NPS)
      return wp ? RF_P + 4096 + (2 * j + half) * 1024 : j < 2 ? RF_P + (2 * j + half) * 1024 : L::O_Z;
    return RF_KBT + w * 8192 + (2 * (j - NPS) + half) * 1024;
  };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    raw[j][0] = frag(rec_off(j, 0));
    raw[j][1] = frag(rec_off(j, 1));
  }
  // D^T pieces, tokens 16 s + 8 g .. + 7 (the records' token order)
#pragma unroll
  for (int s = 0; s < 4; ++s) load_pieces8(sD + col * DL + 16 * s + 8 * g, PD, dp[s]);
  // Diag(Gam) S0 first: the state tile is free until the Kb^T products
  const f32x4* gmp = reinterpret_cast<const f32x4*>(slot + RF_GM);
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const f32x4 gm = gmp[(32 * w + 8 * e4 + 4 * g) / 4];
#pragma unroll
    for (int i = 0; i < 4; ++i) S[4 * e4 + i] *= gm[i];
  }
  split8(raw[0][0], raw[0][1], rr[0]);
#pragma unroll
  for (int j = 0; j < NST; ++j) {
    if (j + 2 < NST) {
      raw[j + 2][0] = frag(rec_off(j + 2, 0));
      raw[j + 2][1] = frag(rec_off(j + 2, 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    const int jn = j + 1 < NST ? j + 1 : j;
    if (j < NPS)  // out^T += D^T P^T: P rows 32wp.. are the columns
      X = mma_x6_pipe<false>(rr[j], dp[j], X, true, raw[jn][0], raw[jn][1], rr[jn]);
    else  // S_next = Diag(Gam) S0 + Kb^T D, rows 32w.. of Kb^T, 64 tokens contracted
      S = mma_x6_pipe<true>(rr[j], dp[j - NPS], S, j + 1 < NST, raw[jn][0], raw[jn][1], rr[jn]);
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store_pieces4(sS + col * SL + 32 * w + 8 * e4 + 4 * g, PS,
                  f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  if constexpr (ROLE == 1) {
    ro.X = X;
    ro.ctok = ctok;
    ro.len = FULL ? CHUNK : len;
    ro.valid = true;
  }
  wait_lds();
  ring_barrier();  // new S0 complete; D and the late operands may be overwritten
}

template <typename TO, bool RECT = false>
__global__ __launch_bounds__(512) void kda_scan_ring32_kernel(ScanArgs p) {
  typedef Ring32Lds L;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* slot = smem + L::O_SLOT;
  bf16* sS = reinterpret_cast<bf16*>(smem + L::O_S);
  bf16* sD = reinterpret_cast<bf16*>(smem + L::O_D);

  int pair, vb;
  scan_unit(blockIdx.x + 32 * blockIdx.y, pair, vb);  // grid (32, pairs / 8)
  if (pair >= p.N * p.H) return;
  if (RECT && DVB * vb >= p.dv) return;  // a value block past the value width
  const int n = pair / p.H, h = pair - n * p.H;
  int cbeg, cend;
  chunk_range(p.cu, p.cfirst, n, cbeg, cend);
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 31, g = l >> 5;
  const int H = p.H;
  const char* recb = reinterpret_cast<const char*>(p.rec);
  const char* gamb = reinterpret_cast<const char*>(p.gam);
  auto rec_of = [&](int c) { return recb + ((size_t)c * H + h) * (size_t)Frag<float>::REC_ELEMS * 4; };
  auto gam_of = [&](int c) { return gamb + ((size_t)c * H + h) * DH * 4; };

  if (w >= 4) {
    // ------------------------------------------------------------ loaders
    // Barriers: one after the prologue, two per chunk -- the same sequence as
    // the compute waves.
    if (cbeg == cend) return;
    const int lw = w - 4, clast = cend - 1;
    ring32_copy_early(rec_of(cbeg), slot, vb, lw, l);
    wait_vm<0>();
    ring_barrier();  // early operands of chunk cbeg in; start state in sS
    for (int c = cbeg; c < cend; ++c) {
      ring32_copy_late(rec_of(c), gam_of(c), slot, lw, l);
      wait_vm<0>();
      ring_barrier();  // late operands of chunk c in; early ones consumed
      ring32_copy_early(rec_of(min(c + 1, clast)), slot, vb, lw, l);
      wait_vm<0>();
      ring_barrier();  // early operands of chunk c+1 in; late ones of c consumed
    }
    return;
  }
  // -------------------------------------------------------------- compute
  auto sidx = [&](int e) { return state_index<RECT>(p, pair, 32 * w + row32(e, l), DVB * vb + col); };
  f32x16 S;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t i = sidx(e);
    S[e] = (p.init && i >= 0) ? p.init[i] : 0.0f;
  }
  if (cbeg == cend) {
    if (p.fin) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (sidx(e) >= 0) p.fin[sidx(e)] = S[e];
    }
    return;
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    store_pieces4(sS + col * L::SL + 32 * w + 8 * e4 + 4 * g, L::PS,
                  f32x4{S[4 * e4], S[4 * e4 + 1], S[4 * e4 + 2], S[4 * e4 + 3]});
  if (w == 2) *reinterpret_cast<f32x4*>(smem + L::O_Z + 16 * l) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  wait_lds();
  ring_barrier();
  const int cfull = cbeg + (tend - tseq) / CHUNK;
  Ring32Out ro;
  ro.valid = false;
  for (int c = cbeg; c < cend; ++c) {
    const int ctok = tseq + (c - cbeg) * CHUNK;
    if (c < cfull) {
      if (w < 2) ring32_step<TO, 0, true, RECT>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l, ro);
      else ring32_step<TO, 1, true, RECT>(p, slot, S, sS, sD, h, ctok, CHUNK, vb, w, l, ro);
    } else {
      if (w < 2) ring32_step<TO, 0, false, RECT>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l, ro);
      else ring32_step<TO, 1, false, RECT>(p, slot, S, sS, sD, h, ctok, tend - ctok, vb, w, l, ro);
    }
  }
  if (w >= 2 && ro.valid) ring_out_store<TO, RECT>(p, ro.X, ro.ctok, ro.len, h, vb, w, l);  // last chunk
  if (p.fin) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (sidx(e) >= 0) p.fin[sidx(e)] = S[e];
  }
}

}  // namespace kda
