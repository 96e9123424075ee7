// kda_window.hpp -- the windowed forward (BF16 intermediates): the chunks
// are cut into windows of WIN_CHUNKS, and launch k runs the intra-chunk work
// of window k together with the state pass over window k-1.  Kernel
// boundaries order the two (no workgroup waits for another), the state pass
// reads records its predecessor launch has just written (memory-side cache),
// and the records live in a ring of two windows, so the workspace does not
// grow with the sequence length.
//
// State-pass role: one workgroup (4 waves) per (sequence, head) of the
// window; wave w owns value channels 32w..32w+31 and keeps the state for all
// 128 key channels (four 32x32 FP32 tiles) in its MFMA accumulators.  Per
// chunk (the inter-chunk algebra of kda_intra.hpp / kda_scan.hpp):
//   X   = W S0                      two 32x32 tiles over 8 key steps
//   D   = U - X
//   O^T = S0^T Qt^T + D^T P^T       output, transposed so a lane holds values
//   S   = Diag(Gam) S0 + Kb^T D
// With the contracted-index order of the FragW records, the bf16 operand
// fragment of step s of a 32x32 accumulator tile is its elements 8(s%2) ..
// 8(s%2)+7: S0 and D feed every product from registers, as the B operand of
// W S0 and Kb^T D and as the A operand of S0^T Qt^T and D^T P^T: no wave
// needs another's results.  The four waves read the same W, Qt, Kb^T, P and
// Gam, so each chunk's record is staged once through LDS (WS_A .. WS_C
// below), the copies shared by the waves, with three barriers per chunk.
#pragma once

#include "kda_common.hpp"
#include "kda_intra.hpp"
#include "kda_scan.hpp"

namespace kda {

constexpr int WIN_CHUNKS = 24;  // chunks per window
constexpr int WIN_MAX_SEQS = 64;  // sequences per batch the windowed path takes

struct WinArgs {
  IntraArgs ia;  // intra role: FragW records in the ring (ia.ring = ring)
  int intra_c0;  // first chunk of this launch's intra window, or -1
  int scan_win;  // window of this launch's state-pass role, or -1
  int nseg;      // grid rows of the state-pass role (one per sequence)
  int W;         // chunks per window
  const int32_t* cu;
  const int32_t* cfirst;  // [N+1], or null for one sequence
  int N;
  int H;
  float scale;
  const float* gam;   // [ring][H][128]
  const bf16* rec;    // [ring][H][RECW]
  int ring;           // ring length in chunks
  void* out;          // [T][H][128]
  const float* init;  // [N][H][128][128] or null
  float* fin;         // [N][H][128][128] or null
  float* carry;       // [2][H][128][128]: the state at a window boundary
};

// LDS of the state-pass role (bytes; the buffer the intra role uses in other
// workgroups): each chunk's record in three regions, in the order the step
// reads them.  A region is refilled for the next chunk as soon as every wave
// is done with it, so each copy has about two thirds of a step to land.
constexpr int WS_A = 0;                  // W [16 KB], U of all four value blocks [16 KB]
constexpr int WS_B = 32768;              // Qt [16 KB], P [6 KB]
constexpr int WS_C = 32768 + 22528;      // Kb^T [16 KB], Gam [512 B]
constexpr int WS_BYTES = WS_C + 16384 + 512;
static_assert(WS_BYTES <= IntraLds<bf16>::BYTES, "the roles share one LDS buffer");

// The copies of one chunk, split over the four waves in 1 KB units (unit u
// of a region: lane l moves bytes 16 l .. 16 l + 15).  Staged in registers:
// loaded from the record after the region is released, written to LDS one
// phase later.
struct WinStage {
  u32x4 a[8];  // region A: units w + 4 i (W for i < 4, U after)
  u32x4 b[6];  // region B: units w + 4 i < 22 (Qt for i < 4, P after)
  u32x4 c[5];  // region C: Kb^T units w + 4 i (i < 4); Gam on wave 0, lanes 0..31
};
__device__ __forceinline__ const u32x4* rec_u(const bf16* rc, int elem_off, int unit, int l) {
  return reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(rc + elem_off) + 1024 * unit) + l;
}
__device__ __forceinline__ void stage_load_a(const bf16* rc, int w, int l, WinStage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st.a[i] = *rec_u(rc, OFF_W, w + 4 * i, l);
#pragma unroll
  for (int i = 0; i < 4; ++i) st.a[4 + i] = *rec_u(rc, OFF_UT, w + 4 * i, l);
}
__device__ __forceinline__ void stage_load_b(const bf16* rc, int w, int l, WinStage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st.b[i] = *rec_u(rc, OFF_QT, w + 4 * i, l);
  st.b[4] = *rec_u(rc, OFFW_P, w, l);
  if (w < 2) st.b[5] = *rec_u(rc, OFFW_P, 4 + w, l);
}
__device__ __forceinline__ void stage_load_c(const bf16* rc, const float* gm, int w, int l,
                                             WinStage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st.c[i] = *rec_u(rc, OFF_KBT, w + 4 * i, l);
  if (w == 0 && l < 32) st.c[4] = *(reinterpret_cast<const u32x4*>(gm) + l);
}
__device__ __forceinline__ void stage_write_a(char* sm, int w, int l, const WinStage& st) {
  u32x4* d = reinterpret_cast<u32x4*>(sm + WS_A) + l;
#pragma unroll
  for (int i = 0; i < 8; ++i) d[64 * (w + 4 * i)] = st.a[i];
}
__device__ __forceinline__ void stage_write_b(char* sm, int w, int l, const WinStage& st) {
  u32x4* d = reinterpret_cast<u32x4*>(sm + WS_B) + l;
#pragma unroll
  for (int i = 0; i < 5; ++i) d[64 * (w + 4 * i)] = st.b[i];
  if (w < 2) d[64 * (w + 20)] = st.b[5];
}
__device__ __forceinline__ void stage_write_c(char* sm, int w, int l, const WinStage& st) {
  u32x4* d = reinterpret_cast<u32x4*>(sm + WS_C) + l;
#pragma unroll
  for (int i = 0; i < 4; ++i) d[64 * (w + 4 * i)] = st.c[i];
  if (w == 0 && l < 32) d[64 * 16] = st.c[4];
}
__device__ __forceinline__ bf16x8 lds_frag(const char* sm, int region, int frag, int l) {
  return *reinterpret_cast<const bf16x8*>(sm + region + 1024 * frag + 16 * l);
}

// One chunk of the state pass for wave w (value block w).  On entry region A
// holds chunk c's W and U; st.b and st.c hold the copies of its Qt, P and
// Kb^T, Gam, loaded earlier (written to regions B and C once every wave has
// released them).  `nrc`, `ngm`: the next chunk's record (or this one's again
// at the last chunk).
template <typename TO>
__device__ __forceinline__ void win_step(const WinArgs& p, char* sm, WinStage& st, const bf16* nrc,
                                         const float* ngm, int ctok, int len, int h, int w, int l,
                                         f32x16 (&S)[4]) {
  const int g = l >> 5, col = l & 31;
  // Each phase reads its LDS fragments in batches ahead of the products that
  // use them (the scheduling barriers keep the reads together), so the LDS
  // latency is paid once per batch rather than once per product.

  // ---- phase A: X = W S0, D = U - X
  bf16x8 bS[8];  // S0 as bf16 operand fragments, key step s = 16 keys
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int q = 0; q < 8; ++q) bS[s][q] = (bf16)S[s >> 1][8 * (s & 1) + q];
  f32x16 X0, X1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { X0[e] = 0.0f; X1[e] = 0.0f; }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 fa[8];  // W (s, r) = fragment 2 s + r
#pragma unroll
    for (int f = 0; f < 8; ++f) fa[f] = lds_frag(sm, WS_A, 8 * half + f, l);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int s = 4 * half + s2;
      X0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[2 * s2], bS[s], X0, 0, 0, 0);
      X1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[2 * s2 + 1], bS[s], X1, 0, 0, 0);
    }
  }
  bf16x8 dB[4];  // the 16-token steps of D as operand fragments
  {
    const bf16x8* pu = reinterpret_cast<const bf16x8*>(sm + WS_A + 16384) + (w * 2 * 64 + l) * 2;
    const bf16x8 u00 = pu[0], u01 = pu[1], u10 = pu[128], u11 = pu[129];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dB[0][q] = (bf16)((float)u00[q] - X0[q]);
      dB[1][q] = (bf16)((float)u01[q] - X0[8 + q]);
      dB[2][q] = (bf16)((float)u10[q] - X1[q]);
      dB[3][q] = (bf16)((float)u11[q] - X1[8 + q]);
    }
  }
  stage_write_b(sm, w, l, st);  // Qt, P of this chunk
  wait_lds();
  ring_barrier();  // region A released, region B complete
  stage_load_a(nrc, w, l, st);
  stage_write_c(sm, w, l, st);  // Kb^T, Gam of this chunk (region C is free)

  // ---- phase B: O^T = S0^T Qt^T + D^T P^T (rows: this wave's 32 values)
  f32x16 O0, O1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { O0[e] = 0.0f; O1[e] = 0.0f; }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 fq[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) fq[f] = lds_frag(sm, WS_B, 8 * half + f, l);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int s = 4 * half + s2;
      O0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bS[s], fq[2 * s2], O0, 0, 0, 0);
      O1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bS[s], fq[2 * s2 + 1], O1, 0, 0, 0);
    }
  }
  {
    // P is causal: output tokens 0..31 take input tokens 0..31 only
    bf16x8 fp[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) fp[f] = lds_frag(sm, WS_B, 16 + f, l);
    __builtin_amdgcn_sched_barrier(0);
    O0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dB[0], fp[0], O0, 0, 0, 0);
    O0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dB[1], fp[1], O0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) O1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dB[s], fp[2 + s], O1, 0, 0, 0);
  }

  // Output: lane (token col, g) holds values 8 e4 + 4 g + (0..3) of token
  // 32 r + col; one exchange between the lane halves per pair of e4 leaves 8
  // consecutive values per lane: 16-byte stores.
  TO* __restrict__ out = reinterpret_cast<TO*>(p.out);
  constexpr int NW = (int)sizeof(TO);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const f32x16& O = r == 0 ? O0 : O1;
    u32 wd[4][NW];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      if constexpr (sizeof(TO) == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wd[e4][j] = __builtin_bit_cast(u32, bf16x2{(bf16)(p.scale * O[4 * e4 + 2 * j]),
                                                     (bf16)(p.scale * O[4 * e4 + 2 * j + 1])});
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wd[e4][j] = __builtin_bit_cast(u32, p.scale * O[4 * e4 + j]);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const auto x = __builtin_amdgcn_permlane32_swap(wd[2 * q][j], wd[2 * q + 1][j], false, false);
        wd[2 * q][j] = x[0];
        wd[2 * q + 1][j] = x[1];
      }
    const int tk = 32 * r + col;
    if (tk < len) {
      u32x4* o = reinterpret_cast<u32x4*>(out + ((size_t)(ctok + tk) * p.H + h) * DH + 32 * w + 8 * g);
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
  wait_lds();
  ring_barrier();  // region B released, region C complete
  stage_load_b(nrc, w, l, st);

  // ---- phase C: S = Diag(Gam) S0 + Kb^T D; lane (col, g) holds keys 32 t + 8 j + 4 g + (0..3)
  // two state tiles at a time: their Gam scaling, then their 8 products
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    bf16x8 fk[8];  // Kb^T (s, t) = fragment 4 s + t, t = 2 tp, 2 tp + 1
    f32x4 gv[8];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u) fk[2 * s + u] = lds_frag(sm, WS_C, 4 * s + 2 * tp + u, l);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gv[4 * u + j] = *reinterpret_cast<const f32x4*>(sm + WS_C + 16384 +
                                                         4 * (32 * (2 * tp + u) + 8 * j + 4 * g));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[2 * tp + u][4 * j + i] *= gv[4 * u + j][i];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        S[2 * tp + u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[2 * s + u], dB[s], S[2 * tp + u],
                                                                0, 0, 0);
  }
  stage_write_a(sm, w, l, st);  // W, U of the next chunk
  wait_lds();
  ring_barrier();  // region C released, region A holds the next chunk
  stage_load_c(nrc, ngm, w, l, st);
}

// The state-pass role: sequence `seg` (counted from the first sequence that
// reaches into the window) and head h over the chunks of window p.scan_win.
template <typename TO>
__device__ __forceinline__ void win_scan(const WinArgs& p, int seg, int h, char* sm) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, col = l & 31;
  const int win = p.scan_win;
  const int Ctot = p.cfirst ? p.cfirst[p.N] : (p.cu[1] - p.cu[0] + CHUNK - 1) / CHUNK;
  const int A = win * p.W, B = min(A + p.W, Ctot);
  int n = 0;
  if (p.cfirst) {
    // first sequence whose chunks end at or after the window start
    int lo = 0, hi = p.N;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.cfirst[mid + 1] >= A) hi = mid; else lo = mid + 1;
    }
    n = lo + seg;
    if (n >= p.N) return;
  } else if (seg != 0) {
    return;
  }
  const int cb = p.cfirst ? p.cfirst[n] : 0, ce = p.cfirst ? p.cfirst[n + 1] : Ctot;
  const size_t nh = (size_t)n * p.H + h;
  // state entry (key 32 t + row32(e, l), value 32 w + col) of array base x
  auto at = [&](size_t x, int t, int e) {
    return (x * DH + 32 * t + row32(e, l)) * DH + 32 * w + col;
  };
  if (cb == ce) {
    // an empty sequence: its end state is its start state, written once (by
    // the window its position falls in, or the last one)
    // (at least one window: with no chunks at all, as after a failed
    // cu_seqlens check, every sequence is empty and window 0 writes them)
    const int nwin = max(1, (Ctot + p.W - 1) / p.W);
    if (min(cb / p.W, nwin - 1) != win || !p.fin) return;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) p.fin[at(nh, t, e)] = p.init ? p.init[at(nh, t, e)] : 0.0f;
    return;
  }
  const int lo_c = max(cb, A), hi_c = min(ce, B);
  if (lo_c >= hi_c) return;
  f32x16 S[4];
  const size_t cin = (size_t)(win & 1) * p.H + h, cout = (size_t)((win + 1) & 1) * p.H + h;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      S[t][e] = lo_c > cb ? p.carry[at(cin, t, e)] : (p.init ? p.init[at(nh, t, e)] : 0.0f);
  const int tseq = p.cu[n], tend = p.cu[n + 1];
  auto rec_of = [&](int c) { return p.rec + ((size_t)(c % p.ring) * p.H + h) * RECW; };
  auto gam_of = [&](int c) { return p.gam + ((size_t)(c % p.ring) * p.H + h) * DH; };
  // the first chunk's record: region A written, B and C staged
  WinStage st;
  stage_load_a(rec_of(lo_c), w, l, st);
  stage_load_b(rec_of(lo_c), w, l, st);
  stage_load_c(rec_of(lo_c), gam_of(lo_c), w, l, st);
  stage_write_a(sm, w, l, st);
  wait_lds();
  ring_barrier();
  for (int c = lo_c; c < hi_c; ++c) {
    const int ctok = tseq + (c - cb) * CHUNK;
    const int nx = min(c + 1, hi_c - 1);  // past the last chunk: reload it (unused)
    win_step<TO>(p, sm, st, rec_of(nx), gam_of(nx), ctok, min(CHUNK, tend - ctok), h, w, l, S);
  }
  if (hi_c < ce) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) p.carry[at(cout, t, e)] = S[t][e];
  } else if (p.fin) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) p.fin[at(nh, t, e)] = S[t][e];
  }
}

// Launch k of the windowed forward: grid (H, rows); rows [0, nseg) are the
// state pass over window k-1 (when scan_win >= 0), the next W rows the intra
// work of window k (when intra_c0 >= 0).  State-pass rows come first so they
// are dispatched first.
template <typename TA, typename TO, bool CONV>
__global__ __launch_bounds__(256, 2) void kda_window_kernel(WinArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[IntraLds<bf16>::BYTES];
  const int y = (int)blockIdx.y, h = (int)blockIdx.x;
  const int nscan = p.scan_win >= 0 ? p.nseg : 0;
  if (y < nscan) {
    win_scan<TO>(p, y, h, smem);
    return;
  }
  intra_chunk<TA, bf16, CONV, FragW<bf16>, false>(p.ia, p.intra_c0 + (y - nscan), h, smem);
}

}  // namespace kda
