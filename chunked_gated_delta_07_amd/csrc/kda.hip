// kda.hip -- libkda: C ABI entry points (include/kda.h), argument checks,
// workspace layout and kernel launches for the KDA chunked forward on gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_intra.hpp"
#include "kda_scan.hpp"
#include "kda_window.hpp"
#include "kda_recurrent.hpp"
#include "kda_bwd.hpp"
#include "kda_conv_bwd.hpp"

namespace kda {

// ------------------------------------------------------------ chunk table
// cfirst[n] = number of 64-token chunks in sequences 0..n-1 (chunks restart
// at every sequence start: packed offsets, xtuner PR #2301 section Change).
// One workgroup of 1024 threads; each thread owns a contiguous slice of
// sequences.  Also writes cfirst[N] = total chunks.
// With a status pointer (KDA_MODE_CHECK_CU) the offsets are checked first:
// bit 0 cu[0] != 0, bit 1 a decrease, bit 2 cu[N] != T.  The code is stored at
// *status (0: valid); when it is not 0 the table says every sequence is empty,
// so no later kernel touches token data (every token range is derived from it).
__global__ __launch_bounds__(1024) void kda_chunk_table_kernel(const int32_t* __restrict__ cu, int N,
                                                                int32_t* __restrict__ cfirst,
                                                                int64_t T, int32_t* __restrict__ status) {
  __shared__ int32_t part[1024];
  __shared__ int32_t bad;
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int lo = min(N, tid * per), hi = min(N, lo + per);
  if (status) {
    if (tid == 0) bad = 0;
    __syncthreads();
    int code = 0;
    for (int n = lo; n < hi; ++n)
      if (cu[n + 1] < cu[n]) code |= 2;
    if (tid == 0 && cu[0] != 0) code |= 1;
    if (tid == 0 && (int64_t)cu[N] != T) code |= 4;
    if (code) atomicOr(&bad, code);
    __syncthreads();
    if (bad) {
      for (int n = tid; n <= N; n += 1024) cfirst[n] = 0;
      if (tid == 0) *status = bad;
      return;
    }
    if (tid == 0) *status = 0;
  }
  int32_t s = 0;
  for (int n = lo; n < hi; ++n) s += (cu[n + 1] - cu[n] + CHUNK - 1) / CHUNK;
  part[tid] = s;
  __syncthreads();
  // inclusive scan over the 1024 partial sums (Hillis-Steele)
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int32_t run = part[tid] - s;  // exclusive prefix of this thread's slice
  for (int n = lo; n < hi; ++n) {
    cfirst[n] = run;
    run += (cu[n + 1] - cu[n] + CHUNK - 1) / CHUNK;
  }
  if (tid == 1023) cfirst[N] = part[1023];
}

// The backward's per-chunk kernels address a chunk's rows of a [T][H][128]
// tensor with 32-bit offsets from the chunk's first token (up to 64 H 128).
static inline bool bwd_heads_fit(int64_t H) { return H * DH * CHUNK <= (int64_t)INT32_MAX; }

// A dispatch counts each grid dimension in work-items with a 32-bit field:
// blocks x threads must stay below 2^32 in every dimension.
static inline bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks * threads <= (int64_t)UINT32_MAX;
}

// The chunk table (checked when `check`); a single unchecked sequence needs
// none (its chunk c starts at token 64 c) and gets a null table.
static inline int32_t* launch_table(const int32_t* cu, int32_t N, int64_t T, int32_t* cfirst,
                                    void* ws, bool check, hipStream_t stream) {
  if (N == 1 && !check) return nullptr;
  hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(1024), 0, stream, cu, (int)N, cfirst, T,
                     check ? reinterpret_cast<int32_t*>(ws) : (int32_t*)nullptr);
  return cfirst;
}

// ------------------------------------------------------------ workspace
// [cfirst: (N+1) int32, 256-aligned][gam: chunks*H*128 float][rec: chunks*H*REC MT]
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Upper bound on the number of chunks: each non-empty sequence of length L has
// ceil(L/64) <= (L + 63)/64 chunks, at most min(N, T) sequences are non-empty.
static inline int64_t max_chunks(int64_t T, int64_t N) {
  const int64_t ne = N < T ? N : T;
  return (T + 63 * ne) / 64;
}

// The windowed schedule (kda_window.hpp) when asked for, with BF16
// intermediates and at most WIN_MAX_SEQS sequences (the state-pass role of a
// window has one grid row per sequence); otherwise two passes.
static inline bool use_windows(int32_t N, uint32_t mode) {
  return (mode & KDA_MODE_WINDOWED) && !(mode & KDA_MODE_FP32_INTERMEDIATE) && N <= WIN_MAX_SEQS;
}

// Segments of the two-pass schedule: with BF16 intermediates a long batch
// runs as segments of SEG_CHUNKS chunks, each an intra-chunk launch followed
// by a state-pass launch over the same chunks, the records in a ring of one
// segment and the state of a sequence crossing a boundary carried in FP32
// (the results are those of one pass over everything, bit for bit).  A
// segment's records (about 150 MB at 64 heads) stay in the memory-side cache
// until the state pass reads them.  FP32 intermediates run as one segment:
// their records are twice the size, and segments made that forward slower
// (2.07 -> 2.13 ms with four); its state pass is bound by its split products
// rather than by the record reads.
static inline int64_t seg_count(int64_t T, int32_t N, uint32_t mode) {
  const int64_t C = max_chunks(T, N);
  if ((mode & KDA_MODE_FP32_INTERMEDIATE) || C <= SEG_CHUNKS) return 1;
  return (C + SEG_CHUNKS - 1) / SEG_CHUNKS;
}

// Record slots: every chunk (two passes), or a ring of two windows.
static inline int64_t ring_chunks(int64_t T, int32_t N) {
  const int64_t C = max_chunks(T, N);
  return C < 2 * WIN_CHUNKS ? C : 2 * WIN_CHUNKS;
}

struct WsLayout {
  size_t off_cfirst, off_gam, off_rec, off_carry, total;
};

// two passes: [cfirst][gam: chunks x H x 128 f32][rec: chunks x H x Frag<MT> record]
// segmented:  [cfirst][gam: 32 x H x 128 f32][rec: 32 x H x Frag<bf16> record][carry: 2 x H x 128 x 128 f32]
// windowed:   [cfirst][gam: ring x H x 128 f32][rec: ring x H x RECW bf16][carry: 2 x H x 128 x 128 f32]
static inline WsLayout ws_layout(int64_t T, int32_t N, int32_t H, uint32_t mode) {
  const size_t mt = (mode & KDA_MODE_FP32_INTERMEDIATE) ? 4 : 2;
  const bool win = use_windows(N, mode), seg = !win && seg_count(T, N, mode) > 1;
  const int64_t C = win ? ring_chunks(T, N) : seg ? SEG_CHUNKS : max_chunks(T, N);
  WsLayout L;
  L.off_cfirst = 256;  // [0, 4): status word of KDA_MODE_CHECK_CU
  L.off_gam = L.off_cfirst + align256(sizeof(int32_t) * (size_t)(N + 1));
  L.off_rec = L.off_gam + align256(sizeof(float) * (size_t)C * H * DH);
  const size_t rec_elems = win ? RECW : mt == 2 ? Frag<bf16>::REC_ELEMS : Frag<float>::REC_ELEMS;
  L.off_carry = L.off_rec + align256(mt * (size_t)C * H * rec_elems);
  L.total = L.off_carry + (win || seg ? align256(sizeof(float) * 2 * (size_t)H * DH * DH) : 0);
  return L;
}

// End states of an empty batch (every sequence empty): fin = init, or zero.
__global__ __launch_bounds__(256) void kda_state_copy_kernel(const float* __restrict__ init,
                                                             float* __restrict__ fin, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    fin[i] = init ? init[i] : 0.0f;
}

template <typename TA, typename MT, typename TO, bool RECT = false>
static int launch_all(const void* q, const void* k, const void* v, const void* f, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                      int64_t T, int32_t H, uint32_t mode, void* out, void* ws,
                      const float* init, float* fin, const float* conv_w, const float* conv_b,
                      int conv_silu, hipStream_t stream, hipEvent_t const* ev, int dk = DH,
                      int dv = DH) {
  const WsLayout W = ws_layout(T, N, H, mode);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* cfirst = reinterpret_cast<int32_t*>(base + W.off_cfirst);
  float* gam = reinterpret_cast<float*>(base + W.off_gam);
  void* rec = base + W.off_rec;
  const int64_t C = max_chunks(T, N);

  if (ev) (void)hipEventRecord(ev[0], stream);
  cfirst = launch_table(cu, N, T, cfirst, ws, mode & KDA_MODE_CHECK_CU, stream);
  if (ev) (void)hipEventRecord(ev[1], stream);

  // one segment, or segments of SEG_CHUNKS chunks (BF16 intermediates only)
  const int64_t nseg = seg_count(T, N, mode);
  const int64_t per = nseg > 1 ? SEG_CHUNKS : C;
  float* carry = nseg > 1 ? reinterpret_cast<float*>(base + W.off_carry) : nullptr;

  IntraArgs ia;
  ia.q = q; ia.k = k; ia.v = v; ia.f = f; ia.b = b;
  ia.A_log = A_log; ia.dt_bias = dt_bias; ia.cu = cu; ia.cfirst = cfirst;
  ia.N = N; ia.H = H; ia.eps = 1e-6f; ia.gam = gam; ia.rec = rec;
  ia.conv_w = conv_w; ia.conv_b = conv_b; ia.conv_silu = conv_silu;
  ia.tmat = nullptr; ia.bw = nullptr; ia.wt = nullptr; ia.kbr = nullptr;
  ia.ring = nseg > 1 ? SEG_CHUNKS : 0;
  ia.dk = dk; ia.dv = dv;

  ScanArgs sa;
  sa.cu = cu; sa.cfirst = cfirst; sa.N = N; sa.H = H;
  sa.scale = (float)(1.0 / sqrt((double)dk));  // 1/sqrt(d_k), correctly rounded
  sa.gam = gam; sa.rec = rec; sa.out = out; sa.init = init; sa.fin = fin;
  sa.dk = dk; sa.dv = dv;
  sa.ring = ia.ring;
  // 32 workgroups (four value blocks of eight (sequence, head) pairs) per
  // grid row; workgroup id = x + 32 y
  const int64_t pairs = (int64_t)N * H;
  const dim3 gscan(32, (unsigned)((pairs + 7) / 8));
  const size_t cstride = (size_t)H * DH * DH;
  for (int64_t sg = 0; sg < nseg; ++sg) {
    const int64_t c0 = sg * per, rows = (C - c0 < per) ? C - c0 : per;
    ia.c0 = (int)c0;
    const dim3 gintra((unsigned)H, (unsigned)rows);  // heads x chunks (sizes checked by the caller)
    if constexpr (RECT)
      hipLaunchKernelGGL((kda_intra_kernel<TA, MT, false, Frag<MT>, false, true>), gintra, dim3(256),
                         0, stream, ia);
    else if (conv_w)
      hipLaunchKernelGGL((kda_intra_kernel<TA, MT, true>), gintra, dim3(256), 0, stream, ia);
    else
      hipLaunchKernelGGL((kda_intra_kernel<TA, MT, false>), gintra, dim3(256), 0, stream, ia);
    if (ev) (void)hipEventRecord(ev[2 + 2 * sg], stream);

    sa.c0 = (int)c0;
    sa.c1 = sg + 1 < nseg ? (int)(c0 + per) : INT32_MAX;  // the last one takes everything after
    sa.carry_in = carry ? carry + ((sg + 1) & 1) * cstride : nullptr;
    sa.carry_out = carry ? carry + (sg & 1) * cstride : nullptr;
    if constexpr (sizeof(MT) == 2)
      hipLaunchKernelGGL((kda_scan_ring_kernel<TO, RECT>), gscan, dim3(512), 0, stream, sa);
    else
      hipLaunchKernelGGL((kda_scan_ring32_kernel<TO, RECT>), gscan, dim3(512), 0, stream, sa);
    if (ev) (void)hipEventRecord(ev[3 + 2 * sg], stream);
  }
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// The windowed forward: the chunk table, then launch k = 0 .. nwin of
// kda_window_kernel (intra work of window k, state pass over window k-1).
template <typename TA, typename TO>
static int launch_windows(const void* q, const void* k, const void* v, const void* f, const void* b,
                          const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                          int64_t T, int32_t H, uint32_t mode, void* out, void* ws,
                          const float* init, float* fin, const float* conv_w, const float* conv_b,
                          int conv_silu, hipStream_t stream, hipEvent_t const* ev) {
  const WsLayout L = ws_layout(T, N, H, mode);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* cfirst = reinterpret_cast<int32_t*>(base + L.off_cfirst);
  const int64_t C = max_chunks(T, N);  // upper bound; the kernels know the real count
  const int W = WIN_CHUNKS;
  const int64_t nwin = (C + W - 1) / W;

  if (ev) (void)hipEventRecord(ev[0], stream);
  cfirst = launch_table(cu, N, T, cfirst, ws, mode & KDA_MODE_CHECK_CU, stream);
  if (ev) (void)hipEventRecord(ev[1], stream);

  WinArgs wa;
  IntraArgs& ia = wa.ia;
  ia.q = q; ia.k = k; ia.v = v; ia.f = f; ia.b = b;
  ia.A_log = A_log; ia.dt_bias = dt_bias; ia.cu = cu; ia.cfirst = cfirst;
  ia.N = N; ia.H = H; ia.eps = 1e-6f;
  ia.gam = reinterpret_cast<float*>(base + L.off_gam);
  ia.rec = base + L.off_rec;
  ia.ring = (int)ring_chunks(T, N);
  ia.c0 = 0;
  ia.conv_w = conv_w; ia.conv_b = conv_b; ia.conv_silu = conv_silu;
  ia.tmat = nullptr; ia.bw = nullptr; ia.wt = nullptr; ia.kbr = nullptr;
  wa.nseg = N; wa.W = W;
  wa.cu = cu; wa.cfirst = cfirst; wa.N = N; wa.H = H;
  wa.scale = 0.08838834764831845f;  // 1/sqrt(128)
  wa.gam = ia.gam;
  wa.rec = reinterpret_cast<const bf16*>(ia.rec);
  wa.ring = ia.ring;
  wa.out = out; wa.init = init; wa.fin = fin;
  wa.carry = reinterpret_cast<float*>(base + L.off_carry);
  for (int64_t kw = 0; kw <= nwin; ++kw) {
    wa.scan_win = kw >= 1 ? (int)(kw - 1) : -1;
    wa.intra_c0 = kw < nwin ? (int)(kw * W) : -1;
    const unsigned rows = (unsigned)((kw >= 1 ? N : 0) + (kw < nwin ? W : 0));
    if (conv_w)
      hipLaunchKernelGGL((kda_window_kernel<TA, TO, true>), dim3((unsigned)H, rows), dim3(256), 0,
                         stream, wa);
    else
      hipLaunchKernelGGL((kda_window_kernel<TA, TO, false>), dim3((unsigned)H, rows), dim3(256), 0,
                         stream, wa);
  }
  if (ev) (void)hipEventRecord(ev[2], stream);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static int dispatch(const void* q, const void* k, const void* v, const void* f, const void* b,
                    const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                    int64_t T, int32_t H, uint32_t mode, void* out, void* ws, const float* init,
                    float* fin, const float* conv_w, const float* conv_b, int conv_silu,
                    hipStream_t s, hipEvent_t const* ev) {
  const bool f32i = mode & KDA_MODE_FP32_INTERMEDIATE;
  const bool a32 = mode & KDA_ACT_FP32;
  const bool o32 = (mode & KDA_OUT_FP32) || a32;
  if (use_windows(N, mode)) {
#define KDA_WIN(TA, TO)                                                                             \
  return launch_windows<TA, TO>(q, k, v, f, b, A_log, dt_bias, cu, N, T, H, mode, out, ws, init, \
                                fin, conv_w, conv_b, conv_silu, s, ev)
    if (a32) KDA_WIN(float, float);
    if (o32) KDA_WIN(bf16, float);
    KDA_WIN(bf16, bf16);
#undef KDA_WIN
  }
#define KDA_GO(TA, MT, TO) \
  return launch_all<TA, MT, TO>(q, k, v, f, b, A_log, dt_bias, cu, N, T, H, mode, out, ws, init, \
                                fin, conv_w, conv_b, conv_silu, s, ev)
  if (!a32 && !f32i && !o32) KDA_GO(bf16, bf16, bf16);
  if (!a32 && !f32i && o32) KDA_GO(bf16, bf16, float);
  if (!a32 && f32i && !o32) KDA_GO(bf16, float, bf16);
  if (!a32 && f32i && o32) KDA_GO(bf16, float, float);
  if (a32 && !f32i) KDA_GO(float, bf16, float);
  KDA_GO(float, float, float);
#undef KDA_GO
}


// ------------------------------------------------------------ backward
// Workspace of the backward, FP32 arrays per (chunk, head) after the chunk
// table.  The outputs of the products kernel take the space of arrays whose
// only readers are the two scans, which have finished by then: dQt, dKb and
// dP the records, dBw W^T, dA the Kb copy, dGam Gam (dW never leaves it).
struct BwdLayout {
  size_t off_cfirst, off_gam, off_rec, off_t, off_bw, off_wt, off_kbr, off_s0, off_dsn, off_d,
      off_dd, off_dqt, off_dkb, off_dbw, off_dp, off_da, off_dgam, off_db1, off_pp, total;
};

static inline BwdLayout bwd_layout(int64_t T, int32_t N, int32_t H) {
  const size_t CH = (size_t)max_chunks(T, N) * H;
  BwdLayout L;
  size_t o = 256;  // [0, 4): status word of KDA_MODE_CHECK_CU
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.off_cfirst = take(sizeof(int32_t) * (size_t)(N + 1));
  L.off_gam = take(4 * CH * DH);
  L.off_rec = take(4 * CH * REC);
  L.off_t = take(4 * CH * SQM);
  L.off_bw = take(4 * CH * MAT);
  L.off_wt = take(4 * CH * MAT);
  L.off_kbr = take(4 * CH * MAT);
  L.off_s0 = take(4 * CH * STM);
  L.off_dsn = take(4 * CH * STM);
  L.off_d = take(4 * CH * MAT);
  L.off_dd = take(4 * CH * MAT);
  static_assert(2 * MAT + SQM <= REC, "dQt, dKb and dP fit in the records");
  L.off_dqt = L.off_rec;
  L.off_dkb = L.off_dqt + 4 * CH * MAT;
  L.off_dp = L.off_dkb + 4 * CH * MAT;
  L.off_dbw = L.off_wt;
  L.off_da = L.off_kbr;
  L.off_dgam = L.off_gam;
  L.off_db1 = take(4 * CH * CHUNK);
  L.off_pp = take(4 * CH * PPART);
  L.total = o;
  return L;
}

template <typename TA, typename TG, typename TR>
static int launch_bwd(const void* q, const void* k, const void* v, const void* f, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                      int64_t T, int32_t H, const float* init, const void* dout, const float* dfin,
                      void* dq, void* dk, void* dv, void* df, void* db, float* dA_log, float* ddt,
                      float* dinit, void* ws, hipStream_t stream, bool check) {
  const BwdLayout L = bwd_layout(T, N, H);
  char* base = reinterpret_cast<char*>(ws);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  int32_t* cfirst = reinterpret_cast<int32_t*>(base + L.off_cfirst);
  const int64_t C = max_chunks(T, N);
  // the backward's kernels always take a table
  hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(1024), 0, stream, cu, (int)N, cfirst, T,
                     check ? reinterpret_cast<int32_t*>(ws) : (int32_t*)nullptr);

  IntraArgs ia;
  ia.q = q; ia.k = k; ia.v = v; ia.f = f; ia.b = b;
  ia.A_log = A_log; ia.dt_bias = dt_bias; ia.cu = cu; ia.cfirst = cfirst;
  ia.N = N; ia.H = H; ia.eps = 1e-6f; ia.gam = fp(L.off_gam); ia.rec = fp(L.off_rec);
  ia.conv_w = nullptr; ia.conv_b = nullptr; ia.conv_silu = 0;
  ia.tmat = fp(L.off_t); ia.bw = fp(L.off_bw); ia.wt = fp(L.off_wt); ia.kbr = fp(L.off_kbr); ia.ring = 0;
  ia.c0 = 0;
  const dim3 gch((unsigned)C, (unsigned)H);
  hipLaunchKernelGGL((kda_intra_kernel<TA, float, false, PlainRec<float>, true>), gch, dim3(256), 0,
                     stream, ia);

  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.f = f; a.b = b; a.dout = dout;
  a.A_log = A_log; a.dt_bias = dt_bias; a.cu = cu; a.cfirst = cfirst;
  a.init = init; a.dfin = dfin; a.N = N; a.H = H; a.eps = 1e-6f;
  a.scale = 0.08838834764831845f;  // 1/sqrt(128)
  a.rec = fp(L.off_rec); a.gam = fp(L.off_gam); a.tmat = fp(L.off_t); a.bw = fp(L.off_bw);
  a.wt = fp(L.off_wt); a.kbr = fp(L.off_kbr);
  a.s0 = fp(L.off_s0); a.dsn = fp(L.off_dsn); a.dmat = fp(L.off_d); a.ddmat = fp(L.off_dd);
  a.dqt = fp(L.off_dqt); a.dkb = fp(L.off_dkb); a.dbw = fp(L.off_dbw);
  a.dpm = fp(L.off_dp); a.dam = fp(L.off_da); a.dgam = fp(L.off_dgam); a.db1 = fp(L.off_db1);
  a.ppart = fp(L.off_pp);
  a.dq = dq; a.dk = dk; a.dv = dv; a.df = df; a.db = db;
  a.dinit = dinit; a.dA_log = dA_log; a.ddt_bias = ddt;
  const int64_t pairs = (int64_t)N * H;
  const dim3 gscan(32, (unsigned)((pairs + 7) / 8));  // workgroup id = x + 32 y
  hipLaunchKernelGGL(kda_bwd_fscan_kernel, gscan, dim3(SCAN_THREADS), 0, stream, a);
  hipLaunchKernelGGL((kda_bwd_bscan_kernel<TG>), gscan, dim3(SCAN_THREADS), 0, stream, a);
  hipLaunchKernelGGL((kda_bwd_prod_kernel<TA, TG, TR>), gch, dim3(256), 0, stream, a);
  hipLaunchKernelGGL((kda_bwd_gate_kernel<TA, TR>), gch, dim3(512), 0, stream, a);
  hipLaunchKernelGGL(kda_bwd_param_kernel, dim3((unsigned)H), dim3(DH), 0, stream, a);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward through the fused convolution: the backward's own workspace, then
// the convolution outputs (activation dtype), their FP32 gradients, FP32
// gradients of f_raw and b_raw (cast at the end when the gradients are bf16)
// and the per-chunk tap / bias partials.
struct ConvBwdLayout {
  BwdLayout core;
  size_t off_y, off_dy, off_df, off_db, off_part, total;
};

static inline ConvBwdLayout conv_bwd_layout(int64_t T, int32_t N, int32_t H, uint32_t mode) {
  ConvBwdLayout L;
  L.core = bwd_layout(T, N, H);
  const size_t act = (mode & KDA_ACT_FP32) ? 4 : 2;
  const size_t n = (size_t)T * H * DH;
  size_t o = L.core.total;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.off_y = take(3 * n * act);
  L.off_dy = take(3 * n * 4);
  L.off_df = take(n * 4);
  L.off_db = take((size_t)T * H * 4);
  L.off_part = take((size_t)max_chunks(T, N) * H * 3 * DH * 5 * 4);
  L.total = o;
  return L;
}

template <typename TA, typename TG, typename TR>
static int launch_bwd_conv(const void* q, const void* k, const void* v, const void* f, const void* b,
                           const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                           int64_t T, int32_t H, uint32_t mode, const float* conv_w,
                           const float* conv_b, int conv_silu, const float* init, const void* dout,
                           const float* dfin, void* dq, void* dk, void* dv, void* df, void* db,
                           float* dA_log, float* ddt, float* dinit, float* dconv_w, float* dconv_b,
                           void* ws, hipStream_t stream) {
  const ConvBwdLayout L = conv_bwd_layout(T, N, H, mode);
  char* base = reinterpret_cast<char*>(ws);
  const size_t n = (size_t)T * H * DH;
  const size_t act = sizeof(TA);
  const int64_t C = max_chunks(T, N);
  ConvBwdArgs a;
  a.cu = cu;
  a.cfirst = reinterpret_cast<int32_t*>(base + L.core.off_cfirst);
  a.N = N; a.H = H;
  a.x[0] = q; a.x[1] = k; a.x[2] = v;
  for (int i = 0; i < 3; ++i) {
    a.y[i] = base + L.off_y + i * n * act;
    a.dy[i] = reinterpret_cast<float*>(base + L.off_dy) + i * n;
  }
  a.dx[0] = dq; a.dx[1] = dk; a.dx[2] = dv;
  a.w = conv_w; a.b = conv_b; a.silu = conv_silu;
  a.part = reinterpret_cast<float*>(base + L.off_part);
  a.dw = dconv_w; a.db = dconv_b;
  // chunk table (the core's backward rebuilds the same one), convolution outputs
  const bool check = mode & KDA_MODE_CHECK_CU;
  hipLaunchKernelGGL(kda_chunk_table_kernel, dim3(1), dim3(1024), 0, stream, cu, (int)N,
                     const_cast<int32_t*>(a.cfirst), T,
                     check ? reinterpret_cast<int32_t*>(ws) : (int32_t*)nullptr);
  const dim3 gconv((unsigned)C, (unsigned)((H + CONV_HEADS_PER_BLOCK - 1) / CONV_HEADS_PER_BLOCK), 3);
  hipLaunchKernelGGL((kda_conv_apply_kernel<TA>), gconv, dim3(256), 0, stream, a);
  // the core's backward on the convolution outputs, FP32 gradients
  const bool cast = sizeof(TR) != 4;
  float* df32 = reinterpret_cast<float*>(base + L.off_df);
  float* db32 = reinterpret_cast<float*>(base + L.off_db);
  const int st = launch_bwd<TA, TG, float>(
      a.y[0], a.y[1], a.y[2], f, b, A_log, dt_bias, cu, N, T, H, init, dout, dfin,
      const_cast<float*>(a.dy[0]), const_cast<float*>(a.dy[1]), const_cast<float*>(a.dy[2]),
      cast ? (void*)df32 : df, cast ? (void*)db32 : db, dA_log, ddt, dinit, ws, stream, check);
  if (st != KDA_OK) return st;
  // input gradients through the convolution, tap and bias gradients
  hipLaunchKernelGGL((kda_conv_bwd_kernel<TA, TR>), gconv, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(kda_conv_param_kernel, dim3((unsigned)H, 3), dim3(128), 0, stream, a);
  if (cast) {
    const int64_t blocks = ((int64_t)n + 255) / 256 < 8192 ? ((int64_t)n + 255) / 256 : 8192;
    hipLaunchKernelGGL((kda_cast_kernel<TR>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float*)df32, df, (int64_t)n);
    hipLaunchKernelGGL((kda_cast_kernel<TR>), dim3(1024), dim3(256), 0, stream,
                       (const float*)db32, db, (int64_t)T * H);
  }
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda

// ================================================================ C ABI
static int check_args(const void* q, const void* k, const void* v, const void* f, const void* b,
                      const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N,
                      int64_t T, int32_t H, int32_t d, uint32_t mode, void* out, void* ws,
                      size_t ws_bytes) {
  if (mode & ~KDA_MODE_ALL_BITS) return KDA_ERR_INVALID_ARG;
  if (N < 1 || T < 0 || H < 1) return KDA_ERR_INVALID_ARG;
  if (d != kda::DH) return KDA_ERR_UNSUPPORTED;
  if (T == 0) return KDA_OK;
  if (!q || !k || !v || !f || !b || !A_log || !dt_bias || !cu || !out || !ws)
    return KDA_ERR_INVALID_ARG;
  if (T > (int64_t)INT32_MAX / 64 || (int64_t)N * H > (int64_t)INT32_MAX / 64)
    return KDA_ERR_UNSUPPORTED;
  // grids: intra (H x 256 threads, chunks), state pass (32 x 512, N H / 8)
  if (!kda::grid_fits(H, 256) || !kda::grid_fits(kda::max_chunks(T, N), 1) ||
      !kda::grid_fits(((int64_t)N * H + 7) / 8, 1))
    return KDA_ERR_UNSUPPORTED;
  if (ws_bytes < kda::ws_layout(T, N, H, mode).total) return KDA_ERR_WORKSPACE;
  return KDA_OK;
}

extern "C" size_t kda_chunk_fwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                                int32_t d, uint32_t mode) {
  if ((mode & ~KDA_MODE_ALL_BITS) || total_tokens < 0 || num_seqs < 1 || H < 1 || d != kda::DH)
    return (size_t)-1;
  if (total_tokens == 0) return 0;
  return kda::ws_layout(total_tokens, num_seqs, H, mode).total;
}

extern "C" int kda_chunk_fwd_num_stages(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                        uint32_t mode) {
  (void)H;
  if ((mode & ~KDA_MODE_ALL_BITS) || num_seqs < 1 || total_tokens < 0) return -1;
  // windowed: table, windows; two passes: table, then intra and state pass per segment
  return kda::use_windows(num_seqs, mode) ? 2 : (int)(1 + 2 * kda::seg_count(total_tokens, num_seqs, mode));
}

static int fwd_impl(const void* q, const void* k, const void* v, const void* f_raw, const void* b_raw,
                    const float* A_log, const float* dt_bias, const int32_t* cu, int32_t N, int64_t T,
                    int32_t H, int32_t d, uint32_t mode, void* out, void* ws, size_t ws_bytes,
                    const float* init, float* fin, const float* conv_w, const float* conv_b,
                    int conv_silu, void* stream, void* const* events, int32_t num_events) {
  int st = check_args(q, k, v, f_raw, b_raw, A_log, dt_bias, cu, N, T, H, d, mode, out, ws, ws_bytes);
  if (st != KDA_OK) return st;
  if (T == 0) {
    if (!fin) return KDA_OK;
    (void)hipGetLastError();
    const int64_t n = (int64_t)N * H * kda::DH * kda::DH;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(kda::kda_state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), init, fin, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  if (events && num_events != kda_chunk_fwd_num_stages(T, N, H, mode) + 1) return KDA_ERR_INVALID_ARG;
  if (events)
    for (int i = 0; i < num_events; ++i)
      if (!events[i]) return KDA_ERR_INVALID_ARG;
  (void)hipGetLastError();  // clear a stale error so the status reflects these launches
  return kda::dispatch(q, k, v, f_raw, b_raw, A_log, dt_bias, cu, N, T, H, mode, out, ws, init, fin,
                       conv_w, conv_b, conv_silu, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<hipEvent_t const*>(events));
}

extern "C" int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* f_raw,
                             const void* b_raw, const float* A_log, const float* dt_bias,
                             const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                             int32_t H, int32_t d, uint32_t mode, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, d,
                  mode, out, workspace, workspace_bytes, nullptr, nullptr, nullptr, nullptr, 0, stream,
                  nullptr, 0);
}

// ------------------------------------------------------------ no-allocation forward
// The workspace of kda_chunk_fwd_noalloc: a device array of the library's own
// (every GPU the library runs on holds one until the process ends).  In host
// code `scratch` names a host-side stand-in, not device memory, so kernels get
// the address hipGetSymbolAddress returns for the current device instead.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, set once

// Device address of `scratch` on device dev (made current for the lookup).
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KDA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return KDA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return KDA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}
}  // namespace

extern "C" int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const void* f_raw, const void* b_raw, const float* A_log,
                                     const float* dt_bias, const int32_t* cu_seqlens,
                                     int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d,
                                     uint32_t mode, void* out, void* stream) {
  // every size check comes before the first HIP call; a workspace larger than
  // the library's array is refused
  if (mode & KDA_MODE_CHECK_CU) return (mode & ~KDA_MODE_ALL_BITS) ? KDA_ERR_INVALID_ARG : KDA_ERR_UNSUPPORTED;
  const size_t need = kda_chunk_fwd_workspace_bytes(total_tokens, num_seqs, H, d, mode);
  if (need == (size_t)-1) {
    if (mode & ~KDA_MODE_ALL_BITS) return KDA_ERR_INVALID_ARG;
    if (num_seqs < 1 || total_tokens < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    return KDA_ERR_UNSUPPORTED;
  }
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  if (total_tokens == 0)
    return check_args(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, 0, H, d, mode,
                      out, nullptr, 0);
  // argument errors before the device lookup (the workspace is ours and large enough)
  int st = check_args(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H,
                      d, mode, out, reinterpret_cast<void*>(256), (size_t)KDA_NOALLOC_SCRATCH_BYTES);
  if (st != KDA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &dev) != hipSuccess) return KDA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return KDA_ERR_HIP;
  }
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != KDA_OK) return st;
  return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, d,
                  mode, out, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, nullptr, nullptr, nullptr,
                  nullptr, 0, stream, nullptr, 0);
}

extern "C" int kda_chunk_fwd_state(const void* q, const void* k, const void* v, const void* f_raw,
                                   const void* b_raw, const float* A_log, const float* dt_bias,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t d, uint32_t mode,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   const float* initial_state, float* final_state, void* stream) {
  return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, d,
                  mode, out, workspace, workspace_bytes, initial_state, final_state, nullptr, nullptr, 0,
                  stream, nullptr, 0);
}

extern "C" int kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* f_raw,
                                   const void* b_raw, const float* A_log, const float* dt_bias,
                                   const int32_t* cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t d, uint32_t mode,
                                   void* out, void* workspace, size_t workspace_bytes, void* stream,
                                   void* const* events, int32_t num_events) {
  if (!events) return KDA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, d,
                  mode, out, workspace, workspace_bytes, nullptr, nullptr, nullptr, nullptr, 0, stream,
                  events, num_events);
}

extern "C" int kda_chunk_fwd_rect(const void* q, const void* k, const void* v, const void* f_raw,
                                  const void* b_raw, const float* A_log, const float* dt_bias,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                  int32_t H, int32_t dk, int32_t dv, uint32_t mode, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  const float* initial_state, float* final_state, void* stream) {
  if (dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
  if (dk > kda::DH || dv > kda::DH) return KDA_ERR_UNSUPPORTED;
  const uint32_t m = (mode & ~KDA_MODE_ALL_BITS) ? mode : (mode & ~KDA_MODE_WINDOWED);
  if (dk == kda::DH && dv == kda::DH)
    return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H,
                    kda::DH, m, out, workspace, workspace_bytes, initial_state, final_state,
                    nullptr, nullptr, 0, stream, nullptr, 0);
  // the host checks of the square call (its workspace layout serves here)
  int st = check_args(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens,
                      H, kda::DH, m, out, workspace, workspace_bytes);
  if (st != KDA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (total_tokens == 0) {
    if (!final_state) return KDA_OK;
    const int64_t n = (int64_t)num_seqs * H * dk * dv;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(kda::kda_state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       initial_state, final_state, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  const bool f32i = m & KDA_MODE_FP32_INTERMEDIATE;
  const bool a32 = m & KDA_ACT_FP32;
  const bool o32 = (m & KDA_OUT_FP32) || a32;
#define KDA_RECT(TA, MT, TO)                                                                   \
  return kda::launch_all<TA, MT, TO, true>(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, \
                                           num_seqs, total_tokens, H, m, out, workspace,      \
                                           initial_state, final_state, nullptr, nullptr, 0, s, \
                                           nullptr, dk, dv)
  if (!a32 && !f32i && !o32) KDA_RECT(kda::bf16, kda::bf16, kda::bf16);
  if (!a32 && !f32i && o32) KDA_RECT(kda::bf16, kda::bf16, float);
  if (!a32 && f32i && !o32) KDA_RECT(kda::bf16, float, kda::bf16);
  if (!a32 && f32i && o32) KDA_RECT(kda::bf16, float, float);
  if (a32 && !f32i) KDA_RECT(float, kda::bf16, float);
  KDA_RECT(float, float, float);
#undef KDA_RECT
}

extern "C" int kda_chunk_fwd_conv(const void* q, const void* k, const void* v, const void* f_raw,
                                  const void* b_raw, const float* A_log, const float* dt_bias,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                  int32_t H, int32_t d, uint32_t mode, const float* conv_weight,
                                  const float* conv_bias, int32_t conv_silu, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  const float* initial_state, float* final_state, void* stream) {
  if (total_tokens > 0 && !conv_weight) return KDA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, d,
                  mode, out, workspace, workspace_bytes, initial_state, final_state, conv_weight,
                  conv_bias, conv_silu, stream, nullptr, 0);
}

template <int DK>
static void launch_recurrent(const kda::RecArgs& ra, bool a32, bool o32, hipStream_t s) {
  const int need = DK > ra.dv ? DK : ra.dv;
  const dim3 grid((unsigned)((int64_t)ra.N * ra.H)), block((unsigned)(64 * ((need + 63) / 64)));
  if (!a32 && !o32)
    hipLaunchKernelGGL((kda::kda_recurrent_kernel<kda::bf16, kda::bf16, DK>), grid, block, 0, s, ra);
  else if (!a32)
    hipLaunchKernelGGL((kda::kda_recurrent_kernel<kda::bf16, float, DK>), grid, block, 0, s, ra);
  else
    hipLaunchKernelGGL((kda::kda_recurrent_kernel<float, float, DK>), grid, block, 0, s, ra);
}

static int recurrent_impl(const void* q, const void* k, const void* v, const void* f_raw,
                          const void* b_raw, const float* A_log, const float* dt_bias,
                          const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          int32_t H, int32_t dk, int32_t dv, uint32_t mode, void* out,
                          const float* initial_state, float* final_state, void* stream) {
  if (mode & ~KDA_MODE_ALL_BITS) return KDA_ERR_INVALID_ARG;
  if (mode & KDA_MODE_CHECK_CU) return KDA_ERR_UNSUPPORTED;  // no workspace to report into
  if (num_seqs < 1 || total_tokens < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
  if ((dk != 16 && dk != 32 && dk != 64 && dk != 128) || dv > kda::rec_max_threads(dk))
    return KDA_ERR_UNSUPPORTED;
  // one workgroup of up to 512 threads per (sequence, head), one grid dimension
  if ((int64_t)num_seqs * H > (int64_t)INT32_MAX / 2 ||
      !kda::grid_fits((int64_t)num_seqs * H, 64 * (((dk > dv ? dk : dv) + 63) / 64)))
    return KDA_ERR_UNSUPPORTED;
  if (total_tokens == 0 && !final_state) return KDA_OK;
  if (total_tokens > 0 && (!q || !k || !v || !f_raw || !b_raw || !A_log || !dt_bias || !out ||
                           !cu_seqlens))
    return KDA_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (total_tokens == 0) {  // final = initial state (zero if none)
    const int64_t n = (int64_t)num_seqs * H * dk * dv;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(kda::kda_state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       initial_state, final_state, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  kda::RecArgs ra;
  ra.q = q; ra.k = k; ra.v = v; ra.f = f_raw; ra.b = b_raw; ra.A_log = A_log; ra.dt_bias = dt_bias;
  ra.cu = cu_seqlens; ra.init = initial_state; ra.fin = final_state; ra.out = out;
  ra.N = num_seqs; ra.H = H; ra.dv = dv; ra.eps = 1e-6f;
  ra.scale = 1.0f / sqrtf((float)dk);
  const bool a32 = mode & KDA_ACT_FP32;
  const bool o32 = (mode & KDA_OUT_FP32) || a32;
  switch (dk) {
    case 16: launch_recurrent<16>(ra, a32, o32, s); break;
    case 32: launch_recurrent<32>(ra, a32, o32, s); break;
    case 64: launch_recurrent<64>(ra, a32, o32, s); break;
    default: launch_recurrent<128>(ra, a32, o32, s); break;
  }
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" int kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* f_raw,
                                 const void* b_raw, const float* A_log, const float* dt_bias,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                 int32_t H, int32_t d, uint32_t mode, void* out,
                                 const float* initial_state, float* final_state, void* stream) {
  if (d != kda::DH) return d < 1 ? KDA_ERR_INVALID_ARG : KDA_ERR_UNSUPPORTED;
  return recurrent_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens,
                        H, d, d, mode, out, initial_state, final_state, stream);
}

extern "C" int kda_recurrent_fwd_rect(const void* q, const void* k, const void* v,
                                      const void* f_raw, const void* b_raw, const float* A_log,
                                      const float* dt_bias, const int32_t* cu_seqlens,
                                      int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t dk,
                                      int32_t dv, uint32_t mode, void* out,
                                      const float* initial_state, float* final_state,
                                      void* stream) {
  return recurrent_impl(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens,
                        H, dk, dv, mode, out, initial_state, final_state, stream);
}

extern "C" size_t kda_chunk_bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                                int32_t d, uint32_t mode) {
  if ((mode & ~KDA_MODE_ALL_BITS) || total_tokens < 0 || num_seqs < 1 || H < 1 || d != kda::DH)
    return (size_t)-1;
  if (total_tokens == 0) return 0;
  return kda::bwd_layout(total_tokens, num_seqs, H).total;
}

extern "C" int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* f_raw,
                             const void* b_raw, const float* A_log, const float* dt_bias,
                             const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                             int32_t H, int32_t d, uint32_t mode, const float* initial_state,
                             const void* dout, const float* dfinal_state, void* dq, void* dk,
                             void* dv, void* df_raw, void* db_raw, float* dA_log, float* ddt_bias,
                             float* dinitial_state, void* workspace, size_t workspace_bytes,
                             void* stream) {
  // every host-side check comes before the first HIP call
  if (mode & ~KDA_MODE_ALL_BITS) return KDA_ERR_INVALID_ARG;
  if (num_seqs < 1 || total_tokens < 0 || H < 1) return KDA_ERR_INVALID_ARG;
  if (d != kda::DH) return KDA_ERR_UNSUPPORTED;
  if (!dA_log || !ddt_bias) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0) {
    if (!q || !k || !v || !f_raw || !b_raw || !A_log || !dt_bias || !cu_seqlens || !dout || !dq ||
        !dk || !dv || !df_raw || !db_raw || !workspace)
      return KDA_ERR_INVALID_ARG;
    if (total_tokens > (int64_t)INT32_MAX / 64 || (int64_t)num_seqs * H > (int64_t)INT32_MAX / 64 ||
        !kda::bwd_heads_fit(H))
      return KDA_ERR_UNSUPPORTED;
    // grids: (chunks x up to 512 threads, H) per chunk; (32 x 512, N H / 8) scans
    if (!kda::grid_fits(kda::max_chunks(total_tokens, num_seqs), 512) ||
        !kda::grid_fits(((int64_t)num_seqs * H + 7) / 8, 1))
      return KDA_ERR_UNSUPPORTED;
    if (workspace_bytes < kda::bwd_layout(total_tokens, num_seqs, H).total)
      return KDA_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status reflects these launches
  if (total_tokens == 0) {
    const int64_t n = (int64_t)num_seqs * H * kda::DH * kda::DH;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(kda::kda_bwd_empty_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)),
                       dim3(256), 0, s, dfinal_state, dinitial_state, n, dA_log, ddt_bias, (int)H);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  const bool a32 = mode & KDA_ACT_FP32;
  const bool o32 = (mode & KDA_OUT_FP32) || a32;
#define KDA_BWD(TA, TG, TR)                                                                      \
  return kda::launch_bwd<TA, TG, TR>(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, \
                                     total_tokens, H, initial_state, dout, dfinal_state, dq, dk, \
                                     dv, df_raw, db_raw, dA_log, ddt_bias, dinitial_state,       \
                                     workspace, s, (mode & KDA_MODE_CHECK_CU) != 0)
  if (a32) KDA_BWD(float, float, float);
  if (o32) KDA_BWD(kda::bf16, float, float);
  KDA_BWD(kda::bf16, kda::bf16, kda::bf16);
#undef KDA_BWD
}

extern "C" size_t kda_chunk_bwd_conv_workspace_bytes(int64_t total_tokens, int32_t num_seqs,
                                                     int32_t H, int32_t d, uint32_t mode) {
  if ((mode & ~KDA_MODE_ALL_BITS) || total_tokens < 0 || num_seqs < 1 || H < 1 || d != kda::DH)
    return (size_t)-1;
  if (total_tokens == 0) return 0;
  return kda::conv_bwd_layout(total_tokens, num_seqs, H, mode).total;
}

extern "C" int kda_chunk_bwd_conv(const void* q, const void* k, const void* v, const void* f_raw,
                                  const void* b_raw, const float* A_log, const float* dt_bias,
                                  const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                  int32_t H, int32_t d, uint32_t mode, const float* conv_weight,
                                  const float* conv_bias, int32_t conv_silu,
                                  const float* initial_state, const void* dout,
                                  const float* dfinal_state, void* dq, void* dk, void* dv,
                                  void* df_raw, void* db_raw, float* dA_log, float* ddt_bias,
                                  float* dinitial_state, float* dconv_weight, float* dconv_bias,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  // every host-side check comes before the first HIP call
  if (mode & ~KDA_MODE_ALL_BITS) return KDA_ERR_INVALID_ARG;
  if (num_seqs < 1 || total_tokens < 0 || H < 1) return KDA_ERR_INVALID_ARG;
  if (d != kda::DH) return KDA_ERR_UNSUPPORTED;
  if (!dA_log || !ddt_bias || !dconv_weight) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0) {
    if (!q || !k || !v || !f_raw || !b_raw || !A_log || !dt_bias || !cu_seqlens || !dout || !dq ||
        !dk || !dv || !df_raw || !db_raw || !workspace || !conv_weight)
      return KDA_ERR_INVALID_ARG;
    if (total_tokens > (int64_t)INT32_MAX / 64 || (int64_t)num_seqs * H > (int64_t)INT32_MAX / 64 ||
        !kda::bwd_heads_fit(H))
      return KDA_ERR_UNSUPPORTED;
    if (!kda::grid_fits(kda::max_chunks(total_tokens, num_seqs), 512) ||
        !kda::grid_fits(((int64_t)num_seqs * H + 7) / 8, 1))
      return KDA_ERR_UNSUPPORTED;
    if (workspace_bytes < kda::conv_bwd_layout(total_tokens, num_seqs, H, mode).total)
      return KDA_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (total_tokens == 0) {
    // the core's empty case (dA_log, ddt_bias zeroed, dinitial_state = dfinal_state or 0)
    // and zero tap / bias gradients
    const int st = kda_chunk_bwd(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, 0, H,
                                 d, mode, initial_state, dout, dfinal_state, dq, dk, dv, df_raw,
                                 db_raw, dA_log, ddt_bias, dinitial_state, workspace,
                                 workspace_bytes, stream);
    if (st != KDA_OK) return st;
    hipLaunchKernelGGL(kda::kda_state_copy_kernel, dim3(64), dim3(256), 0, s, (const float*)nullptr,
                       dconv_weight, (int64_t)3 * H * kda::DH * 4);
    if (dconv_bias)
      hipLaunchKernelGGL(kda::kda_state_copy_kernel, dim3(16), dim3(256), 0, s,
                         (const float*)nullptr, dconv_bias, (int64_t)3 * H * kda::DH);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  const bool a32 = mode & KDA_ACT_FP32;
  const bool o32 = (mode & KDA_OUT_FP32) || a32;
#define KDA_BWDC(TA, TG, TR)                                                                   \
  return kda::launch_bwd_conv<TA, TG, TR>(                                                    \
      q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, num_seqs, total_tokens, H, mode,      \
      conv_weight, conv_bias, conv_silu, initial_state, dout, dfinal_state, dq, dk, dv, df_raw, \
      db_raw, dA_log, ddt_bias, dinitial_state, dconv_weight, dconv_bias, workspace, s)
  if (a32) KDA_BWDC(float, float, float);
  if (o32) KDA_BWDC(kda::bf16, float, float);
  KDA_BWDC(kda::bf16, kda::bf16, kda::bf16);
#undef KDA_BWDC
}

extern "C" const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: return "unknown";
  }
}
