/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) Kimi Delta Attention (KDA)
 * chunked forward, its token-serial form and its backward.
 *
 * Operation (per head h and per packed sequence; zero initial state except
 * in kda_chunk_fwd_state):
 *   q^_t   = q_t / sqrt(|q_t|^2 + 1e-6),   k^_t likewise       (FP32 math)
 *   g_t[c] = -exp(A_log[h]) * softplus(f_raw_t[c] + dt_bias[h][c])
 *   beta_t = sigmoid(b_raw_t)
 *   S_t    = Diag(exp(g_t)) S_{t-1};  S_t += beta_t k^_t (v_t - S_t^T k^_t)^T
 *   out_t  = S_t^T q^_t / sqrt(d)
 * computed in 64-token chunks (intra-chunk decay-weighted blocks, a
 * unit-lower-triangular chunk solve, a chunk-to-chunk state pass, and an
 * output combine).
 *
 * What the pages fix: the operator is the chunked KDA forward of xtuner PR
 * #2153 "GLM-5.3-Flash F6.2: KDA correctness and FLA sequence parallelism"
 * (KDA module section: gate computed outside the kernel from FP32 A_log and
 * dt_bias, sigmoid beta, packed multi-document inputs, a fixed-layout FP32
 * gate prefix); its two precision modes and the packed-offset interface come
 * from xtuner PR #2301 "[Enhancement] Add opt-in FP32 KDA chunk computation"
 * (section Change: promote Q/K/V before the L2 norm, keep normalised vectors
 * and chunk solve / state intermediates in FP32, cast only the visible output
 * back; no initial/final state).  The 64-head x 128-dim geometry is the one
 * both pages measure.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device memory owned by the caller; the
 *    library never frees or retains them.  All arrays are row-major,
 *    contiguous and at least 16-byte aligned.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the default stream).  The library performs no device allocation, no
 *    host<->device copy and no synchronisation inside a call, so a call can
 *    be captured into a HIP graph.
 *  - Host-side argument errors are reported before anything is launched.
 *  - Status codes are the KDA_* values below; kda_status_string() names them.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

/* Status codes. */
#define KDA_OK 0
#define KDA_ERR_INVALID_ARG 1 /* null pointer, H < 1, num_seqs < 1, T < 0, unknown mode bit */
#define KDA_ERR_UNSUPPORTED 2 /* d != 128 (the only head dimension built)                 */
#define KDA_ERR_WORKSPACE 3   /* workspace_bytes smaller than kda_chunk_fwd_workspace_bytes */
#define KDA_ERR_HIP 4         /* a kernel launch failed (hipGetLastError)                 */

/* Mode bits (bitwise OR).  Unknown bits are rejected.
 * KDA_MODE_FP32_INTERMEDIATE: 0 = BF16 intermediates (normalised q/k, the
 *   chunk-solve outputs W/U, the output-combine matrices and the state
 *   snapshots used as matrix operands are bfloat16, accumulation is FP32);
 *   1 = every intermediate stored in FP32 and every matrix product
 *   FP32-accurate (xtuner PR #2301, section Change): FP32 matrix cores in
 *   the intra-chunk kernel; in the state pass bf16 matrix cores on a
 *   three-piece bf16 split of each FP32 operand, six piece products per
 *   product, FP32 accumulation (omitted terms below 2^-23 of the product).
 *   In both modes the gate, its chunk prefix, the forward substitution and
 *   the running state are FP32.
 * KDA_ACT_FP32: activation dtype of q, k, v, f_raw, b_raw: 0 = bfloat16,
 *   1 = float32.
 * KDA_OUT_FP32: dtype of out: 0 = the activation dtype, 1 = float32.
 * KDA_MODE_WINDOWED: schedule only, same arithmetic.  By default the
 *   forward makes two passes (intra-chunk kernel, then state pass): with FP32
 *   intermediates over all chunks at once, with a record per chunk and head in
 *   the workspace; with BF16 intermediates over segments of 32 chunks (per
 *   segment one intra-chunk launch and one state-pass launch, the records in a
 *   ring of one segment: 160 MB at 64 heads, whatever the length; the results
 *   are bit for bit those of one pass over all chunks).  With this bit, BF16
 *   intermediates and at most 64 sequences the forward runs as a pipeline of
 *   windows of 24 chunks instead: each launch does the intra-chunk work of one
 *   window and the state pass over the window before, the records in a ring of
 *   two windows (230 MB at 64 heads).  Slower than the default segments; kept
 *   as the alternative schedule it measures against.  Ignored with FP32
 *   intermediates or more than 64 sequences.
 * KDA_MODE_CHECK_CU: debugging aid.  The device checks cu_seqlens before any
 *   kernel reads token data: cu_seqlens[0] == 0, non-decreasing,
 *   cu_seqlens[num_seqs] == total_tokens.  It stores a code in the first 4
 *   bytes of the workspace (int32, readable once the call has completed):
 *   0 when valid, else bit 0 (cu_seqlens[0] != 0) | bit 1 (a decrease) |
 *   bit 2 (last offset != total_tokens).  When the code is not 0 every
 *   sequence is treated as empty: no token data is read or written (out and
 *   the input gradients are left as they were), end states are the start
 *   states (zero without), the parameter gradients are zero and the start-state
 *   gradient is the end-state gradient.  Cost: one small launch.  Taken by the chunked forward entry points
 *   and the backward ones when total_tokens > 0 (with total_tokens == 0
 *   nothing is launched and no code is written); kda_chunk_fwd_noalloc and the
 *   token-serial entry points, which have no workspace to report into, return
 *   KDA_ERR_UNSUPPORTED for it.  Without the bit the offsets are a
 *   precondition and are not checked. */
#define KDA_MODE_FP32_INTERMEDIATE 0x1u
#define KDA_ACT_FP32 0x2u
#define KDA_OUT_FP32 0x4u
#define KDA_MODE_WINDOWED 0x8u
#define KDA_MODE_CHECK_CU 0x10u
#define KDA_MODE_ALL_BITS 0x1Fu

/* Bytes of caller-provided scratch that kda_chunk_fwd needs for this shape.
 * Depends only on the arguments; non-decreasing in total_tokens.  FP32
 * intermediates need about 144 KB per 64-token chunk and head.  BF16
 * intermediates need about 72 KB per chunk and head up to 32 chunks and stop
 * growing there: about 2.4 MB per head (the records of one 32-chunk segment and
 * two 64 KB boundary states).  The windowed schedule (KDA_MODE_WINDOWED with
 * BF16 intermediates and at most 64 sequences) stops growing at 48 chunks:
 * about 3.6 MB per head (two 24-chunk windows).  Returns 0 when total_tokens == 0, and
 * (size_t)-1 when the arguments are invalid (negative sizes, d != 128,
 * unknown mode bits). */
KDA_API size_t kda_chunk_fwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t d,
                                     uint32_t mode);

/* KDA chunked forward over a packed batch.
 *  q, k, v, f_raw : device, [total_tokens][H][d], activation dtype
 *  b_raw          : device, [total_tokens][H], activation dtype (beta logits)
 *  A_log          : device, [H], float32
 *  dt_bias        : device, [H][d], float32
 *  cu_seqlens     : device, [num_seqs + 1], int32; sequence n covers tokens
 *                   [cu_seqlens[n], cu_seqlens[n+1]).  Preconditions (not
 *                   checked, since checking would need a device read):
 *                   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[num_seqs] =
 *                   total_tokens.  Empty sequences are allowed.  The state is
 *                   zero at every sequence start and never crosses a
 *                   boundary; no final state is returned.
 *  num_seqs >= 1, total_tokens >= 0, H >= 1, d == 128.
 *  out            : device, [total_tokens][H][d], dtype per KDA_OUT_FP32;
 *                   every element is written.  Must not alias any input.
 *  workspace      : device scratch of workspace_bytes >= the query above,
 *                   256-byte aligned; contents on entry are ignored.
 * total_tokens == 0 returns KDA_OK without launching anything (out and the
 * inputs may then be NULL).  Two host threads may call concurrently only with
 * distinct workspaces. */
KDA_API int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* f_raw,
                  const void* b_raw, const float* A_log, const float* dt_bias,
                  const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t H,
                  int32_t d, uint32_t mode, void* out, void* workspace, size_t workspace_bytes,
                  void* stream);

/* kda_chunk_fwd with a start state and an end state per sequence and head.
 * The pages' wrapper takes neither (xtuner PR #2301, section Change: no start
 * or end state is added); the sequence-parallel design of xtuner PR #2153
 * (contiguous shards exchanging recurrent boundary states) is what needs
 * them: a sequence run in two calls, the second starting from the first
 * call's final state, gives the outputs of one call over the whole sequence.
 *  initial_state : device, [num_seqs][H][d][d] float32, or NULL (zero start).
 *                  Entry [n][h][i][j] is S[key i][value j] of sequence n,
 *                  head h before its first token (out_t = S_t^T q^_t).
 *  final_state   : device, [num_seqs][H][d][d] float32, or NULL (not written).
 *                  Receives S after each sequence's last token; for an empty
 *                  sequence it is the initial state (zero if NULL).  It may be
 *                  the same array as initial_state (updated in place), and
 *                  must not overlap any other argument.
 * Everything else as for kda_chunk_fwd; with total_tokens == 0 and a
 * final_state, final_state is still written (one small launch).  The running
 * state is FP32 in both precision modes. */
KDA_API int kda_chunk_fwd_state(const void* q, const void* k, const void* v, const void* f_raw,
                        const void* b_raw, const float* A_log, const float* dt_bias,
                        const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        int32_t H, int32_t d, uint32_t mode, void* out, void* workspace,
                        size_t workspace_bytes, const float* initial_state, float* final_state,
                        void* stream);

/* kda_chunk_fwd_state with the short causal convolution in front of the core
 * fused in: q, k and v each pass through their own depthwise causal
 * convolution of width 4 (xtuner PR #2153, KDA module description: separate
 * q/k/v causal convolutions; FP32 master parameters, forward in the
 * activation dtype), optionally followed by SiLU:
 *   x'_t[c] = act(bias[c] + sum_{i<4} w[c][i] x_{t-3+i}[c]),
 * with zero history at every sequence start (no history input: a sequence
 * split across calls needs its first 3 tokens' history, which this entry
 * point does not take).
 *  conv_weight : device, [3][H][d][4] float32 (tensor q, k, v; tap 3 is the
 *                current token); required when total_tokens > 0.
 *  conv_bias   : device, [3][H][d] float32, or NULL (no bias).
 *  conv_silu   : nonzero applies SiLU (x * sigmoid(x)) after the convolution.
 * Weights and bias are rounded to the activation dtype, products accumulate
 * in FP32 and the convolution output is rounded to the activation dtype
 * before the KDA core (L2 norm, gate, ...), as a separate convolution op in
 * that dtype would do.  Everything else as for kda_chunk_fwd_state. */
KDA_API int kda_chunk_fwd_conv(const void* q, const void* k, const void* v, const void* f_raw,
                       const void* b_raw, const float* A_log, const float* dt_bias,
                       const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t H, int32_t d, uint32_t mode, const float* conv_weight,
                       const float* conv_bias, int32_t conv_silu, void* out, void* workspace,
                       size_t workspace_bytes, const float* initial_state, float* final_state,
                       void* stream);

/* kda_chunk_fwd_state with a rectangular state: dk key channels (q, k, f_raw
 * [T][H][dk], dt_bias [H][dk]) and dv value channels (v, out [T][H][dv]),
 * 1 <= dk, dv <= 128 (larger: KDA_ERR_UNSUPPORTED); states [num_seqs][H][dk]
 * [dv] (NULL allowed, as for kda_chunk_fwd_state); the output scale is
 * 1/sqrt(dk).  The pages record the rectangular case dk = 16, dv = 24 failing
 * to compile in their TileLang chunk kernels (xtuner PR #2301, section
 * Validation).  Here the chunked kernels run on the 128 x 128 layout with the
 * missing key and value channels read as zero (they stay zero in every
 * intermediate and in the state), and only the dk x dv part is written: the
 * cost is that of a 128 x 128 call, less the value blocks of 32 channels
 * that lie wholly past dv.  Workspace: kda_chunk_fwd_workspace_bytes(T,
 * num_seqs, H, 128, mode); KDA_MODE_WINDOWED is ignored (two passes).
 * Everything else as for kda_chunk_fwd_state; dk = dv = 128 is that call. */
KDA_API int kda_chunk_fwd_rect(const void* q, const void* k, const void* v, const void* f_raw,
                       const void* b_raw, const float* A_log, const float* dt_bias,
                       const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t H, int32_t dk, int32_t dv, uint32_t mode, void* out,
                       void* workspace, size_t workspace_bytes, const float* initial_state,
                       float* final_state, void* stream);

/* Token-serial KDA forward: the same operator as kda_chunk_fwd_state, taken
 * one token at a time with the state in FP32 (the serving-side FP32
 * recurrence that xtuner PR #2301 validates its chunked path against,
 * sections Problem and Validation).  Meant for decode steps and short
 * sequences (work per token is sequential); long prefills belong to the
 * chunked path.  Arguments as for kda_chunk_fwd_state, except:
 *  - no workspace;
 *  - mode: KDA_ACT_FP32 and KDA_OUT_FP32 as usual; KDA_MODE_FP32_INTERMEDIATE
 *    is accepted and changes nothing (all intermediates are FP32);
 *  - with total_tokens == 0 and a final_state, final_state receives the
 *    initial state (zero if NULL) and no other pointer is read;
 *  - initial_state / final_state ([num_seqs][H][d][d] float32, NULL
 *    allowed) may be the same array: each state entry is read before the
 *    first token and written after the last by the same thread.
 * Returns KDA_OK without launching when total_tokens == 0 and final_state is
 * NULL. */
KDA_API int kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* f_raw,
                      const void* b_raw, const float* A_log, const float* dt_bias,
                      const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      int32_t H, int32_t d, uint32_t mode, void* out,
                      const float* initial_state, float* final_state, void* stream);

/* kda_recurrent_fwd with a rectangular state: dk key channels (q, k, f_raw
 * [T][H][dk], dt_bias [H][dk]) and dv value channels (v, out [T][H][dv]);
 * states [num_seqs][H][dk][dv]; the output scale is 1/sqrt(dk).  Supported:
 * dk in {16, 32, 64, 128} (else KDA_ERR_UNSUPPORTED), 1 <= dv <= 512 for
 * dk <= 64 and dv <= 128 for dk = 128 (larger: KDA_ERR_UNSUPPORTED).  The pages record the rectangular case dk = 16,
 * dv = 24 failing to compile in their TileLang kernels (xtuner PR #2301,
 * section Validation); here it runs on the token-serial path.  Everything
 * else as for kda_recurrent_fwd. */
KDA_API int kda_recurrent_fwd_rect(const void* q, const void* k, const void* v, const void* f_raw,
                           const void* b_raw, const float* A_log, const float* dt_bias,
                           const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                           int32_t H, int32_t dk, int32_t dv, uint32_t mode, void* out,
                           const float* initial_state, float* final_state, void* stream);

/* Workspace bytes needed by kda_chunk_bwd (same arguments and failure value
 * as kda_chunk_fwd_workspace_bytes).  FP32 throughout: about 460 KB per
 * (64-token chunk, head), e.g. 7.5 GB for 16384 tokens x 64 heads. */
KDA_API size_t kda_chunk_bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                     int32_t d, uint32_t mode);

/* Backward (vector-Jacobian product) of kda_chunk_fwd_state, recomputed in
 * FP32: the pages' training path recomputes the backward in FP32 and
 * casts the input gradients back to the activation dtype (xtuner PR #2301,
 * section Change), checks the gradients of q, k, v, the gate and beta against
 * an FP64 recurrence VJP (same PR, section Validation), and sums the dt_bias
 * gradient in FP32 (xtuner PR #2153, KDA module section).
 * For L = <dout, out> + <dfinal_state, final_state> of the forward with the
 * same inputs, writes
 *   dq, dk, dv, df_raw [T][H][d], db_raw [T][H]: dL/d(input), in dout's dtype;
 *   dA_log [H], ddt_bias [H][d]: float32 (overwritten, not accumulated);
 *   dinitial_state [num_seqs][H][d][d] float32 (NULL: not returned): dL/dS_0,
 *   also when initial_state is NULL (the forward then started from zero).
 * Arguments as for kda_chunk_fwd_state, plus:
 *  - dout [T][H][d]: float32 when mode has KDA_OUT_FP32 or KDA_ACT_FP32 (then
 *    the gradients are float32 too), else bfloat16 (gradients bfloat16);
 *  - dfinal_state: NULL means zero;
 *  - KDA_MODE_FP32_INTERMEDIATE is accepted and changes nothing (every
 *    intermediate of the backward is FP32, whatever the forward used);
 *  - workspace of kda_chunk_bwd_workspace_bytes bytes, caller-owned, 256-byte
 *    aligned; its contents on return are unspecified.
 * total_tokens == 0: only dA_log, ddt_bias (zeroed) and dinitial_state
 * (= dfinal_state, or zero) are written; the other pointers are not read.
 * No output may alias an input.  Asynchronous on `stream`, no allocation, no
 * host synchronisation.  Errors as for kda_chunk_fwd (dA_log and ddt_bias
 * are required); besides, H > 262143 gives KDA_ERR_UNSUPPORTED (the kernels
 * address a chunk's 64 rows of an activation with 32-bit offsets). */
KDA_API int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* f_raw,
                  const void* b_raw, const float* A_log, const float* dt_bias,
                  const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, int32_t H,
                  int32_t d, uint32_t mode, const float* initial_state, const void* dout,
                  const float* dfinal_state, void* dq, void* dk, void* dv, void* df_raw,
                  void* db_raw, float* dA_log, float* ddt_bias, float* dinitial_state,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by kda_chunk_bwd_conv (same arguments and failure
 * value as kda_chunk_fwd_workspace_bytes; the mode decides the activation
 * dtype of the stored convolution outputs).  kda_chunk_bwd's workspace plus
 * the three convolution outputs, their FP32 gradients, FP32 gradients of
 * f_raw and b_raw and per-chunk tap partial sums: about 650 KB per (64-token
 * chunk, head) with bf16 activations, e.g. 10.7 GB for 16384 tokens x 64
 * heads. */
KDA_API size_t kda_chunk_bwd_conv_workspace_bytes(int64_t total_tokens, int32_t num_seqs,
                                          int32_t H, int32_t d, uint32_t mode);

/* Backward of kda_chunk_fwd_conv: kda_chunk_bwd through the core, then
 * through the q/k/v short causal convolutions, whose weight and bias
 * gradients are FP32 (xtuner PR #2153, KDA module description: separate
 * q/k/v causal convolutions with FP32 master parameters).  With z the
 * pre-activation of x'_t = act(z_t) and dz_t = dL/dx'_t * act'(z_t):
 *   dx_u = sum_{i<4} w[i] dz_{u+3-i}   (tokens of u's own sequence),
 *   dw[i] = sum_t dz_t x_{t-3+i},  dbias = sum_t dz_t   (over all sequences).
 * The forward rounds x' to the activation dtype; the backward recomputes x'
 * the same way for the core's backward and takes that rounding as the
 * identity (its derivative is 1).  Arguments as for kda_chunk_bwd (q, k, v
 * are the convolution's raw inputs, dq, dk, dv the gradients with respect to
 * them), plus those of kda_chunk_fwd_conv and:
 *  dconv_weight : device, [3][H][d][4] float32, required; overwritten.
 *  dconv_bias   : device, [3][H][d] float32, or NULL (not written).
 * The tap and bias sums are reduced in a fixed order (deterministic).
 * total_tokens == 0: as kda_chunk_bwd, and dconv_weight (dconv_bias when
 * given) is zeroed.  Workspace of kda_chunk_bwd_conv_workspace_bytes bytes;
 * errors, aliasing and asynchrony as for kda_chunk_bwd. */
KDA_API int kda_chunk_bwd_conv(const void* q, const void* k, const void* v, const void* f_raw,
                       const void* b_raw, const float* A_log, const float* dt_bias,
                       const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       int32_t H, int32_t d, uint32_t mode, const float* conv_weight,
                       const float* conv_bias, int32_t conv_silu, const float* initial_state,
                       const void* dout, const float* dfinal_state, void* dq, void* dk, void* dv,
                       void* df_raw, void* db_raw, float* dA_log, float* ddt_bias,
                       float* dinitial_state, float* dconv_weight, float* dconv_bias,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device array that kda_chunk_fwd_noalloc uses as its workspace
 * (256 MiB, on every GPU the library runs on, held until the process ends). */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)

/* kda_chunk_fwd without a workspace argument and without any allocation:
 * for callers that cannot allocate device memory (code being captured into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a library-owned device array of KDA_NOALLOC_SCRATCH_BYTES per
 * GPU; shapes whose kda_chunk_fwd_workspace_bytes exceeds it return
 * KDA_ERR_WORKSPACE before anything is launched.  With BF16 intermediates
 * that is any length up to 107 heads (74 with KDA_MODE_WINDOWED); with FP32
 * intermediates up to 28 chunks of 64 tokens at 64 heads.  Every
 * byte of the array that a call reads it has written earlier in the same
 * call, so nothing needs clearing between calls.  Calls that overlap in time
 * on one GPU (two streams, two host threads) share the one array and race:
 * serialise them.  The first call on a device looks the array's address up
 * once (hipGetSymbolAddress); no call allocates or frees memory.
 * Arguments, results and errors otherwise as for kda_chunk_fwd. */
KDA_API int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* f_raw,
                          const void* b_raw, const float* A_log, const float* dt_bias,
                          const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          int32_t H, int32_t d, uint32_t mode, void* out, void* stream);

/* Number of stages kda_chunk_fwd_timed separates for this shape and mode:
 * 1 + 2 s for two passes in s segments (the chunk table, then for each
 * segment its intra-chunk launch and its state-pass launch; s = 1 with FP32
 * intermediates or up to 32 chunks, else ceil(chunks / 32) with chunks the
 * workspace query's upper bound), 2 for the windowed schedule (chunk table,
 * all window launches); -1 for invalid arguments.  The chunk table is
 * launched only when num_seqs > 1 or the cu_seqlens check is asked for (the
 * stage is otherwise empty). */
KDA_API int kda_chunk_fwd_num_stages(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                     uint32_t mode);

/* Same as kda_chunk_fwd, and additionally records events[i] (hipEvent_t,
 * created by the caller) on `stream` before stage i and events[n] after the
 * last stage, n = kda_chunk_fwd_num_stages(total_tokens, num_seqs, H, mode);
 * num_events must be n + 1.
 * Used by the benchmark to time each kernel on the stream it runs on. */
KDA_API int kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* f_raw,
                        const void* b_raw, const float* A_log, const float* dt_bias,
                        const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        int32_t H, int32_t d, uint32_t mode, void* out, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* events,
                        int32_t num_events);

/* Static, NUL-terminated name of a status code ("KDA_OK", ...; "unknown"
 * for other values). */
KDA_API const char* kda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
