/*
 * kda_oracle.c -- CPU reference ("oracle") for the Kimi Delta Attention (KDA)
 * chunked forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct FP64
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * What is computed (per head h, per packed sequence; the state starts at zero,
 * or at a caller-given initial state):
 *
 *   q^_t = q_t / sqrt(|q_t|^2 + eps),  k^_t = k_t / sqrt(|k_t|^2 + eps)
 *   g_t[c] = -exp(A_log[h]) * softplus(f_t[c] + dt_bias[h][c])
 *   beta_t = sigmoid(b_t)
 *   S_t  = Diag(exp(g_t)) S_{t-1}                  (d_k x d_v state)
 *   S_t += beta_t k^_t (v_t - S_t^T k^_t)^T        (delta rule on the decayed S)
 *   o_t  = scale * S_t^T q^_t                      (includes token t's own write)
 *
 * Sources.  The pages name KDA's chunked operator and its serving-side FP32
 * token recurrence, packed variable-length inputs with per-document state
 * isolation, FP32 A_log / dt_bias feeding a separately computed gate, a sigmoid
 * beta, and q/k L2 normalisation done in FP32 (q, k, v raised to FP32 first):
 *   - xtuner PR #2301 "[Enhancement] Add opt-in FP32 KDA chunk computation",
 *     sections Problem, Change and Validation (an FP64 recurrence written
 *     independently of the kernels is the reference there);
 *   - xtuner PR #2153 "GLM-5.3-Flash F6.2: KDA correctness and FLA sequence
 *     parallelism", KDA module description (fused_kda_gate outside the kernel,
 *     use_beta_sigmoid_in_kernel, packed multi-document isolation).
 * The pages do not print the equations; the recurrence above is the standard
 * KDA / gated delta rule with per-channel (diagonal) decay.  Readings where the
 * pages are silent: eps = 1e-6 is a parameter (tests also use 0); the output
 * scale multiplies the read-out; softplus uses the exact stable form
 * max(x,0) + log1p(exp(-|x|)) with no linear cut-over.
 *
 * Layouts (row-major, contiguous): q,k,v,f [T][H][d]; b [T][H]; A_log [H];
 * dt_bias [H][d]; cu_seqlens [N+1] with cu[0]=0, cu[N]=T, non-decreasing.
 *
 * Initial / final state (optional, NULL = absent): S_init and S_final are
 * [N][H][d_k][d_v], the state of sequence n, head h before its first token
 * and after its last (for an empty sequence the final state is the initial
 * one).  The wrapper on the pages leaves them out (PR #2301, section Change);
 * PR #2153 (FLA sequence parallelism: contiguous shards that exchange their
 * recurrent boundary states) is the use that needs them: running a sequence
 * in two pieces, the second starting from the first one's final state, must
 * give the same outputs as running it whole.
 *
 * kda_oracle_chunked() is a second, independent FP64 implementation in chunk
 * form (intra-chunk decay-weighted blocks, unit-lower-triangular solve by
 * forward substitution, chunk-to-chunk state pass).  It exists to localise
 * disagreements stage by stage and is itself pinned to the token recurrence by
 * the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Deliberate-mistake switches.  They exist only so the tests can show that
 * each plausible mistake is caught by at least one pin; 0 means "no mistake".
 */
enum {
  PLANT_NO_DECAY = 1u << 0,          /* skip S <- Diag(exp g) S                 */
  PLANT_DELTA_UNDECAYED = 1u << 1,   /* delta reads S_{t-1} instead of decayed S */
  PLANT_READ_BEFORE_WRITE = 1u << 2, /* o_t read before token t's write         */
  PLANT_TRANSPOSED_READ = 1u << 3,   /* o = S q instead of S^T q                */
  PLANT_DELTA_SIGN = 1u << 4,        /* v + S^T k instead of v - S^T k          */
  PLANT_NO_BETA = 1u << 5,           /* beta forced to 1                        */
  PLANT_NO_RESET = 1u << 6,          /* state carried across sequences          */
  PLANT_NO_L2NORM = 1u << 7,         /* q, k used un-normalised                 */
  PLANT_NO_SOFTPLUS = 1u << 8,       /* g = -exp(A_log) * x                     */
  PLANT_GATE_SIGN = 1u << 9,         /* decay by exp(-g)                        */
  PLANT_NO_SCALE = 1u << 10,         /* output scale dropped                    */
  PLANT_OUTER_SWAP = 1u << 11,       /* write (v - S^T k) k^T, operands swapped */
  PLANT_DROP_CARRY_64 = 1u << 12,    /* state reset every 64 tokens             */
  PLANT_INIT_TRANSPOSED = 1u << 13,  /* initial state read as S_init^T          */
  PLANT_FINAL_EARLY = 1u << 14,      /* final state taken before the last token */
  PLANT_CONV_NO_RESET = 1u << 15,    /* convolution history crosses sequences   */
  PLANT_CONV_TAPS_REVERSED = 1u << 16, /* taps applied in reverse order          */
  PLANT_CONVB_NO_SILU_DERIV = 1u << 21, /* backward: SiLU derivative taken as 1     */
  PLANT_CONVB_TAPS_FORWARD = 1u << 22,  /* backward: dx correlates the taps forward */
  /* mistakes of the backward (kda_oracle_bwd_rect) */
  PLANT_BWD_BETA_SCALE = 1u << 17,   /* beta gradient scaled by 1.25            */
  PLANT_BWD_NO_STATE_DECAY = 1u << 18, /* dS passed back without Diag(exp g)    */
  PLANT_BWD_NO_NORM_PROJ = 1u << 19, /* dq = dq^ / |q|, radial term dropped      */
  PLANT_BWD_GATE_NO_SIGMOID = 1u << 20 /* softplus' taken as 1                   */
};

static double softplus(double x) {
  /* softplus(x) = log(1 + e^x), in the overflow-free form. */
  return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

static double sigmoid(double x) {
  if (x >= 0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/* L2-normalise one d-vector: y = x / sqrt(sum x^2 + eps). */
static void l2norm(const double* x, int d, double eps, double* y) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) ss += x[c] * x[c];
  double r = 1.0 / sqrt(ss + eps);
  for (int c = 0; c < d; ++c) y[c] = x[c] * r;
}

/* Per-channel log-decay of one token-head: g[c] = -exp(A_log) softplus(f + dt_bias). */
static void gate(const double* f, double A_log, const double* dtb, int d, unsigned plant,
                 double* g) {
  double lam = exp(A_log);
  for (int c = 0; c < d; ++c) {
    double x = f[c] + dtb[c];
    double sp = (plant & PLANT_NO_SOFTPLUS) ? x : softplus(x);
    /* lam == 0 (A_log = -inf) must give g = 0 exactly, whatever sp is. */
    g[c] = (lam == 0.0) ? 0.0 : -lam * sp;
  }
}

/* Stage 1 alone: normalised q, k, the log-decay g and beta for every token-head. */
void kda_oracle_prep(const double* q, const double* k, const double* f, const double* b,
                     const double* A_log, const double* dt_bias, int64_t T, int H, int d,
                     double eps, double* qn, double* kn, double* g, double* beta) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      int64_t o = (t * H + h) * (int64_t)d;
      l2norm(q + o, d, eps, qn + o);
      l2norm(k + o, d, eps, kn + o);
      gate(f + o, A_log[h], dt_bias + (int64_t)h * d, d, 0u, g + o);
      beta[t * H + h] = sigmoid(b[t * H + h]);
    }
  }
}

/* Start state of sequence n, head h (dk x dv): S_init's block, or zero.  The
 * transposed plant reads a square block transposed. */
static void load_init_rect(double* S, const double* S_init, int n, int H, int h, int dk, int dv,
                           unsigned plant) {
  const size_t dd = (size_t)dk * dv;
  if (!S_init) { memset(S, 0, sizeof(double) * dd); return; }
  const double* src = S_init + ((size_t)n * H + h) * dd;
  if ((plant & PLANT_INIT_TRANSPOSED) && dk == dv) {
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = src[(size_t)j * dv + i];
  } else {
    memcpy(S, src, sizeof(double) * dd);
  }
}
static void load_init(double* S, const double* S_init, int n, int H, int h, int d,
                      unsigned plant) {
  load_init_rect(S, S_init, n, H, h, d, d, plant);
}

/* Token-serial recurrence for heads [h_lo, h_hi).  out is [T][H][d]; rows of
 * heads outside the range are left untouched.  S_init / S_final: see the
 * header (NULL = zero start / not returned; only the blocks of heads in range
 * are read or written).  Returns 0, or -1 on bad args. */
int kda_oracle_fwd_rect(const double* q, const double* k, const double* v, const double* f,
                        const double* b, const double* A_log, const double* dt_bias,
                        const int32_t* cu_seqlens, int N, int64_t T, int H, int dk, int dv,
                        int h_lo, int h_hi, double scale, double eps, unsigned plant,
                        const double* S_init, double* S_final, double* out);

int kda_oracle_fwd(const double* q, const double* k, const double* v, const double* f,
                   const double* b, const double* A_log, const double* dt_bias,
                   const int32_t* cu_seqlens, int N, int64_t T, int H, int d, int h_lo,
                   int h_hi, double scale, double eps, unsigned plant, const double* S_init,
                   double* S_final, double* out) {
  return kda_oracle_fwd_rect(q, k, v, f, b, A_log, dt_bias, cu_seqlens, N, T, H, d, d, h_lo, h_hi,
                             scale, eps, plant, S_init, S_final, out);
}

/* The same with a rectangular state: q, k, f, dt_bias have dk channels, v
 * and out dv channels, S and the states are dk x dv. */
int kda_oracle_fwd_rect(const double* q, const double* k, const double* v, const double* f,
                        const double* b, const double* A_log, const double* dt_bias,
                        const int32_t* cu_seqlens, int N, int64_t T, int H, int dk, int dv,
                        int h_lo, int h_hi, double scale, double eps, unsigned plant,
                        const double* S_init, double* S_final, double* out) {
  if (N < 1 || H < 1 || dk < 1 || dv < 1 || h_lo < 0 || h_hi > H || h_lo > h_hi) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int nh = h_hi - h_lo;
  /* With PLANT_NO_RESET the sequences of one head are walked in order with one
   * state, so the parallel unit is the head; otherwise it is (sequence, head). */
  const int64_t units = (plant & PLANT_NO_RESET) ? (int64_t)nh : (int64_t)N * nh;
  const size_t sz = (size_t)dk * dv;
  const int square = dk == dv; /* the transposing plants only exist for square states */

#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * sz);
    double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* g = (double*)malloc(sizeof(double) * (size_t)dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* Sprev = (plant & PLANT_DELTA_UNDECAYED) ? (double*)malloc(sizeof(double) * sz) : NULL;
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < units; ++w) {
      int h, n_lo, n_hi;
      if (plant & PLANT_NO_RESET) {
        h = h_lo + (int)w; n_lo = 0; n_hi = N;
      } else {
        h = h_lo + (int)(w % nh); n_lo = (int)(w / nh); n_hi = n_lo + 1;
      }
      load_init_rect(S, S_init, n_lo, H, h, dk, dv, plant);
      for (int n = n_lo; n < n_hi; ++n) {
        if (!(plant & PLANT_NO_RESET)) load_init_rect(S, S_init, n, H, h, dk, dv, plant);
        double* fin = S_final ? S_final + ((size_t)n * H + h) * sz : NULL;
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
          if (fin && (plant & PLANT_FINAL_EARLY) && t == cu_seqlens[n + 1] - 1)
            memcpy(fin, S, sizeof(double) * sz);
          if ((plant & PLANT_DROP_CARRY_64) && ((t - cu_seqlens[n]) % 64) == 0)
            memset(S, 0, sizeof(double) * sz);
          const int64_t ok_ = (t * H + h) * (int64_t)dk; /* q, k, f rows */
          const int64_t ov = (t * H + h) * (int64_t)dv;  /* v, out rows */
          if (plant & PLANT_NO_L2NORM) {
            memcpy(qn, q + ok_, sizeof(double) * dk);
            memcpy(kn, k + ok_, sizeof(double) * dk);
          } else {
            l2norm(q + ok_, dk, eps, qn);
            l2norm(k + ok_, dk, eps, kn);
          }
          gate(f + ok_, A_log[h], dt_bias + (int64_t)h * dk, dk, plant, g);
          double beta = (plant & PLANT_NO_BETA) ? 1.0 : sigmoid(b[t * H + h]);
          if (Sprev) memcpy(Sprev, S, sizeof(double) * sz);
          /* S <- Diag(exp(g)) S : row i of S (key channel i) scales by exp(g_i). */
          if (!(plant & PLANT_NO_DECAY)) {
            for (int i = 0; i < dk; ++i) {
              double e = (plant & PLANT_GATE_SIGN) ? exp(-g[i]) : exp(g[i]);
              for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= e;
            }
          }
          double* o_t = out + ov;
          if (plant & PLANT_READ_BEFORE_WRITE) {
            for (int j = 0; j < dv; ++j) {
              double acc = 0.0;
              for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qn[i];
              o_t[j] = ((plant & PLANT_NO_SCALE) ? 1.0 : scale) * acc;
            }
          }
          /* u = v - S^T k  (S^T k)_j = sum_i S[i][j] k_i, on the decayed S. */
          const double* Sd = Sprev ? Sprev : S;
          for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += Sd[(size_t)i * dv + j] * kn[i];
            u[j] = (plant & PLANT_DELTA_SIGN) ? v[ov + j] + acc : v[ov + j] - acc;
          }
          /* S += beta k u^T */
          if ((plant & PLANT_OUTER_SWAP) && square) {
            for (int i = 0; i < dk; ++i)
              for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += beta * u[i] * kn[j];
          } else {
            for (int i = 0; i < dk; ++i) {
              double bk = beta * kn[i];
              for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * u[j];
            }
          }
          if (!(plant & PLANT_READ_BEFORE_WRITE)) {
            /* o_t = scale S^T q */
            for (int j = 0; j < dv; ++j) {
              double acc = 0.0;
              if ((plant & PLANT_TRANSPOSED_READ) && square)
                for (int i = 0; i < dk; ++i) acc += S[(size_t)j * dv + i] * qn[i];
              else
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qn[i];
              o_t[j] = ((plant & PLANT_NO_SCALE) ? 1.0 : scale) * acc;
            }
          }
        }
        if (fin && !((plant & PLANT_FINAL_EARLY) && cu_seqlens[n + 1] > cu_seqlens[n]))
          memcpy(fin, S, sizeof(double) * sz);
      }
    }
    free(S); free(qn); free(kn); free(g); free(u); free(Sprev);
  }
  return 0;
}

/* Number of chunks of size C over all sequences (chunks restart at each
 * sequence start; a sequence of length L has ceil(L/C) chunks). */
int64_t kda_oracle_num_chunks(const int32_t* cu_seqlens, int N, int C) {
  int64_t nc = 0;
  for (int n = 0; n < N; ++n) {
    int64_t L = cu_seqlens[n + 1] - cu_seqlens[n];
    nc += (L + C - 1) / C;
  }
  return nc;
}

/* Size in doubles of one (chunk, head) record written by kda_oracle_chunked. */
int64_t kda_oracle_chunk_record_len(int C, int d) {
  return (int64_t)C * d       /* G    */
         + C                  /* beta */
         + 2 * (int64_t)C * C /* A, P */
         + 4 * (int64_t)C * d /* W, U, Qt, Kb */
         + d                  /* Gamma */
         + (int64_t)d * d;    /* S0   */
}

/* Chunk-form forward with chunk size C (chunks restart at each sequence
 * start).  For a chunk of n <= C tokens entering with state S0:
 *   G[r]   = sum_{j<=r} g_j                      (chunk-local prefix)
 *   A[r,i] = beta_r sum_c k^_rc k^_ic exp(G_rc - G_ic),  i < r
 *   P[r,i] = sum_c q^_rc k^_ic exp(G_rc - G_ic),         i <= r
 *   (I + A) W = Diag(beta) (k^ * exp(G)),  (I + A) U = Diag(beta) V
 *       (unit lower-triangular: forward substitution)
 *   D = U - W S0
 *   O = scale (Qt S0 + P D),  Qt = q^ * exp(G)
 *   S_next = Diag(Gamma) S0 + Kb^T D,  Gamma = exp(G_{n-1}),  Kb = k^ * exp(G_{n-1} - G)
 * This is the token recurrence re-associated: unrolling S over the chunk gives
 * D_r = beta_r (v_r - S_r^-T k^_r) with S_r^- the decayed state before token r.
 * If rec != NULL it receives, per chunk (sequence-major order) and head, the
 * record [G, beta, A, P, W, U, Qt, Kb, Gamma, S0] with rows >= n zero.
 * S_init / S_final as for kda_oracle_fwd. */
int kda_oracle_chunked(const double* q, const double* k, const double* v, const double* f,
                       const double* b, const double* A_log, const double* dt_bias,
                       const int32_t* cu_seqlens, int N, int64_t T, int H, int d, int h_lo,
                       int h_hi, double scale, double eps, int C, const double* S_init,
                       double* S_final, double* out, double* rec) {
  if (N < 1 || H < 1 || d < 1 || C < 1 || h_lo < 0 || h_hi > H || h_lo > h_hi) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int nh = h_hi - h_lo;
  const int64_t RL = kda_oracle_chunk_record_len(C, d);
  /* first chunk index of each sequence */
  int64_t* cfirst = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  cfirst[0] = 0;
  for (int n = 0; n < N; ++n)
    cfirst[n + 1] = cfirst[n] + (cu_seqlens[n + 1] - cu_seqlens[n] + C - 1) / C;

#pragma omp parallel
  {
    const size_t Cd = (size_t)C * d, CC = (size_t)C * C, dd = (size_t)d * d;
    double* S = (double*)malloc(sizeof(double) * dd);
    double* Qn = (double*)malloc(sizeof(double) * Cd);
    double* Kn = (double*)malloc(sizeof(double) * Cd);
    double* G = (double*)malloc(sizeof(double) * Cd);
    double* g = (double*)malloc(sizeof(double) * (size_t)d);
    double* bet = (double*)malloc(sizeof(double) * (size_t)C);
    double* A = (double*)malloc(sizeof(double) * CC);
    double* P = (double*)malloc(sizeof(double) * CC);
    double* W = (double*)malloc(sizeof(double) * Cd);
    double* U = (double*)malloc(sizeof(double) * Cd);
    double* Qt = (double*)malloc(sizeof(double) * Cd);
    double* Kb = (double*)malloc(sizeof(double) * Cd);
    double* Dl = (double*)malloc(sizeof(double) * Cd);
    double* Gam = (double*)malloc(sizeof(double) * (size_t)d);
    double* Sn = (double*)malloc(sizeof(double) * dd);
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < (int64_t)N * nh; ++w) {
      const int h = h_lo + (int)(w % nh), n = (int)(w / nh);
      const int64_t t0 = cu_seqlens[n], L = cu_seqlens[n + 1] - t0;
      load_init(S, S_init, n, H, h, d, 0u);
      for (int64_t j = 0; j * C < L; ++j) {
        const int64_t c0 = t0 + j * C;
        const int nr = (int)((L - j * C) < C ? (L - j * C) : C);
        memset(Qn, 0, sizeof(double) * Cd); memset(Kn, 0, sizeof(double) * Cd);
        memset(G, 0, sizeof(double) * Cd); memset(bet, 0, sizeof(double) * C);
        /* prep: normalised q, k; chunk-local prefix of the log-decay; beta */
        for (int r = 0; r < nr; ++r) {
          const int64_t o = ((c0 + r) * H + h) * (int64_t)d;
          l2norm(q + o, d, eps, Qn + (size_t)r * d);
          l2norm(k + o, d, eps, Kn + (size_t)r * d);
          gate(f + o, A_log[h], dt_bias + (int64_t)h * d, d, 0u, g);
          for (int c = 0; c < d; ++c)
            G[(size_t)r * d + c] = (r ? G[(size_t)(r - 1) * d + c] : 0.0) + g[c];
          bet[r] = sigmoid(b[(c0 + r) * H + h]);
        }
        /* decay-weighted blocks */
        memset(A, 0, sizeof(double) * CC); memset(P, 0, sizeof(double) * CC);
        for (int r = 0; r < nr; ++r)
          for (int i = 0; i <= r; ++i) {
            double sa = 0.0, sp = 0.0;
            for (int c = 0; c < d; ++c) {
              double e = exp(G[(size_t)r * d + c] - G[(size_t)i * d + c]);
              double ke = Kn[(size_t)i * d + c] * e;
              sa += Kn[(size_t)r * d + c] * ke;
              sp += Qn[(size_t)r * d + c] * ke;
            }
            if (i < r) A[(size_t)r * C + i] = bet[r] * sa;
            P[(size_t)r * C + i] = sp;
          }
        /* forward substitution: row r of (I + A) X = B gives
         * X_r = B_r - sum_{i<r} A[r,i] X_i */
        memset(W, 0, sizeof(double) * Cd); memset(U, 0, sizeof(double) * Cd);
        for (int r = 0; r < nr; ++r) {
          const int64_t o = ((c0 + r) * H + h) * (int64_t)d;
          for (int c = 0; c < d; ++c) {
            double xw = bet[r] * Kn[(size_t)r * d + c] * exp(G[(size_t)r * d + c]);
            double xu = bet[r] * v[o + c];
            for (int i = 0; i < r; ++i) {
              xw -= A[(size_t)r * C + i] * W[(size_t)i * d + c];
              xu -= A[(size_t)r * C + i] * U[(size_t)i * d + c];
            }
            W[(size_t)r * d + c] = xw;
            U[(size_t)r * d + c] = xu;
          }
        }
        memset(Qt, 0, sizeof(double) * Cd); memset(Kb, 0, sizeof(double) * Cd);
        const double* Gl = G + (size_t)(nr - 1) * d;
        for (int c = 0; c < d; ++c) Gam[c] = exp(Gl[c]);
        for (int r = 0; r < nr; ++r)
          for (int c = 0; c < d; ++c) {
            Qt[(size_t)r * d + c] = Qn[(size_t)r * d + c] * exp(G[(size_t)r * d + c]);
            Kb[(size_t)r * d + c] = Kn[(size_t)r * d + c] * exp(Gl[c] - G[(size_t)r * d + c]);
          }
        if (rec) {
          double* R = rec + ((cfirst[n] + j) * H + h) * RL;
          memcpy(R, G, sizeof(double) * Cd); R += Cd;
          memcpy(R, bet, sizeof(double) * C); R += C;
          memcpy(R, A, sizeof(double) * CC); R += CC;
          memcpy(R, P, sizeof(double) * CC); R += CC;
          memcpy(R, W, sizeof(double) * Cd); R += Cd;
          memcpy(R, U, sizeof(double) * Cd); R += Cd;
          memcpy(R, Qt, sizeof(double) * Cd); R += Cd;
          memcpy(R, Kb, sizeof(double) * Cd); R += Cd;
          memcpy(R, Gam, sizeof(double) * d); R += d;
          memcpy(R, S, sizeof(double) * dd);
        }
        /* D = U - W S0 */
        for (int r = 0; r < nr; ++r)
          for (int jv = 0; jv < d; ++jv) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += W[(size_t)r * d + i] * S[(size_t)i * d + jv];
            Dl[(size_t)r * d + jv] = U[(size_t)r * d + jv] - acc;
          }
        /* O = scale (Qt S0 + P D) */
        for (int r = 0; r < nr; ++r) {
          double* o_t = out + ((c0 + r) * H + h) * (int64_t)d;
          for (int jv = 0; jv < d; ++jv) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += Qt[(size_t)r * d + i] * S[(size_t)i * d + jv];
            for (int i = 0; i <= r; ++i) acc += P[(size_t)r * C + i] * Dl[(size_t)i * d + jv];
            o_t[jv] = scale * acc;
          }
        }
        /* S_next = Diag(Gamma) S0 + Kb^T D */
        for (int i = 0; i < d; ++i)
          for (int jv = 0; jv < d; ++jv) {
            double acc = Gam[i] * S[(size_t)i * d + jv];
            for (int r = 0; r < nr; ++r) acc += Kb[(size_t)r * d + i] * Dl[(size_t)r * d + jv];
            Sn[(size_t)i * d + jv] = acc;
          }
        memcpy(S, Sn, sizeof(double) * dd);
      }
      if (S_final) memcpy(S_final + ((size_t)n * H + h) * dd, S, sizeof(double) * dd);
    }
    free(S); free(Qn); free(Kn); free(G); free(g); free(bet); free(A); free(P);
    free(W); free(U); free(Qt); free(Kb); free(Dl); free(Gam); free(Sn);
  }
  free(cfirst);
  return 0;
}

/* Round to the nearest bfloat16 value (8 significant bits), ties to even, in
 * one step from the double value (no intermediate float rounding). */
static double round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  const double m = frexp(x, &e);          /* x = m 2^e, 0.5 <= |m| < 1 */
  const double r = nearbyint(ldexp(m, 8)); /* 8 significant bits, ties to even */
  return ldexp(r, e - 8);
}

/* Short causal convolution on one activation tensor, in place (the
 * "KDAShortConvolution" in front of the KDA core, xtuner PR #2153, KDA
 * module description: separate q/k/v causal convolutions whose forward keeps
 * the activation dtype):
 *   y_t[c] = act(bias[c] + sum_{i<K} w[c][i] x_{t-K+1+i}[c])
 * with x_s = 0 for s before the start of t's sequence (no history crosses a
 * sequence boundary), act = SiLU (x sigmoid(x)) when silu != 0, else the
 * identity, and, when round_bf16 != 0, y rounded to bfloat16 (the activation
 * dtype).  x is [T][H][d]; w is [H*d][K] (tap K-1 multiplies the current
 * token); bias is [H*d] or NULL.  Returns 0, or -1 on bad args. */
int kda_oracle_short_conv(double* x, const int32_t* cu_seqlens, int N, int64_t T, int H, int d,
                          const double* w, const double* bias, int K, int silu, int round_to_bf16,
                          unsigned plant) {
  if (N < 1 || H < 1 || d < 1 || K < 1) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  const int64_t HD = (int64_t)H * d;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < HD; ++ch) {
    double* hist = (double*)malloc(sizeof(double) * (size_t)K);
    for (int n = 0; n < N; ++n) {
      if (!(plant & PLANT_CONV_NO_RESET) || n == 0)
        for (int i = 0; i < K; ++i) hist[i] = 0.0;  /* hist[K-1] = current token */
      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        for (int i = 0; i + 1 < K; ++i) hist[i] = hist[i + 1];
        hist[K - 1] = x[t * HD + ch];
        double acc = bias ? bias[ch] : 0.0;
        for (int i = 0; i < K; ++i) {
          const int tap = (plant & PLANT_CONV_TAPS_REVERSED) ? K - 1 - i : i;
          acc += w[ch * K + tap] * hist[i];
        }
        if (silu) acc = acc / (1.0 + exp(-acc));
        x[t * HD + ch] = round_to_bf16 ? round_bf16(acc) : acc;
      }
    }
    free(hist);
  }
  return 0;
}

/* Vector-Jacobian product of kda_oracle_short_conv (the convolution in front
 * of the core, xtuner PR #2153, KDA module description: FP32 weight and bias
 * gradients).  The rounding of the output to the activation dtype is taken as
 * the identity (the backward differentiates the FP64 convolution).  For
 * L = <dy, y>, per channel ch and sequence, with x = 0 before its start:
 *   z_t  = bias + sum_i w_i x_{t-K+1+i}
 *   dz_t = dy_t * act'(z_t),  act'(z) = s (1 + z (1 - s)), s = 1/(1+e^-z) for
 *          SiLU, 1 without
 *   dx_u = sum_i w_i dz_{u+K-1-i}  over the tokens u+K-1-i of the same sequence
 *   dw_i = sum_t dz_t x_{t-K+1+i},  dbias = sum_t dz_t  (over every sequence)
 * x, dy, dx: [T][H*d]; w, dw: [H*d][K]; bias (may be NULL), dbias: [H*d].
 * Every output is overwritten.  Returns 0, or -1 for invalid arguments. */
int kda_oracle_short_conv_vjp(const double* x, const double* dy, const int32_t* cu_seqlens, int N,
                              int64_t T, int H, int d, const double* w, const double* bias, int K,
                              int silu, unsigned plant, double* dx, double* dw, double* dbias) {
  if (N < 1 || H < 1 || d < 1 || K < 1) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  const int64_t HD = (int64_t)H * d;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < HD; ++ch) {
    double* dz = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int i = 0; i < K; ++i) dw[ch * K + i] = 0.0;
    dbias[ch] = 0.0;
    for (int n = 0; n < N; ++n) {
      const int64_t s0 = cu_seqlens[n], s1 = cu_seqlens[n + 1];
      for (int64_t t = s0; t < s1; ++t) {
        double z = bias ? bias[ch] : 0.0;
        for (int i = 0; i < K; ++i) {
          const int64_t u = t - K + 1 + i;
          if (u >= s0) z += w[ch * K + i] * x[u * HD + ch];
        }
        double g = 1.0;
        if (silu && !(plant & PLANT_CONVB_NO_SILU_DERIV)) {
          const double sg = 1.0 / (1.0 + exp(-z));
          g = sg * (1.0 + z * (1.0 - sg));
        }
        dz[t] = dy[t * HD + ch] * g;
        dbias[ch] += dz[t];
        for (int i = 0; i < K; ++i) {
          const int64_t u = t - K + 1 + i;
          if (u >= s0) dw[ch * K + i] += dz[t] * x[u * HD + ch];
        }
      }
      for (int64_t u = s0; u < s1; ++u) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) {
          const int64_t t = (plant & PLANT_CONVB_TAPS_FORWARD) ? u - K + 1 + i : u + K - 1 - i;
          if (t >= s0 && t < s1) acc += w[ch * K + i] * dz[t];
        }
        dx[u * HD + ch] = acc;
      }
    }
    free(dz);
  }
  return 0;
}

/* Vector-Jacobian product of the token recurrence above (reverse-mode
 * differentiation of exactly the steps kda_oracle_fwd_rect takes; the pages
 * check the chunked operator's gradients for q, k, v, the gate and beta
 * against such an independent FP64 recurrence VJP: xtuner PR #2301, section
 * Validation; PR #2153, KDA module description, for the gradients of the FP32
 * A_log / dt_bias parameters and the initial state of a shard).
 *
 * Given dout = dL/dout [T][H][dv] and optionally dS_final = dL/dS_final
 * [N][H][dk][dv], returns dL/d(input) for L = <dout, out> + <dS_final, S_final>:
 *   dq, dk, df [T][H][dk];  dv [T][H][dv];  db [T][H];  dA_log [H];
 *   ddt_bias [H][dk];  dS_init [N][H][dk][dv] (if non-NULL; the gradient of the
 *   start state, whether S_init was given or the start was zero).
 * Every output is overwritten.  Per token, in reverse order, with S_t stored
 * by a forward sweep and Sd = Diag(a) S_{t-1}, u = v - Sd^T k^, a = exp(g):
 *   dq^ = scale S_t dout_t;        dS += scale q^ dout_t^T
 *   du = beta dS^T k^;             dbeta = k^^T dS u;   dk^ = beta dS u
 *   dv = du;  dSd = dS - k^ du^T;  dk^ -= Sd du
 *   da_i = sum_j dSd_ij S_{t-1,ij};  dS <- Diag(a) dSd;  dg = a * da
 *   x = f + dt_bias:  dx = -exp(A_log) sigmoid(x) dg;  df = dx;  ddt_bias += dx
 *   dA_log += sum_c dg_c g_c   (g is linear in exp(A_log))
 *   db = dbeta beta (1 - beta)
 *   dq = (dq^ - q^ (q^ . dq^)) / sqrt(|q|^2 + eps), dk likewise.
 * Memory: the forward sweep keeps all states of one (sequence, head), i.e.
 * (L+1) dk dv doubles per worker thread.  Returns 0, or -1 on bad args. */
int kda_oracle_bwd_rect(const double* q, const double* k, const double* v, const double* f,
                        const double* b, const double* A_log, const double* dt_bias,
                        const int32_t* cu_seqlens, int N, int64_t T, int H, int dk, int dv,
                        double scale, double eps, unsigned plant, const double* S_init,
                        const double* dout, const double* dS_final, double* dq, double* dkk,
                        double* dvv, double* df, double* db, double* dA_log, double* ddt_bias,
                        double* dS_init) {
  if (N < 1 || H < 1 || dk < 1 || dv < 1) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int64_t units = (int64_t)N * H;
  const size_t sz = (size_t)dk * dv;
  /* per-unit partial parameter gradients, summed in a fixed order afterwards */
  double* part = (double*)calloc((size_t)units * (dk + 1), sizeof(double));
  if (!part) return -1;
  int fail = 0;

#pragma omp parallel
  {
    double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* g = (double*)malloc(sizeof(double) * (size_t)dk);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dqn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* dkn = (double*)malloc(sizeof(double) * (size_t)dk);
    double* Sd = (double*)malloc(sizeof(double) * sz);
    double* dS = (double*)malloc(sizeof(double) * sz);
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < units; ++w) {
      const int n = (int)(w / H), h = (int)(w % H);
      const int64_t t0 = cu_seqlens[n], L = cu_seqlens[n + 1] - t0;
      double* St = (double*)malloc(sizeof(double) * sz * (size_t)(L + 1));
      if (!St) {
#pragma omp atomic write
        fail = 1;
        continue;
      }
      const double lam = exp(A_log[h]);
      const double* dtb = dt_bias + (int64_t)h * dk;
      /* forward sweep: St[s] = state after s tokens of the sequence */
      load_init_rect(St, S_init, n, H, h, dk, dv, 0u);
      for (int64_t s = 0; s < L; ++s) {
        const int64_t t = t0 + s;
        const int64_t ok_ = (t * H + h) * (int64_t)dk, ov = (t * H + h) * (int64_t)dv;
        l2norm(q + ok_, dk, eps, qn);
        l2norm(k + ok_, dk, eps, kn);
        gate(f + ok_, A_log[h], dtb, dk, 0u, g);
        const double beta = sigmoid(b[t * H + h]);
        const double* Sp = St + sz * (size_t)s;
        double* Sn = St + sz * (size_t)(s + 1);
        for (int i = 0; i < dk; ++i) {
          const double e = exp(g[i]);
          for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] = e * Sp[(size_t)i * dv + j];
        }
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += Sn[(size_t)i * dv + j] * kn[i];
          u[j] = v[ov + j] - acc;
        }
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] += beta * kn[i] * u[j];
      }
      /* reverse sweep */
      if (dS_final) memcpy(dS, dS_final + ((size_t)n * H + h) * sz, sizeof(double) * sz);
      else memset(dS, 0, sizeof(double) * sz);
      double* pp = part + (size_t)w * (dk + 1);
      for (int64_t s = L - 1; s >= 0; --s) {
        const int64_t t = t0 + s;
        const int64_t ok_ = (t * H + h) * (int64_t)dk, ov = (t * H + h) * (int64_t)dv;
        double ssq = 0.0, ssk = 0.0;
        for (int c = 0; c < dk; ++c) { ssq += q[ok_ + c] * q[ok_ + c]; ssk += k[ok_ + c] * k[ok_ + c]; }
        const double rq = 1.0 / sqrt(ssq + eps), rk = 1.0 / sqrt(ssk + eps);
        for (int c = 0; c < dk; ++c) { qn[c] = q[ok_ + c] * rq; kn[c] = k[ok_ + c] * rk; }
        gate(f + ok_, A_log[h], dtb, dk, 0u, g);
        for (int i = 0; i < dk; ++i) a[i] = exp(g[i]);
        const double beta = sigmoid(b[t * H + h]);
        const double* Sp = St + sz * (size_t)s;        /* S_{t-1} */
        const double* Sc = St + sz * (size_t)(s + 1);  /* S_t     */
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) Sd[(size_t)i * dv + j] = a[i] * Sp[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += Sd[(size_t)i * dv + j] * kn[i];
          u[j] = v[ov + j] - acc;
        }
        const double* go = dout + ov;
        /* o_t = scale S_t^T q^ */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += Sc[(size_t)i * dv + j] * go[j];
          dqn[i] = scale * acc;
          for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += scale * qn[i] * go[j];
        }
        /* S_t = Sd + beta k^ u^T */
        double dbeta = 0.0;
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += kn[i] * dS[(size_t)i * dv + j];
          du[j] = beta * acc;
          dbeta += acc * u[j];
        }
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * u[j];
          dkn[i] = beta * acc;
        }
        /* u = v - Sd^T k^ */
        for (int j = 0; j < dv; ++j) dvv[ov + j] = du[j];
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) {
            dS[(size_t)i * dv + j] -= kn[i] * du[j];  /* now dSd */
            acc += Sd[(size_t)i * dv + j] * du[j];
          }
          dkn[i] -= acc;
        }
        /* Sd = Diag(a) S_{t-1} */
        for (int i = 0; i < dk; ++i) {
          double da = 0.0;
          for (int j = 0; j < dv; ++j) da += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
          if (!(plant & PLANT_BWD_NO_STATE_DECAY))
            for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= a[i];
          const double dg = a[i] * da;
          const double x = f[ok_ + i] + dtb[i];
          const double sg = (plant & PLANT_BWD_GATE_NO_SIGMOID) ? 1.0 : sigmoid(x);
          const double dx = (lam == 0.0) ? 0.0 : -lam * sg * dg;
          df[ok_ + i] = dx;
          pp[i] += dx;
          pp[dk] += dg * g[i];
        }
        if (plant & PLANT_BWD_BETA_SCALE) dbeta *= 1.25;
        db[t * H + h] = dbeta * beta * (1.0 - beta);
        /* L2 normalisation */
        double pq = 0.0, pk = 0.0;
        for (int c = 0; c < dk; ++c) { pq += qn[c] * dqn[c]; pk += kn[c] * dkn[c]; }
        if (plant & PLANT_BWD_NO_NORM_PROJ) pq = pk = 0.0;
        for (int c = 0; c < dk; ++c) {
          dq[ok_ + c] = rq * (dqn[c] - qn[c] * pq);
          dkk[ok_ + c] = rk * (dkn[c] - kn[c] * pk);
        }
      }
      if (dS_init) memcpy(dS_init + ((size_t)n * H + h) * sz, dS, sizeof(double) * sz);
      free(St);
    }
    free(qn); free(kn); free(g); free(a); free(u); free(du); free(dqn); free(dkn); free(Sd);
    free(dS);
  }
  if (!fail) {
    for (int h = 0; h < H; ++h) {
      dA_log[h] = 0.0;
      for (int c = 0; c < dk; ++c) ddt_bias[(int64_t)h * dk + c] = 0.0;
    }
    for (int64_t w = 0; w < units; ++w) {
      const int h = (int)(w % H);
      const double* pp = part + (size_t)w * (dk + 1);
      for (int c = 0; c < dk; ++c) ddt_bias[(int64_t)h * dk + c] += pp[c];
      dA_log[h] += pp[dk];
    }
  }
  free(part);
  return fail ? -1 : 0;
}

/* Number of threads the OpenMP runtime will use (reported by the benchmark). */
/* Thread count for the OpenMP loops that follow (timing only; results do
 * not depend on it: every (sequence, head) pair is computed by one thread). */
void kda_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
