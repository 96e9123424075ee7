/* oracle_sanitize.c -- drives every entry point of the FP64 oracle
 * (oracle/kda_oracle.c) on small packed inputs, for a build with the address
 * and undefined-behaviour sanitizers.  Test infrastructure: it checks that no
 * call reads or writes outside its arrays, leaks or hits undefined behaviour,
 * plus two cross-checks (chunk form = token recurrence; a rectangular state
 * with zero-padded keys = the square one).  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void kda_oracle_prep(const double*, const double*, const double*, const double*, const double*,
                     const double*, int64_t, int, int, double, double*, double*, double*, double*);
int kda_oracle_fwd(const double*, const double*, const double*, const double*, const double*,
                   const double*, const double*, const int32_t*, int, int64_t, int, int, int, int,
                   double, double, unsigned, const double*, double*, double*);
int kda_oracle_fwd_rect(const double*, const double*, const double*, const double*, const double*,
                        const double*, const double*, const int32_t*, int, int64_t, int, int, int,
                        int, int, double, double, unsigned, const double*, double*, double*);
int64_t kda_oracle_num_chunks(const int32_t*, int, int);
int64_t kda_oracle_chunk_record_len(int, int);
int kda_oracle_chunked(const double*, const double*, const double*, const double*, const double*,
                       const double*, const double*, const int32_t*, int, int64_t, int, int, int,
                       int, double, double, int, const double*, double*, double*, double*);
int kda_oracle_short_conv(double*, const int32_t*, int, int64_t, int, int, const double*,
                          const double*, int, int, int, unsigned);
int kda_oracle_short_conv_vjp(const double*, const double*, const int32_t*, int, int64_t, int, int,
                              const double*, const double*, int, int, unsigned, double*, double*,
                              double*);
int kda_oracle_bwd_rect(const double*, const double*, const double*, const double*, const double*,
                        const double*, const double*, const int32_t*, int, int64_t, int, int, int,
                        double, double, unsigned, const double*, const double*, const double*,
                        double*, double*, double*, double*, double*, double*, double*, double*);
void kda_oracle_set_num_threads(int);
int kda_oracle_num_threads(void);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(size_t n, double scale) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = scale * urand();
  return p;
}
static int fails = 0;
#define CHECK(cond, what)                                 \
  do {                                                    \
    if (!(cond)) { fprintf(stderr, "FAIL: %s\n", what); ++fails; } \
  } while (0)

int main(void) {
  enum { N = 3, H = 2, D = 16, T = 70, DV = 24 };
  const int32_t cu[N + 1] = {0, 37, 37, 70};
  kda_oracle_set_num_threads(2);
  CHECK(kda_oracle_num_threads() >= 1, "num_threads");
  const size_t nk = (size_t)T * H * D, nv = (size_t)T * H * DV, ns = (size_t)N * H * D * D;
  double *q = arr(nk, 1), *k = arr(nk, 1), *v = arr(nk, 1), *f = arr(nk, 1), *b = arr((size_t)T * H, 1);
  double *A_log = arr(H, 1), *dtb = arr((size_t)H * D, 0.5), *S0 = arr(ns, 0.3);
  for (int h = 0; h < H; ++h) A_log[h] = 1.0 + 0.5 * A_log[h];
  const double scale = 1.0 / sqrt((double)D), eps = 1e-6;

  double *qn = arr(nk, 0), *kn = arr(nk, 0), *g = arr(nk, 0), *beta = arr((size_t)T * H, 0);
  kda_oracle_prep(q, k, f, b, A_log, dtb, T, H, D, eps, qn, kn, g, beta);

  double *out = arr(nk, 0), *out2 = arr(nk, 0), *fin = arr(ns, 0), *fin2 = arr(ns, 0);
  CHECK(kda_oracle_fwd(q, k, v, f, b, A_log, dtb, cu, N, T, H, D, 0, H, scale, eps, 0u, S0, fin,
                       out) == 0, "fwd");
  const int C = 16;
  const int64_t nc = kda_oracle_num_chunks(cu, N, C);
  CHECK(nc == 3 + 0 + 3, "num_chunks");
  double* rec = arr((size_t)(nc * H * kda_oracle_chunk_record_len(C, D)), 0);
  CHECK(kda_oracle_chunked(q, k, v, f, b, A_log, dtb, cu, N, T, H, D, 0, H, scale, eps, C, S0, fin2,
                           out2, rec) == 0, "chunked");
  double err = 0;
  for (size_t i = 0; i < nk; ++i) err = fmax(err, fabs(out[i] - out2[i]));
  for (size_t i = 0; i < ns; ++i) err = fmax(err, fabs(fin[i] - fin2[i]));
  CHECK(err < 1e-10, "chunk form = token recurrence");

  /* rectangular state: values of width 24; keys zero-padded from 16 to 24 */
  double *vr = arr(nv, 1), *outr = arr(nv, 0), *finr = arr((size_t)N * H * D * DV, 0);
  CHECK(kda_oracle_fwd_rect(q, k, vr, f, b, A_log, dtb, cu, N, T, H, D, DV, 0, H, scale, eps, 0u,
                            NULL, finr, outr) == 0, "fwd_rect");
  {
    double *qp = arr((size_t)T * H * DV, 0), *kp = arr((size_t)T * H * DV, 0);
    double *fp = arr((size_t)T * H * DV, 0), *dp = arr((size_t)H * DV, 0);
    double* outp = arr(nv, 0);
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h)
        for (int c = 0; c < D; ++c) {
          const size_t a = ((size_t)t * H + h) * DV + c, o = ((size_t)t * H + h) * D + c;
          qp[a] = q[o]; kp[a] = k[o]; fp[a] = f[o];
        }
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < D; ++c) dp[(size_t)h * DV + c] = dtb[(size_t)h * D + c];
    CHECK(kda_oracle_fwd_rect(qp, kp, vr, fp, b, A_log, dp, cu, N, T, H, DV, DV, 0, H, scale, eps,
                              0u, NULL, NULL, outp) == 0, "fwd_rect padded");
    double e2 = 0;
    for (size_t i = 0; i < nv; ++i) e2 = fmax(e2, fabs(outp[i] - outr[i]));
    CHECK(e2 < 1e-10, "zero-padded keys = rectangular state");
    free(qp); free(kp); free(fp); free(dp); free(outp);
  }

  double *dout = arr(nv, 1), *dSf = arr((size_t)N * H * D * DV, 1), *Sr = arr((size_t)N * H * D * DV, 0.3);
  double *dq = arr(nk, 0), *dk = arr(nk, 0), *dvv = arr(nv, 0), *df = arr(nk, 0), *db = arr((size_t)T * H, 0);
  double *dA = arr(H, 0), *ddt = arr((size_t)H * D, 0), *dS0 = arr((size_t)N * H * D * DV, 0);
  CHECK(kda_oracle_bwd_rect(q, k, vr, f, b, A_log, dtb, cu, N, T, H, D, DV, scale, eps, 0u, Sr, dout,
                            dSf, dq, dk, dvv, df, db, dA, ddt, dS0) == 0, "bwd_rect");

  enum { K = 4 };
  double *x = arr(nk, 1), *w = arr((size_t)H * D * K, 0.5), *bias = arr((size_t)H * D, 0.1);
  double* y = arr(nk, 0);
  memcpy(y, x, sizeof(double) * nk);
  CHECK(kda_oracle_short_conv(y, cu, N, T, H, D, w, bias, K, 1, 1, 0u) == 0, "short_conv");
  double *dy = arr(nk, 1), *dx = arr(nk, 0), *dw = arr((size_t)H * D * K, 0), *dbias = arr((size_t)H * D, 0);
  CHECK(kda_oracle_short_conv_vjp(x, dy, cu, N, T, H, D, w, bias, K, 1, 0u, dx, dw, dbias) == 0,
        "short_conv_vjp");
  /* argument errors are refused */
  const int32_t bad[N + 1] = {0, 40, 30, 70};
  CHECK(kda_oracle_fwd(q, k, v, f, b, A_log, dtb, bad, N, T, H, D, 0, H, scale, eps, 0u, NULL, NULL,
                       out) != 0, "fwd refuses a decreasing cu_seqlens");
  CHECK(kda_oracle_short_conv(y, cu, N, T + 1, H, D, w, bias, K, 1, 0, 0u) != 0,
        "short_conv refuses a wrong token count");

  double* all[] = {q, k, v, f, b, A_log, dtb, S0, qn, kn, g, beta, out, out2, fin, fin2, rec, vr, outr,
                   finr, dout, dSf, Sr, dq, dk, dvv, df, db, dA, ddt, dS0, x, w, bias, y, dy, dx, dw,
                   dbias};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  if (fails) return 1;
  printf("oracle sanitizer run: all calls clean\n");
  return 0;
}
