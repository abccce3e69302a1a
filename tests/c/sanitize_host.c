/*
 * Driver for the host sanitizer test (AddressSanitizer + UndefinedBehavior-
 * Sanitizer).  Built twice by tests/test_sanitizers.py, never on a GPU:
 *
 *   ORACLE_PART: the fp64 oracle and the input generator, compiled together
 *     with this file, run on small inputs through every exported function
 *     (N up to 9, T spanning several dw chunks, a dw-only backward, a bf16 add
 *     over every exponent, odd and even generator offsets);
 *   ABI_PART: libattnres's host code (argument validation and overlap checks)
 *     called with invalid arguments that are refused before any HIP call;
 *     every call must return the documented status.
 *
 * Exits 0 and prints "ok" only if every check holds; a sanitizer report
 * aborts the run with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int fails = 0;
#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++fails;                                                       \
    }                                                                \
  } while (0)

#ifdef ORACLE_PART
void synth_u64(uint64_t* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0);
void synth_uniform_f64(double* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0);
void synth_normal_f32(float* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0, float scale);
void synth_rows_bf16(uint16_t* dst, int64_t rows, int64_t D, uint64_t seed, uint64_t stream, int64_t row0,
                     float scale, const float* chan_mult);
void oracle_fwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, double* out,
                double* rstd, double* alpha);
void oracle_bwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, const uint16_t* dout,
                double* dx, double* dw);
void oracle_fwd_f64(int N, int64_t T, int64_t D, const double* x, const double* w, double eps, double* out,
                    double* rstd, double* alpha);
void oracle_bwd_f64(int N, int64_t T, int64_t D, const double* x, const double* w, double eps, const double* g,
                    double* dx, double* dw);
void oracle_add_bf16(int64_t n, const uint16_t* p, const uint16_t* y, uint16_t* out);
void oracle_block_scores(int n, int64_t T, int64_t D, int L, const uint16_t* src, const float* W, double eps,
                         double* rstd, double* z);
void oracle_fwd_scored(int N, int64_t T, int64_t D, const uint16_t* src, const double* zg, const double* rg,
                       const float* w, double eps, double* out, double* rstd, double* alpha);
void oracle_block_sums(int n, int64_t T, int64_t D, int L, const uint16_t* src, const double* z, double* U);
void oracle_fwd_merged(int N, int64_t T, int64_t D, const double* U, const uint16_t* p, const double* zg,
                       const double* rg, const float* w, double eps, double* out, double* rstd, double* alpha);

static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void run_oracle(void) {
  enum { N = 9, T = 70, D = 24 };
  uint16_t* src = malloc(sizeof(uint16_t) * N * T * D);
  uint16_t* dout = malloc(sizeof(uint16_t) * T * D);
  float* w = malloc(sizeof(float) * D);
  float* mult = malloc(sizeof(float) * D);
  for (int d = 0; d < D; ++d) mult[d] = d % 5 == 0 ? 100.f : 1.f;
  for (int i = 0; i < N; ++i) synth_rows_bf16(src + (size_t)i * T * D, T, D, 0, 100 + i, i, 1.f + i, i & 1 ? mult : NULL);
  synth_rows_bf16(dout, T, D, 0, 2, 0, 1.f, NULL);
  synth_normal_f32(w, D, 0, 1, 0, 0.2f);
  uint64_t u[7];
  double un[7];
  synth_u64(u, 7, 3, 4, 5);
  synth_uniform_f64(un, 7, 3, 4, 5);
  for (int k = 0; k < 7; ++k) EXPECT(un[k] >= 0.0 && un[k] < 1.0);

  double* out = malloc(sizeof(double) * T * D);
  double* rstd = malloc(sizeof(double) * T * N);
  double* alpha = malloc(sizeof(double) * T * N);
  double* dx = malloc(sizeof(double) * N * T * D);
  double* dw = malloc(sizeof(double) * D);
  double* dw2 = malloc(sizeof(double) * D);
  oracle_fwd(N, T, D, src, w, 1e-6, out, rstd, alpha);
  oracle_bwd(N, T, D, src, w, 1e-6, dout, dx, dw);
  oracle_bwd(N, T, D, src, w, 1e-6, dout, NULL, dw2);
  for (int t = 0; t < T; ++t) {
    double s = 0;
    for (int i = 0; i < N; ++i) s += alpha[t * N + i];
    EXPECT(fabs(s - 1.0) < 1e-12);
  }
  for (int d = 0; d < D; ++d) EXPECT(dw[d] == dw2[d] && isfinite(dw[d]));
  for (size_t k = 0; k < (size_t)N * T * D; ++k) EXPECT(isfinite(dx[k]));

  /* the fp64 entry on the widened values gives the same numbers */
  double* x = malloc(sizeof(double) * N * T * D);
  double* g = malloc(sizeof(double) * T * D);
  double* wd = malloc(sizeof(double) * D);
  double* out2 = malloc(sizeof(double) * T * D);
  double* dx2 = malloc(sizeof(double) * N * T * D);
  for (size_t k = 0; k < (size_t)N * T * D; ++k) x[k] = bf(src[k]);
  for (size_t k = 0; k < (size_t)T * D; ++k) g[k] = bf(dout[k]);
  for (int d = 0; d < D; ++d) wd[d] = w[d];
  oracle_fwd_f64(N, T, D, x, wd, 1e-6, out2, NULL, NULL);
  oracle_bwd_f64(N, T, D, x, wd, 1e-6, g, dx2, dw2);
  EXPECT(memcmp(out, out2, sizeof(double) * T * D) == 0);
  EXPECT(memcmp(dx, dx2, sizeof(double) * N * T * D) == 0);

  /* block-batched scores of the first N-1 sources for three pseudo-queries (w
   * the last), then the forward from those scores equals the plain forward */
  {
    enum { L = 3 };
    float* W = malloc(sizeof(float) * L * D);
    for (int l = 0; l < L; ++l) synth_normal_f32(W + l * D, D, 0, 7 + l, 0, 0.3f);
    memcpy(W + (L - 1) * D, w, sizeof(float) * D);
    double* rb = malloc(sizeof(double) * T * (N - 1));
    double* zb = malloc(sizeof(double) * L * T * (N - 1));
    double* out3 = malloc(sizeof(double) * T * D);
    double* rstd3 = malloc(sizeof(double) * T * N);
    double* alpha3 = malloc(sizeof(double) * T * N);
    oracle_block_scores(N - 1, T, D, L, src, W, 1e-6, rb, zb);
    oracle_fwd_scored(N, T, D, src, zb + (size_t)(L - 1) * T * (N - 1), rb, w, 1e-6, out3, rstd3, alpha3);
    for (size_t k = 0; k < (size_t)T * D; ++k) EXPECT(fabs(out3[k] - out[k]) <= 1e-12 * (1.0 + fabs(out[k])));
    for (size_t k = 0; k < (size_t)T * N; ++k) EXPECT(fabs(alpha3[k] - alpha[k]) <= 1e-12);
    /* the shared sums of those sources, then the last sub-layer's forward from its sum */
    double* U = malloc(sizeof(double) * L * T * D);
    oracle_block_sums(N - 1, T, D, L, src, zb, U);
    oracle_fwd_merged(N, T, D, U + (size_t)(L - 1) * T * D, src + (size_t)(N - 1) * T * D,
                      zb + (size_t)(L - 1) * T * (N - 1), rb, w, 1e-6, out3, rstd3, alpha3);
    for (size_t k = 0; k < (size_t)T * D; ++k) EXPECT(fabs(out3[k] - out[k]) <= 1e-12 * (1.0 + fabs(out[k])));
    for (size_t k = 0; k < (size_t)T * N; ++k) EXPECT(fabs(alpha3[k] - alpha[k]) <= 1e-12);
    free(U);
    free(W); free(rb); free(zb); free(out3); free(rstd3); free(alpha3);
  }

  /* bf16 add over every exponent and sign of the first operand */
  enum { M = 1 << 16 };
  uint16_t* p = malloc(sizeof(uint16_t) * M);
  uint16_t* y = malloc(sizeof(uint16_t) * M);
  uint16_t* s = malloc(sizeof(uint16_t) * M);
  for (int k = 0; k < M; ++k) {
    p[k] = (uint16_t)k;
    y[k] = (uint16_t)(u[k % 7] >> (k % 48));
  }
  oracle_add_bf16(M, p, y, s);
  for (int k = 0; k < M; ++k) {
    const double a = bf(p[k]), b = bf(y[k]);
    if (isfinite(a) && isfinite(b) && a + b == 0.0) EXPECT(bf(s[k]) == 0.0);
  }
  free(src); free(dout); free(w); free(mult); free(out); free(rstd); free(alpha); free(dx); free(dw); free(dw2);
  free(x); free(g); free(wd); free(out2); free(dx2); free(p); free(y); free(s);
}
#endif

#ifdef ABI_PART
#include "attnres.h"

static void run_abi(void) {
  /* Fake device addresses: every call below is refused during validation,
   * before the library makes any HIP call, so they are never dereferenced. */
  const uintptr_t A = (uintptr_t)1 << 32;
  const int N = 3, D = 64;
  const int64_t T = 16;
  const uint16_t* src = (const uint16_t*)(A);
  const float* w = (const float*)(A + ((uintptr_t)1 << 28));
  uint16_t* out = (uint16_t*)(A + ((uintptr_t)2 << 28));
  float* rstd = (float*)(A + ((uintptr_t)3 << 28));
  float* alpha = (float*)(A + ((uintptr_t)4 << 28));
  uint16_t* dsrc = (uint16_t*)(A + ((uintptr_t)5 << 28));
  float* dw = (float*)(A + ((uintptr_t)6 << 28));
  void* ws = (void*)(A + ((uintptr_t)7 << 28));
  const uint16_t* dout = (const uint16_t*)(A + ((uintptr_t)8 << 28));
  const size_t wsb = ATTNRES_BWD_WORKSPACE_BYTES(T, N, D);

  EXPECT(attnres_fwd(NULL, w, 1e-6f, N, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, 0, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, 10, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, N, -1, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, N, T, 12, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, N, T, ATTNRES_MAX_D + 8, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, -1.f, N, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, NAN, N, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src + 1, w, 1e-6f, N, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, N, T, D, (uint16_t*)src + 64, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd(src, w, 1e-6f, N, (int64_t)1 << 40, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);

  EXPECT(attnres_bwd(dout, src, w, rstd, alpha, N, T, D, dsrc, dw, NULL, wsb, NULL) == ATTNRES_ERR_WORKSPACE);
  EXPECT(attnres_bwd(dout, src, w, rstd, alpha, N, T, D, dsrc, dw, ws, wsb - 16, NULL) == ATTNRES_ERR_WORKSPACE);
  EXPECT(attnres_bwd(dout, src, w, rstd, alpha, N, T, D, (uint16_t*)src, dw, ws, wsb, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_bwd(dout, src, w, rstd, alpha, N, T, D, dsrc, (float*)ws, ws, wsb, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);

  const uint16_t* srcs[ATTNRES_MAX_SOURCES];
  void* dsrcs[ATTNRES_MAX_SOURCES];
  for (int i = 0; i < ATTNRES_MAX_SOURCES; ++i) {
    srcs[i] = src + (size_t)i * D;        /* interleaved by token: pitch N*D */
    dsrcs[i] = dsrc + (size_t)i * D;
  }
  EXPECT(attnres_fwd_sources(srcs, (int64_t)N * D + 4, w, 1e-6f, N, T, D, out, rstd, alpha, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT); /* pitch not a multiple of 8 */
  EXPECT(attnres_fwd_sources(srcs, D - 8, w, 1e-6f, N, T, D, out, rstd, alpha, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT); /* pitch shorter than a row */
  EXPECT(attnres_fwd_decode(srcs, (int64_t)N * D, w, 1e-6f, N, T, D, out, rstd, NULL, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT); /* exactly one of rstd/alpha */
  EXPECT(attnres_fwd_update(srcs, (int64_t)N * D, NULL, dout, w, 1e-6f, N, T, D, (uint16_t*)srcs[N - 1], out, rstd,
                            alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT); /* no partial sum */
  EXPECT(attnres_bwd_sources(dout, srcs, (int64_t)N * D, w, rstd, alpha, N, T, D, dsrcs, (int64_t)N * D, 4, dw, ws,
                             wsb, NULL) == ATTNRES_ERR_INVALID_ARGUMENT); /* unknown grad_mode */
  /* fp32 gradients interleaved with the bf16 pitch collide with each other */
  EXPECT(attnres_bwd_sources(dout, srcs, (int64_t)N * D, w, rstd, alpha, N, T, D, dsrcs, (int64_t)N * D,
                             ATTNRES_GRAD_F32, dw, ws, wsb, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  /* gradients on top of the sources */
  void* bad[ATTNRES_MAX_SOURCES];
  for (int i = 0; i < N; ++i) bad[i] = (void*)srcs[i];
  EXPECT(attnres_bwd_sources(dout, srcs, (int64_t)N * D, w, rstd, alpha, N, T, D, bad, (int64_t)N * D, 0, dw, ws,
                             wsb, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  /* block sums: colliding U rows, U on top of a source; merged forward: out on top of U, misaligned partial sum */
  float* U = (float*)ws;
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 4, N - 1, T, D, U, D, D, ATTNRES_U_F32, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 4, N - 1, T, D, (float*)srcs[0], (int64_t)T * D, D,
                            ATTNRES_U_F32, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 0, N - 1, T, D, U, (int64_t)T * D, D, ATTNRES_U_F32, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged(U, D, ATTNRES_U_F32, srcs[N - 1], (int64_t)N * D, NULL, NULL, rstd, alpha, w, 1e-6f, N, T, D,
                            (uint16_t*)U, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged(U, D, ATTNRES_U_F32, srcs[N - 1] + 1, (int64_t)N * D, NULL, NULL, rstd, alpha, w, 1e-6f, N, T, D, out,
                            rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged(U, D, ATTNRES_U_F32, srcs[N - 1], (int64_t)N * D, NULL, NULL, rstd, alpha, w, 1e-6f, 1, T, D, out, rstd,
                            alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  /* the 24-bit U format: another format number, U bases that are not 4-byte aligned, and 3-byte rows on top of
   * a source */
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 4, N - 1, T, D, U, (int64_t)T * D, D, 2, NULL) ==
         ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 4, N - 1, T, D, (uint8_t*)U + 2, (int64_t)T * D, D,
                            ATTNRES_U_F24, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_block_sums(srcs, (int64_t)N * D, rstd, 4, N - 1, T, D, (void*)srcs[1], (int64_t)T * D, D,
                            ATTNRES_U_F24, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged((uint8_t*)U + 2, D, ATTNRES_U_F24, srcs[N - 1], (int64_t)N * D, NULL, NULL, rstd, alpha, w,
                            1e-6f, N, T, D, out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged(U, D, -1, srcs[N - 1], (int64_t)N * D, NULL, NULL, rstd, alpha, w, 1e-6f, N, T, D, out,
                            rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  /* the update: delta without partial_out, and partial_out on top of delta */
  EXPECT(attnres_fwd_merged(U, D, ATTNRES_U_F32, srcs[N - 1], (int64_t)N * D, dout, NULL, rstd, alpha, w, 1e-6f, N, T, D, out, rstd,
                            alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
  EXPECT(attnres_fwd_merged(U, D, ATTNRES_U_F32, srcs[N - 1], (int64_t)N * D, dout, (uint16_t*)dout, rstd, alpha, w, 1e-6f, N, T, D,
                            out, rstd, alpha, NULL) == ATTNRES_ERR_INVALID_ARGUMENT);
}
#endif

int main(void) {
#ifdef ORACLE_PART
  run_oracle();
#endif
#ifdef ABI_PART
  run_abi();
#endif
  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
