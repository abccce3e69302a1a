/*
 * A plain C consumer of libattnres: no Python, no torch.  Device memory comes
 * from hipMalloc, inputs from the seeded generator (libsynth), the reference
 * from the fp64 oracle (liboracle, test infrastructure).  It runs the stacked
 * forward/backward and the per-source forward on a small workload (N = 8,
 * T = 130, D = 7168, source scales 1, 2, 4 repeated; N = 8 takes the split
 * backward, whose exchange is also run on its recompute route), compares
 * against the oracle with
 * the operator's tolerances, checks that a bad argument is refused with
 * ATTNRES_ERR_INVALID_ARGUMENT, runs the block-level route (block scores of
 * the first seven sources for four pseudo-queries, block sums, the merged
 * forward of one sub-layer with the eighth source as its partial sum) against
 * the oracle's plain forward, and exits 0 only if everything holds.
 */
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attnres.h"

/* libsynth */
void synth_rows_bf16(uint16_t* dst, int64_t rows, int64_t D, uint64_t seed, uint64_t stream, int64_t row0,
                     float scale, const float* chan_mult);
void synth_normal_f32(float* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t c0, float scale);
/* liboracle */
void oracle_fwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, double* out,
                double* rstd, double* alpha);
void oracle_bwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, const uint16_t* dout,
                double* dx, double* dw);

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)

static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double rel_l2_bf16(const uint16_t* got, const double* ref, size_t n) {
  double num = 0, den = 0;
  for (size_t i = 0; i < n; ++i) {
    const double d = bf16_to_f64(got[i]) - ref[i];
    num += d * d;
    den += ref[i] * ref[i];
  }
  return sqrt(num / den);
}

static double rel_l2_f32(const float* got, const double* ref, size_t n) {
  double num = 0, den = 0;
  for (size_t i = 0; i < n; ++i) {
    const double d = (double)got[i] - ref[i];
    num += d * d;
    den += ref[i] * ref[i];
  }
  return sqrt(num / den);
}

int main(void) {
  const int N = 8;
  const int64_t T = 130, D = 7168;
  const float eps = 1e-6f;
  const size_t nsrc = (size_t)N * T * D, nTD = (size_t)T * D, nTN = (size_t)T * N;
  const float scales[8] = {1.f, 2.f, 4.f, 1.f, 2.f, 4.f, 1.f, 2.f};

  uint16_t* src = malloc(nsrc * 2);
  uint16_t* dout = malloc(nTD * 2);
  float* w = malloc(D * 4);
  for (int i = 0; i < N; ++i) synth_rows_bf16(src + (size_t)i * nTD, T, D, 0, 100 + i, 0, scales[i], NULL);
  synth_rows_bf16(dout, T, D, 0, 2, 0, 1.f, NULL);
  synth_normal_f32(w, D, 0, 1, 0, 1.f / sqrtf((float)D));

  uint16_t *d_src, *d_dout, *d_out, *d_out2, *d_dsrc;
  float *d_w, *d_rstd, *d_alpha, *d_rstd2, *d_alpha2, *d_dw;
  void* d_ws;
  const size_t ws_bytes = ATTNRES_BWD_WORKSPACE_BYTES(T, N, D);
  CHECK_HIP(hipMalloc((void**)&d_src, nsrc * 2));
  CHECK_HIP(hipMalloc((void**)&d_dsrc, nsrc * 2));
  CHECK_HIP(hipMalloc((void**)&d_dout, nTD * 2));
  CHECK_HIP(hipMalloc((void**)&d_out, nTD * 2));
  CHECK_HIP(hipMalloc((void**)&d_out2, nTD * 2));
  CHECK_HIP(hipMalloc((void**)&d_w, D * 4));
  CHECK_HIP(hipMalloc((void**)&d_rstd, nTN * 4));
  CHECK_HIP(hipMalloc((void**)&d_alpha, nTN * 4));
  CHECK_HIP(hipMalloc((void**)&d_rstd2, nTN * 4));
  CHECK_HIP(hipMalloc((void**)&d_alpha2, nTN * 4));
  CHECK_HIP(hipMalloc((void**)&d_dw, D * 4));
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMemcpy(d_src, src, nsrc * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_dout, dout, nTD * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w, D * 4, hipMemcpyHostToDevice));

  int fails = 0;
  attnres_status st = attnres_fwd(d_src, d_w, eps, N, T, (int32_t)D, d_out, d_rstd, d_alpha, NULL);
  if (st != ATTNRES_OK) { fprintf(stderr, "attnres_fwd returned %d\n", (int)st); return 1; }
  st = attnres_bwd(d_dout, d_src, d_w, d_rstd, d_alpha, N, T, (int32_t)D, d_dsrc, d_dw, d_ws, ws_bytes, NULL);
  if (st != ATTNRES_OK) { fprintf(stderr, "attnres_bwd returned %d\n", (int)st); return 1; }
  const uint16_t* srcs[8];
  for (int i = 0; i < N; ++i) srcs[i] = d_src + (size_t)i * nTD;
  st = attnres_fwd_sources(srcs, D, d_w, eps, N, T, (int32_t)D, d_out2, d_rstd2, d_alpha2, NULL);
  if (st != ATTNRES_OK) { fprintf(stderr, "attnres_fwd_sources returned %d\n", (int)st); return 1; }
  st = attnres_fwd(d_src, d_w, eps, 10, T, (int32_t)D, d_out, d_rstd, d_alpha, NULL);
  if (st != ATTNRES_ERR_INVALID_ARGUMENT) { fprintf(stderr, "N = 10 not refused (%d)\n", (int)st); ++fails; }
  CHECK_HIP(hipDeviceSynchronize());

  uint16_t* out = malloc(nTD * 2);
  uint16_t* out2 = malloc(nTD * 2);
  uint16_t* dsrc = malloc(nsrc * 2);
  float* rstd = malloc(nTN * 4);
  float* alpha = malloc(nTN * 4);
  float* alpha2 = malloc(nTN * 4);
  float* dw = malloc(D * 4);
  CHECK_HIP(hipMemcpy(out, d_out, nTD * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out2, d_out2, nTD * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dsrc, d_dsrc, nsrc * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(rstd, d_rstd, nTN * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(alpha, d_alpha, nTN * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(alpha2, d_alpha2, nTN * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dw, d_dw, D * 4, hipMemcpyDeviceToHost));

  double* r_out = malloc(nTD * 8);
  double* r_rstd = malloc(nTN * 8);
  double* r_alpha = malloc(nTN * 8);
  double* r_dx = malloc(nsrc * 8);
  double* r_dw = malloc(D * 8);
  oracle_fwd(N, T, D, src, w, eps, r_out, r_rstd, r_alpha);
  oracle_bwd(N, T, D, src, w, eps, dout, r_dx, r_dw);

  double e_alpha = 0, e_rstd = 0;
  for (size_t i = 0; i < nTN; ++i) {
    e_alpha = fmax(e_alpha, fabs((double)alpha[i] - r_alpha[i]));
    e_rstd = fmax(e_rstd, fabs((double)rstd[i] / r_rstd[i] - 1.0));
  }
  const double e_out = rel_l2_bf16(out, r_out, nTD);
  const double e_dsrc = rel_l2_bf16(dsrc, r_dx, nsrc);
  const double e_dw = rel_l2_f32(dw, r_dw, D);
  const int same = memcmp(out, out2, nTD * 2) == 0 && memcmp(alpha, alpha2, nTN * 4) == 0;
  printf("out rel_l2 %.3e  alpha max abs %.3e  rstd max rel %.3e  dsrc rel_l2 %.3e  dw rel_l2 %.3e  "
         "per-source == stacked: %s\n", e_out, e_alpha, e_rstd, e_dsrc, e_dw, same ? "yes" : "no");
  if (!(e_out <= 5e-3 && e_alpha <= 1e-5 && e_rstd <= 1e-5 && e_dsrc <= 1e-2 && e_dw <= 1e-2 && same)) ++fails;

  /* the backward again with every exchanged word recomputed: bitwise the same */
  const uint32_t prev = attnres_set_split_spin(0);
  st = attnres_bwd(d_dout, d_src, d_w, d_rstd, d_alpha, N, T, (int32_t)D, d_dsrc, d_dw, d_ws, ws_bytes, NULL);
  attnres_set_split_spin(prev);
  if (st != ATTNRES_OK) { fprintf(stderr, "attnres_bwd (poll bound 0) returned %d\n", (int)st); return 1; }
  uint16_t* dsrc0 = malloc(nsrc * 2);
  float* dw0 = malloc(D * 4);
  CHECK_HIP(hipMemcpy(dsrc0, d_dsrc, nsrc * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dw0, d_dw, D * 4, hipMemcpyDeviceToHost));
  const int same0 = memcmp(dsrc, dsrc0, nsrc * 2) == 0 && memcmp(dw, dw0, D * 4) == 0;
  printf("recomputed exchange == ring exchange: %s\n", same0 ? "yes" : "no");
  if (prev != ATTNRES_SPLIT_SPIN_DEFAULT || !same0) ++fails;

  /* the block-level route: sources 0..6 shared, source 7 the partial sum, sub-layer 2 of 4 */
  {
    const int L = 4, n = N - 1, l = 2;
    float* W = malloc((size_t)L * D * 4);
    synth_normal_f32(W, (int64_t)L * D, 0, 3, 0, 1.f / sqrtf((float)D));
    float *d_W, *d_rb, *d_zb, *d_U, *d_rstd3, *d_alpha3;
    uint16_t* d_out3;
    void* d_bws;
    const size_t bws = ATTNRES_BLOCK_SCORES_WORKSPACE_BYTES(L, D);
    CHECK_HIP(hipMalloc((void**)&d_W, (size_t)L * D * 4));
    CHECK_HIP(hipMalloc((void**)&d_rb, (size_t)T * n * 4));
    CHECK_HIP(hipMalloc((void**)&d_zb, (size_t)L * T * n * 4));
    CHECK_HIP(hipMalloc((void**)&d_U, (size_t)L * T * D * 4));
    CHECK_HIP(hipMalloc((void**)&d_out3, nTD * 2));
    CHECK_HIP(hipMalloc((void**)&d_rstd3, nTN * 4));
    CHECK_HIP(hipMalloc((void**)&d_alpha3, nTN * 4));
    CHECK_HIP(hipMalloc(&d_bws, bws));
    CHECK_HIP(hipMemcpy(d_W, W, (size_t)L * D * 4, hipMemcpyHostToDevice));
    st = attnres_block_scores(srcs, D, d_W, L, eps, n, T, (int32_t)D, d_rb, d_zb, d_bws, bws, NULL);
    if (st != ATTNRES_OK) { fprintf(stderr, "attnres_block_scores returned %d\n", (int)st); return 1; }
    st = attnres_block_sums(srcs, D, d_zb, L, n, T, (int32_t)D, d_U, T * D, D, ATTNRES_U_F32, NULL);
    if (st != ATTNRES_OK) { fprintf(stderr, "attnres_block_sums returned %d\n", (int)st); return 1; }
    st = attnres_fwd_merged(d_U + (size_t)l * T * D, D, ATTNRES_U_F32, srcs[n], D, NULL, NULL, d_zb + (size_t)l * T * n,
                            d_rb, d_W + (size_t)l * D, eps, N, T, (int32_t)D, d_out3, d_rstd3, d_alpha3, NULL);
    if (st != ATTNRES_OK) { fprintf(stderr, "attnres_fwd_merged returned %d\n", (int)st); return 1; }
    st = attnres_block_sums(srcs, D, d_zb, L, n, T, (int32_t)D, d_U, D, D, ATTNRES_U_F32, NULL);  /* rows would collide */
    if (st != ATTNRES_ERR_INVALID_ARGUMENT) { fprintf(stderr, "colliding U rows not refused (%d)\n", (int)st); ++fails; }
    st = attnres_block_sums(srcs, D, d_zb, L, n, T, (int32_t)D, d_U, T * D, D, 2, NULL);  /* no such format */
    if (st != ATTNRES_ERR_INVALID_ARGUMENT) { fprintf(stderr, "U format 2 not refused (%d)\n", (int)st); ++fails; }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out, d_out3, nTD * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(rstd, d_rstd3, nTN * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(alpha, d_alpha3, nTN * 4, hipMemcpyDeviceToHost));
    oracle_fwd(N, T, D, src, W + (size_t)l * D, eps, r_out, r_rstd, r_alpha);
    double a3 = 0, r3 = 0;
    for (size_t i = 0; i < nTN; ++i) {
      a3 = fmax(a3, fabs((double)alpha[i] - r_alpha[i]));
      r3 = fmax(r3, fabs((double)rstd[i] / r_rstd[i] - 1.0));
    }
    const double o3 = rel_l2_bf16(out, r_out, nTD);
    printf("block route (scores, sums, merged forward): out rel_l2 %.3e  alpha max abs %.3e  rstd max rel %.3e\n", o3,
           a3, r3);
    if (!(o3 <= 5e-3 && a3 <= 1e-5 && r3 <= 1e-5)) ++fails;

    /* the same route with U in the 24-bit format: its bytes are the fp32 sums rounded to nearest even at bit 8 */
    uint8_t* d_U24;
    const size_t nU = (size_t)L * T * D;
    CHECK_HIP(hipMalloc((void**)&d_U24, nU * 3));
    st = attnres_block_sums(srcs, D, d_zb, L, n, T, (int32_t)D, d_U24, T * D, D, ATTNRES_U_F24, NULL);
    if (st != ATTNRES_OK) { fprintf(stderr, "attnres_block_sums (F24) returned %d\n", (int)st); return 1; }
    st = attnres_fwd_merged(d_U24 + (size_t)l * T * D * 3, D, ATTNRES_U_F24, srcs[n], D, NULL, NULL,
                            d_zb + (size_t)l * T * n, d_rb, d_W + (size_t)l * D, eps, N, T, (int32_t)D, d_out3, d_rstd3,
                            d_alpha3, NULL);
    if (st != ATTNRES_OK) { fprintf(stderr, "attnres_fwd_merged (F24) returned %d\n", (int)st); return 1; }
    CHECK_HIP(hipDeviceSynchronize());
    uint32_t* u32 = malloc(nU * 4);
    uint8_t* u24 = malloc(nU * 3);
    CHECK_HIP(hipMemcpy(u32, d_U, nU * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(u24, d_U24, nU * 3, hipMemcpyDeviceToHost));
    size_t bad24 = 0;
    for (size_t i = 0; i < nU; ++i) {
      const uint32_t b = u32[i], r = b + 0x7Fu + ((b >> 8) & 1u);
      if (u24[3 * i] != ((r >> 8) & 0xFF) || u24[3 * i + 1] != ((r >> 16) & 0xFF) || u24[3 * i + 2] != (r >> 24)) ++bad24;
    }
    CHECK_HIP(hipMemcpy(out, d_out3, nTD * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(alpha, d_alpha3, nTN * 4, hipMemcpyDeviceToHost));
    double a4 = 0;
    for (size_t i = 0; i < nTN; ++i) a4 = fmax(a4, fabs((double)alpha[i] - r_alpha[i]));
    const double o4 = rel_l2_bf16(out, r_out, nTD);
    printf("block route with 24-bit U: %zu of %zu elements differ from the rounded fp32 sums; out rel_l2 %.3e  "
           "alpha max abs %.3e\n", bad24, nU, o4, a4);
    if (!(bad24 == 0 && o4 <= 5e-3 && a4 <= 1e-5)) ++fails;
    free(u32);
    free(u24);
  }
  return fails == 0 ? 0 : 1;
}
