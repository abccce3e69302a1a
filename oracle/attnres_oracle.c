/*
 * fp64 CPU oracle for the Attention Residuals operator -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The HIP library never calls it and shares no code with
 * it.  It is plain on purpose: one token at a time, straight loops in double,
 * no blocking, no fusion and no reordering beyond what the formula states.
 *
 * What it computes (the formula box of the architecture figure in "Kimi K3
 * 模型结构（10）：RL 与服务中的状态管理": the weights over the depth sources are
 * softmax(w_l . RMSNorm(sources)), and the operator returns the weighted sum of
 * the sources, scored with the sub-layer's pseudo-query w_l).  For one token
 * with sources x_0 .. x_{N-1} (each of length D):
 *
 *   ms_i    = (1/D) sum_d x_id^2
 *   r_i     = 1 / sqrt(ms_i + eps)                 RMSNorm, no gain
 *   z_i     = sum_d w_d (r_i x_id)                 score of source i
 *   alpha_i = exp(z_i - max_j z_j) / sum_k exp(z_k - max_j z_j)
 *   out_d   = sum_i alpha_i x_id                   raw (un-normalised) sources
 *
 * The backward pass is the chain rule of the above for the loss
 * L = sum_d g_d out_d (g = dout):
 *
 *   da_i  = sum_d g_d x_id
 *   s     = sum_i alpha_i da_i
 *   dz_i  = alpha_i (da_i - s)                     softmax Jacobian
 *         = alpha_i sum_j alpha_j (da_i - da_j)    (the weights sum to 1)
 *   dx_id = alpha_i g_d + dz_i r_i (w_d - z_i r_i x_id / D)
 *   dw_d  = sum over tokens and sources of dz_i r_i x_id
 *
 * Readings where the pages are silent: the normalisation has no learnable
 * gain, eps sits inside the square root and the mean is over D, the score has
 * no temperature, and the weighted sum uses the raw sources.
 *
 * Layout: sources are source-major [N][T][D]; out, dout are [T][D]; rstd and
 * alpha are token-major [T][N]; dx is [N][T][D]; dw is [D].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Tokens whose dw contributions are summed together before the chunks are
 * added in chunk order; fixed, so dw does not depend on the thread count. */
#define DW_CHUNK 32

/* ---- one token ---------------------------------------------------------- */

/* x[i] points at source i's row for this token. */
static void token_forward(int N, int64_t D, const double* const* x, const double* w, double eps, double* out,
                          double* r, double* z, double* alpha) {
  for (int i = 0; i < N; ++i) {
    double ss = 0.0;
    for (int64_t d = 0; d < D; ++d) ss += x[i][d] * x[i][d];
    r[i] = 1.0 / sqrt(ss / (double)D + eps);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += w[d] * (r[i] * x[i][d]);
    z[i] = dot;
  }
  double m = z[0];
  for (int i = 1; i < N; ++i)
    if (z[i] > m) m = z[i];
  double den = 0.0;
  for (int i = 0; i < N; ++i) den += exp(z[i] - m);
  for (int i = 0; i < N; ++i) alpha[i] = exp(z[i] - m) / den;
  for (int64_t d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int i = 0; i < N; ++i) acc += alpha[i] * x[i][d];
    out[d] = acc;
  }
}

static void token_backward(int N, int64_t D, const double* const* x, const double* w, double eps, const double* g,
                           double* const* dx, double* dw) {
  double r[16], z[16], alpha[16], da[16], dz[16];
  double* out = (double*)malloc(sizeof(double) * (size_t)D);
  token_forward(N, D, x, w, eps, out, r, z, alpha);
  free(out);
  for (int i = 0; i < N; ++i) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += g[d] * x[i][d];
    da[i] = acc;
  }
  /* the softmax Jacobian in its second form above: when one weight is within
   * a rounding of 1, da_i - s for that source lies below the rounding of da_i
   * and the first form returns 0 for it, while this one keeps its value */
  for (int i = 0; i < N; ++i) {
    double acc = 0.0;
    for (int j = 0; j < N; ++j) acc += alpha[j] * (da[i] - da[j]);
    dz[i] = alpha[i] * acc;
  }
  for (int i = 0; i < N; ++i)
    for (int64_t d = 0; d < D; ++d)
      dx[i][d] = alpha[i] * g[d] + dz[i] * r[i] * (w[d] - z[i] * r[i] * x[i][d] / (double)D);
  for (int i = 0; i < N; ++i)
    for (int64_t d = 0; d < D; ++d) dw[d] += dz[i] * r[i] * x[i][d];
}

/* ---- fp64 inputs -------------------------------------------------------- */

/* x: [N][T][D]; out: [T][D]; rstd, alpha: [T][N] (either may be NULL). */
void oracle_fwd_f64(int N, int64_t T, int64_t D, const double* x, const double* w, double eps, double* out,
                    double* rstd, double* alpha) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    const double* rows[16];
    double r[16], z[16], a[16];
    for (int i = 0; i < N; ++i) rows[i] = x + ((int64_t)i * T + t) * D;
    token_forward(N, D, rows, w, eps, out + t * D, r, z, a);
    for (int i = 0; i < N; ++i) {
      if (rstd) rstd[t * N + i] = r[i];
      if (alpha) alpha[t * N + i] = a[i];
    }
  }
}

/* x, dx: [N][T][D]; g: [T][D]; dw: [D] (overwritten with the sum over all T tokens). */
void oracle_bwd_f64(int N, int64_t T, int64_t D, const double* x, const double* w, double eps, const double* g,
                    double* dx, double* dw) {
  const int64_t nchunk = (T + DW_CHUNK - 1) / DW_CHUNK;
  double* part = (double*)calloc((size_t)(nchunk > 0 ? nchunk : 1) * (size_t)D, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < nchunk; ++c) {
    const int64_t t1 = (c + 1) * DW_CHUNK < T ? (c + 1) * DW_CHUNK : T;
    for (int64_t t = c * DW_CHUNK; t < t1; ++t) {
      const double* rows[16];
      double* drows[16];
      for (int i = 0; i < N; ++i) {
        rows[i] = x + ((int64_t)i * T + t) * D;
        drows[i] = dx + ((int64_t)i * T + t) * D;
      }
      token_backward(N, D, rows, w, eps, g + t * D, drows, part + c * D);
    }
  }
  for (int64_t d = 0; d < D; ++d) dw[d] = 0.0;
  for (int64_t c = 0; c < nchunk; ++c)
    for (int64_t d = 0; d < D; ++d) dw[d] += part[c * D + d];
  free(part);
}

/* ---- bf16 / fp32 inputs, widened exactly to fp64 ------------------------ */

static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static void widen_token(int N, int64_t T, int64_t D, const uint16_t* src, int64_t t, double* buf, double** rows) {
  for (int i = 0; i < N; ++i) {
    rows[i] = buf + (int64_t)i * D;
    const uint16_t* s = src + ((int64_t)i * T + t) * D;
    for (int64_t d = 0; d < D; ++d) rows[i][d] = bf16_to_f64(s[d]);
  }
}

/* src: bf16 bits [N][T][D]; w: fp32 [D].  Outputs as in oracle_fwd_f64. */
void oracle_fwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, double* out,
                double* rstd, double* alpha) {
  double* wd = (double*)malloc(sizeof(double) * (size_t)D);
  for (int64_t d = 0; d < D; ++d) wd[d] = (double)w[d];
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)N * (size_t)D);
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      double* rows[16];
      double r[16], z[16], a[16];
      widen_token(N, T, D, src, t, buf, rows);
      token_forward(N, D, (const double* const*)rows, wd, eps, out + t * D, r, z, a);
      for (int i = 0; i < N; ++i) {
        if (rstd) rstd[t * N + i] = r[i];
        if (alpha) alpha[t * N + i] = a[i];
      }
    }
    free(buf);
  }
  free(wd);
}

/* src: bf16 bits [N][T][D]; dout: bf16 bits [T][D]; dx: fp64 [N][T][D] (may be
 * NULL to compute dw only); dw: fp64 [D]. */
void oracle_bwd(int N, int64_t T, int64_t D, const uint16_t* src, const float* w, double eps, const uint16_t* dout,
                double* dx, double* dw) {
  const int64_t nchunk = (T + DW_CHUNK - 1) / DW_CHUNK;
  double* part = (double*)calloc((size_t)(nchunk > 0 ? nchunk : 1) * (size_t)D, sizeof(double));
  double* wd = (double*)malloc(sizeof(double) * (size_t)D);
  for (int64_t d = 0; d < D; ++d) wd[d] = (double)w[d];
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)(N + 1) * (size_t)D);
    double* dbuf = (double*)malloc(sizeof(double) * (size_t)N * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < nchunk; ++c) {
      const int64_t t1 = (c + 1) * DW_CHUNK < T ? (c + 1) * DW_CHUNK : T;
      for (int64_t t = c * DW_CHUNK; t < t1; ++t) {
        double* rows[16];
        double* drows[16];
        widen_token(N, T, D, src, t, buf, rows);
        double* g = buf + (int64_t)N * D;
        for (int64_t d = 0; d < D; ++d) g[d] = bf16_to_f64(dout[t * D + d]);
        for (int i = 0; i < N; ++i) drows[i] = dx ? dx + ((int64_t)i * T + t) * D : dbuf + (int64_t)i * D;
        token_backward(N, D, (const double* const*)rows, wd, eps, g, drows, part + c * D);
      }
    }
    free(buf);
    free(dbuf);
  }
  for (int64_t d = 0; d < D; ++d) dw[d] = 0.0;
  for (int64_t c = 0; c < nchunk; ++c)
    for (int64_t d = 0; d < D; ++d) dw[d] += part[c * D + d];
  free(part);
  free(wd);
}

/* ---- block-batched scores ----------------------------------------------- */
/* The architecture figure of "Kimi K3 模型结构（10）：RL 与服务中的状态管理" groups
 * every 12 layers into one AttnRes block and puts the same set of sources
 * before every alpha of a block: the embedding and the completed block sums
 * do not change while a block runs, only the current partial sum does, and
 * each sub-layer has its own pseudo-query.  So for those n sources the RMS
 * statistic is the same for all L sub-layers of the block, and the L scores of
 * each source can be formed together:
 *
 *   rb_ti      = 1 / sqrt(mean_d x_tid^2 + eps)
 *   zb_{l,t,i} = sum_d W_ld (rb_ti x_tid)
 *
 * src: bf16 bits [n][T][D]; W: fp32 [L][D] (row l = sub-layer l's
 * pseudo-query); rstd: [T][n]; z: [L][T][n]. */
void oracle_block_scores(int n, int64_t T, int64_t D, int L, const uint16_t* src, const float* W, double eps,
                         double* rstd, double* z) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const uint16_t* row = src + ((int64_t)i * T + t) * D;
      double sq = 0.0;
      for (int64_t d = 0; d < D; ++d) sq += bf16_to_f64(row[d]) * bf16_to_f64(row[d]);
      const double rb = 1.0 / sqrt(sq / (double)D + eps);
      rstd[t * n + i] = rb;
      for (int l = 0; l < L; ++l) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += (double)W[(int64_t)l * D + d] * (rb * bf16_to_f64(row[d]));
        z[((int64_t)l * T + t) * n + i] = acc;
      }
    }
  }
}

/* The forward of one sub-layer whose first N-1 sources were scored by
 * oracle_block_scores: their rstd and this sub-layer's scores are given, and
 * only the last source -- the current block's partial sum -- is normalised
 * and scored here with the sub-layer's w; then the softmax over all N scores
 * and the weighted sum of all N raw sources, as in the plain forward.
 * src: bf16 bits [N][T][D] (all N sources, the partial sum last);
 * zg, rg: [T][N-1] given scores and rstd; outputs as oracle_fwd. */
void oracle_fwd_scored(int N, int64_t T, int64_t D, const uint16_t* src, const double* zg, const double* rg,
                       const float* w, double eps, double* out, double* rstd, double* alpha) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    double zs[16], rs[16], as[16];
    for (int i = 0; i + 1 < N; ++i) {
      zs[i] = zg[t * (N - 1) + i];
      rs[i] = rg[t * (N - 1) + i];
    }
    const uint16_t* last = src + ((int64_t)(N - 1) * T + t) * D;
    double sq = 0.0;
    for (int64_t d = 0; d < D; ++d) sq += bf16_to_f64(last[d]) * bf16_to_f64(last[d]);
    rs[N - 1] = 1.0 / sqrt(sq / (double)D + eps);
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += (double)w[d] * (rs[N - 1] * bf16_to_f64(last[d]));
    zs[N - 1] = acc;
    double top = zs[0];
    for (int i = 1; i < N; ++i)
      if (zs[i] > top) top = zs[i];
    double sum = 0.0;
    for (int i = 0; i < N; ++i) sum += exp(zs[i] - top);
    for (int i = 0; i < N; ++i) as[i] = exp(zs[i] - top) / sum;
    for (int64_t d = 0; d < D; ++d) {
      double o = 0.0;
      for (int i = 0; i < N; ++i) o += as[i] * bf16_to_f64(src[((int64_t)i * T + t) * D + d]);
      out[t * D + d] = o;
    }
    for (int i = 0; i < N; ++i) {
      rstd[t * N + i] = rs[i];
      alpha[t * N + i] = as[i];
    }
  }
}

/* ---- block-batched shared sums ----------------------------------------- */
/* The weighted sum of a sub-layer is linear in the sources, and within a
 * block only the last source (the current partial sum) changes from one
 * sub-layer to the next (architecture figure of "Kimi K3 模型结构（10）：RL
 * 与服务中的状态管理").  So the part of sub-layer l's weighted sum that the n
 * shared sources contribute can be formed once for the whole block, from the
 * block-batched scores, up to the softmax normaliser, which also depends on
 * the partial sum's score:
 *
 *   m_{l,t}   = max_i zb_{l,t,i}
 *   U_{l,t,d} = sum_i exp(zb_{l,t,i} - m_{l,t}) x_tid        (raw sources)
 *
 * src: bf16 bits [n][T][D]; z: [L][T][n]; U: [L][T][D]. */
void oracle_block_sums(int n, int64_t T, int64_t D, int L, const uint16_t* src, const double* z, double* U) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    for (int l = 0; l < L; ++l) {
      const double* zt = z + ((int64_t)l * T + t) * n;
      double m = zt[0];
      for (int i = 1; i < n; ++i)
        if (zt[i] > m) m = zt[i];
      double* u = U + ((int64_t)l * T + t) * D;
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i) acc += exp(zt[i] - m) * bf16_to_f64(src[((int64_t)i * T + t) * D + d]);
        u[d] = acc;
      }
    }
  }
}

/* The forward of one sub-layer from its shared sum (oracle_block_sums) and
 * the current partial sum p, the last of its N sources.  The partial sum is
 * normalised and scored with the sub-layer's w as in the plain forward; the
 * other N-1 scores and rstd are given.  With M the largest of all N scores
 * and m the largest of the N-1 given ones:
 *
 *   den     = sum_i exp(z_i - M)                  over all N sources
 *   alpha_i = exp(z_i - M) / den
 *   out_d   = (exp(m - M) U_d + exp(z_p - M) p_d) / den
 *
 * which is the plain forward's weighted sum, as exp(m - M) exp(z_i - m) =
 * exp(z_i - M) for every shared source.
 * U: [T][D] (the sub-layer's rows of the shared sum); p: bf16 bits [T][D];
 * zg, rg: [T][N-1]; outputs as oracle_fwd. */
void oracle_fwd_merged(int N, int64_t T, int64_t D, const double* U, const uint16_t* p, const double* zg,
                       const double* rg, const float* w, double eps, double* out, double* rstd, double* alpha) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    double zs[16], rs[16];
    for (int i = 0; i + 1 < N; ++i) {
      zs[i] = zg[t * (N - 1) + i];
      rs[i] = rg[t * (N - 1) + i];
    }
    const uint16_t* pt = p + t * D;
    double sq = 0.0;
    for (int64_t d = 0; d < D; ++d) sq += bf16_to_f64(pt[d]) * bf16_to_f64(pt[d]);
    rs[N - 1] = 1.0 / sqrt(sq / (double)D + eps);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += (double)w[d] * (rs[N - 1] * bf16_to_f64(pt[d]));
    zs[N - 1] = dot;
    double m = zs[0];
    for (int i = 1; i + 1 < N; ++i)
      if (zs[i] > m) m = zs[i];
    const double top = zs[N - 1] > m ? zs[N - 1] : m;
    double den = 0.0;
    for (int i = 0; i < N; ++i) den += exp(zs[i] - top);
    const double shared = exp(m - top), own = exp(zs[N - 1] - top);
    for (int64_t d = 0; d < D; ++d) out[t * D + d] = (shared * U[t * D + d] + own * bf16_to_f64(pt[d])) / den;
    for (int i = 0; i < N; ++i) {
      rstd[t * N + i] = rs[i];
      alpha[t * N + i] = exp(zs[i] - top) / den;
    }
  }
}

/* ---- partial-sum update ------------------------------------------------- */
/* The architecture figure of "Kimi K3 模型结构（10）：RL 与服务中的状态管理" lists
 * the current block's partial sum (the sum of the sub-layer outputs already
 * computed in the block) as one of the depth sources.  Adding a sub-layer
 * output y to a partial sum p held in bf16 stores the exact value p + y
 * rounded once to the nearest bf16, ties to even.  When the block is complete
 * the same sum is the block's entry among the completed-block sources. */

/* Round a double to the nearest bf16 (8 significant bits, float's exponent
 * range, subnormals included), ties to even; returns the bit pattern. */
static uint16_t f64_to_bf16_rne(double v) {
  if (v != v) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  const double m = frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1: leading bit has weight 2^(e-1) */
  int keep = 8;                  /* significant bits of a normal bf16 */
  if (e - 1 < -126) keep -= -126 - (e - 1); /* below the normal range: fixed quantum 2^-133 */
  const double q = nearbyint(ldexp(m, keep)); /* default rounding mode: nearest, ties to even */
  const double r = ldexp(q, e - keep);         /* a bf16 value, or 2^128 when it overflows */
  const float f = (float)r;                    /* exact; 2^128 becomes inf */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* out[k] = bf16(p[k] + y[k]) for k < n; all bf16 bit patterns.  The sum of two
 * doubles widened from bf16 is exact whenever it can matter: if the exponents
 * differ by more than 44 bits the smaller value is below half a bf16 unit of
 * the larger and the rounded result is the larger value either way. */
void oracle_add_bf16(int64_t n, const uint16_t* p, const uint16_t* y, uint16_t* out) {
  for (int64_t k = 0; k < n; ++k) out[k] = f64_to_bf16_rne(bf16_to_f64(p[k]) + bf16_to_f64(y[k]));
}

/* The block sums' 24-bit element format (the library's ATTNRES_U_F24, a
 * storage choice of the block-level route, not of the pages): a value rounded
 * to 16 significant bits, nearest, ties to even, in the fp32 exponent range
 * (below 2^-126 the quantum stays 2^-141, and values that round to 2^128
 * become infinity), stored as the upper three bytes of the rounded value's
 * fp32 bit pattern, least significant first.  The rounding is done on the
 * value, as f64_to_bf16_rne does for bf16, not on the bit pattern. */
void oracle_round24(int64_t n, const float* x, uint8_t* out) {
  for (int64_t k = 0; k < n; ++k) {
    const double v = (double)x[k];
    float f;
    if (v != v) {
      f = x[k];
    } else {
      const double a = fabs(v);
      double r = 0.0;
      if (a != 0.0) {
        int e;
        const double m = frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1 */
        int keep = 16;                 /* significant bits kept */
        if (e - 1 < -126) keep -= -126 - (e - 1);
        r = ldexp(nearbyint(ldexp(m, keep)), e - keep);
      }
      f = (float)(signbit(v) ? -r : r); /* exact; 2^128 becomes inf */
    }
    uint32_t u;
    memcpy(&u, &f, 4);
    out[3 * k] = (uint8_t)(u >> 8);
    out[3 * k + 1] = (uint8_t)(u >> 16);
    out[3 * k + 2] = (uint8_t)(u >> 24);
  }
}

/* The fp32 value of each 24-bit element: its three bytes as the upper bytes
 * of an fp32 bit pattern whose low byte is zero. */
void oracle_decode24(int64_t n, const uint8_t* in, float* out) {
  for (int64_t k = 0; k < n; ++k) {
    const uint32_t u = ((uint32_t)in[3 * k] << 8) | ((uint32_t)in[3 * k + 1] << 16) | ((uint32_t)in[3 * k + 2] << 24);
    memcpy(&out[k], &u, 4);
  }
}
