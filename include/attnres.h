/*
 * libattnres -- Attention Residuals (depth mixing) forward and backward on
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (formula box of the architecture figure in "Kimi K3 模型结构
 * （10）：RL 与服务中的状态管理"): before each sub-layer, every token mixes up to
 * nine depth sources -- the token embedding, the sum of each completed
 * 12-layer block, and the current block's partial sum -- with weights
 *
 *     alpha = softmax_i( w_l . RMSNorm(x_i) )
 *
 * where w_l is the sub-layer's learnable pseudo-query, and returns
 * out = sum_i alpha_i x_i.  Per token t and source i (D = hidden size):
 *
 *     rstd[t][i]  = 1 / sqrt( (1/D) sum_d x[i][t][d]^2 + eps )
 *     z_i         = rstd[t][i] * sum_d w[d] x[i][t][d]
 *     alpha[t][i] = exp(z_i - max_j z_j) / sum_k exp(z_k - max_j z_j)
 *     out[t][d]   = sum_i alpha[t][i] x[i][t][d]
 *
 * The normalisation has no gain and the weighted sum uses the raw sources.
 * The section on Attention Residuals in "Kimi K3 on Fireworks: Fast RL at
 * frontier scale" motivates fusing the normalisation and the weighted sum so
 * that no per-source intermediate reaches memory; these calls materialise
 * only out, rstd and alpha (forward) and dsources, dw (backward).
 *
 * Conventions for every call
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 as float; the
 *     block sums (attnres_block_sums) as void*, fp32 or 24-bit elements.
 *   - Layouts are row-major: stacked sources/dsources [N][T][D]
 *     (source-major), per-source rows with a pitch (see
 *     attnres_fwd_sources), out/dout [T][D], rstd/alpha [T][N]
 *     (token-major).
 *   - Every pointer is a device pointer owned by the caller (the per-source
 *     calls take a host array of device pointers).  The library allocates no
 *     device memory, frees nothing and never synchronises; its only state is
 *     a mutex-guarded host cache of kernel occupancy per device, the split
 *     backward's poll bound (attnres_set_split_spin, an atomic) and the static
 *     scratch array of attnres_bwd_noalloc, so calls are thread-safe and
 *     reentrant (apart from that array: see attnres_bwd_noalloc).  All work
 *     is enqueued on `stream`
 *     (a hipStream_t; NULL selects the null stream) and the call returns once
 *     the work is enqueued.
 *   - Outputs are overwritten, never accumulated (except by the
 *     accumulating modes of attnres_bwd_sources).  Inputs are not modified
 *     (except the partial sum that attnres_fwd_update or attnres_fwd_merged
 *     updates when partial_out is the partial sum itself).
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error the call returns a non-zero status and enqueues nothing.
 *   - Results for one token depend only on that token's inputs (and w): they
 *     are bitwise independent of T, of the token's position in the batch and
 *     of the run, for every call with the same (N, D).  dw is bitwise
 *     reproducible for a given (T, N, D).  (attnres_bwd_noalloc runs the
 *     one-token backward also where attnres_bwd runs the split one,
 *     ATTNRES_BWD_SPLIT; the two agree within rounding, not bit for bit.)
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTNRES_OK = 0,
  ATTNRES_ERR_INVALID_ARGUMENT = 1, /* bad size, null/misaligned/overlapping pointer, bad eps */
  ATTNRES_ERR_WORKSPACE = 2,        /* backward workspace missing or too small */
  ATTNRES_ERR_HIP = 3               /* the HIP runtime refused a launch */
} attnres_status;

/* At most nine depth sources per token (architecture figure, same page). */
#define ATTNRES_MAX_SOURCES 9
/* Largest hidden size the kernels accept (a row group lives on chip). */
#define ATTNRES_MAX_D 16384
/* Rows of dw partial sums the backward's final sum reads (P <= 256 of them,
 * at the start of the workspace): for the one-token backward, workgroup c of
 * P = min(T, 256) sums tokens c, c+P, c+2P, ...; for the split backward, fold
 * row b sums the 4-token spans b, b+P, b+2P, ... with P = min(spans, 256). */
#define ATTNRES_DW_PARTIALS 256
/* grad_mode flags of attnres_bwd_sources. */
#define ATTNRES_GRAD_BF16 0
#define ATTNRES_GRAD_ACCUMULATE 1
#define ATTNRES_GRAD_F32 2
/* The split backward spreads every token over ceil(D / 1024) workgroups, each
 * taking one 1024-channel slice of ATTNRES_SPLIT_TOKENS consecutive tokens side by
 * side (a span); the per-token sums are exchanged through a ring of
 * ATTNRES_SPLIT_RING tokens in the workspace, and every workgroup writes one dw
 * partial row slice.  The spans run in chunks of ATTNRES_SPLIT_CHUNK_SPANS, each
 * followed by a fold of its partial rows, so the workspace holds the partial rows of
 * one chunk.  It runs where it was measured faster on MI355X than the
 * one-token-per-workgroup backward: ATTNRES_BWD_SPLIT(N, D), i.e. D <= 1024, or
 * N >= 8 with D <= ATTNRES_SPLIT_MAX_D.  The choice depends on (N, D) only, so every
 * call with the same N and D uses the same reduction trees. */
#define ATTNRES_SPLIT_MAX_D 7168
#define ATTNRES_SPLIT_ANY_N_MAX_D 1024
#define ATTNRES_SPLIT_MIN_N 8
#define ATTNRES_BWD_SPLIT(N, D)                                                                                    \
  ((D) <= ATTNRES_SPLIT_ANY_N_MAX_D || ((N) >= ATTNRES_SPLIT_MIN_N && (D) <= ATTNRES_SPLIT_MAX_D))
#define ATTNRES_SPLIT_TOKENS 4
#define ATTNRES_SPLIT_RING 4096
#define ATTNRES_SPLIT_CHUNK_SPANS 8192
/* Polls of a member's ring word before the waiting workgroup recomputes that
 * member's partial sums itself (attnres_set_split_spin). */
#define ATTNRES_SPLIT_SPIN_DEFAULT 4096
/* Spans whose dw partial rows the split backward's workspace holds at once:
 * ceil(T / ATTNRES_SPLIT_TOKENS), at most one chunk. */
#define ATTNRES_SPLIT_PARTIAL_ROWS(T)                                                                              \
  ((((T) + ATTNRES_SPLIT_TOKENS - 1) / ATTNRES_SPLIT_TOKENS) < ATTNRES_SPLIT_CHUNK_SPANS                         \
       ? (((T) + ATTNRES_SPLIT_TOKENS - 1) / ATTNRES_SPLIT_TOKENS)                                               \
       : ATTNRES_SPLIT_CHUNK_SPANS)
/* Bytes of device workspace attnres_bwd / attnres_bwd_sources need for T
 * tokens, N sources and hidden size D: ATTNRES_DW_PARTIALS fp32 rows of D,
 * plus, where the split backward runs (ATTNRES_BWD_SPLIT), the exchange ring
 * (8-byte words) and ATTNRES_SPLIT_PARTIAL_ROWS(T) fp32 partial rows of D (at
 * T >= 32768, N = 9, D = 7168: 7.3 + 4.1 + 234.9 MB). */
#define ATTNRES_BWD_WORKSPACE_BYTES(T, N, D)                                                                       \
  ((size_t)ATTNRES_DW_PARTIALS * (size_t)(D) * sizeof(float) +                                                   \
   (ATTNRES_BWD_SPLIT(N, D)                                                                                      \
        ? (size_t)ATTNRES_SPLIT_RING * (size_t)(((D) + 1023) / 1024) * 2 * (size_t)(N) * 8 +                      \
              (size_t)ATTNRES_SPLIT_PARTIAL_ROWS(T) * (size_t)(D) * sizeof(float)                                \
        : 0))

/*
 * Forward.
 *   src   [N][T][D] bf16   depth sources, row (i, t) at src + (i*T + t)*D
 *   w     [D]       fp32   pseudo-query of this sub-layer
 *   eps             fp32   finite, >= 0; added to the mean square inside the root
 *                          (with eps == 0 an all-zero source row has rstd = inf
 *                          and makes that token's scores NaN, as the formula does)
 *   N               1 .. ATTNRES_MAX_SOURCES
 *   T               >= 0 tokens, T*N*D <= 2^40 (T == 0 enqueues nothing and
 *                   returns OK)
 *   D               8 .. ATTNRES_MAX_D, a multiple of 8
 *   out   [T][D]    bf16   sum_i alpha_i x_i, fp32-accumulated, rounded to nearest even
 *   rstd  [T][N]    fp32   saved for the backward pass
 *   alpha [T][N]    fp32   saved for the backward pass
 * Alignment: src, w, out 16-byte aligned; rstd, alpha 4-byte aligned.
 * Pointers other than w may be NULL when T == 0.  Outputs must not overlap
 * each other or the inputs.
 * Arithmetic is fp32 (sums of squares and dots of bf16 products): a row's sum
 * of squares must stay inside the fp32 range -- rms up to ~1e17 at D = 7168,
 * and with eps == 0 at least ~1e-19.
 */
attnres_status attnres_fwd(const uint16_t* src, const float* w, float eps, int32_t N, int64_t T, int32_t D,
                           uint16_t* out, float* rstd, float* alpha, void* stream);

/*
 * Backward of L = sum_{t,d} dout[t][d] * out[t][d]:
 *   dsrc[i][t][d] = alpha_i g_d + dz_i rstd_i (w_d - z_i rstd_i x_id / D)
 *   dw[d]         = sum over t and i of dz_i rstd_i x_id
 * with g = dout[t], da_i = g . x_i, dz_i = alpha_i (da_i - sum_j alpha_j da_j)
 * and z_i = rstd_i (w . x_i) recomputed from the sources (eps enters only
 * through the saved rstd).
 *   dout  [T][D]    bf16   output gradient
 *   src, w                 as passed to attnres_fwd
 *   rstd, alpha [T][N] fp32 as written by attnres_fwd for these inputs
 *   dsrc  [N][T][D] bf16   gradient of every source (overwritten)
 *   dw    [D]       fp32   gradient of w summed over all T tokens (overwritten;
 *                          zero-filled when T == 0)
 *   workspace              device scratch of at least
 *                          ATTNRES_BWD_WORKSPACE_BYTES(T, N, D) bytes, 16-byte
 *                          aligned; contents on entry are ignored and on exit
 *                          unspecified.  May be NULL when T == 0.  It holds the
 *                          call's dw partial rows and, for the split backward,
 *                          its exchange ring: calls that can run at the same
 *                          time (on different streams) need different
 *                          workspaces; calls in order on one stream can share
 *                          one.
 * Alignment: dout, src, w, dsrc, dw, workspace 16-byte aligned; rstd, alpha
 * 4-byte aligned.  dsrc, dw and the workspace must not overlap each other or
 * any input.  Status ATTNRES_ERR_WORKSPACE if the workspace is NULL or
 * smaller than required while T > 0.
 */
attnres_status attnres_bwd(const uint16_t* dout, const uint16_t* src, const float* w, const float* rstd,
                           const float* alpha, int32_t N, int64_t T, int32_t D, uint16_t* dsrc, float* dw,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward with the N sources given as N row sets instead of one stacked
 * [N][T][D] tensor -- the form a model holds them in: the embedding, each
 * completed block sum and the current partial sum (architecture figure of
 * "Kimi K3 模型结构（10）") live in their own buffers, or side by side in one
 * depth-source cache, and stacking them would cost a copy of N*T*D values per
 * sub-layer.
 *   srcs       host array of N device pointers; row t of source i starts at
 *              srcs[i] + t*src_pitch (bf16 elements), 16-byte aligned.  A
 *              pointer may appear more than once.  May be NULL when T == 0.
 *   src_pitch  elements between consecutive tokens' rows: D for separate
 *              [T][D] buffers; N*D with srcs[i] = base + i*D for a cache
 *              interleaved by token ([T][N][D]).  A multiple of 8, >= D.
 * Everything else as attnres_fwd.  Results are bitwise identical to
 * attnres_fwd on the same rows stacked.
 */
attnres_status attnres_fwd_sources(const uint16_t* const* srcs, int64_t src_pitch, const float* w, float eps,
                                   int32_t N, int64_t T, int32_t D, uint16_t* out, float* rstd, float* alpha,
                                   void* stream);

/*
 * Forward for decoding and rollout: the per-source forward with the saved
 * state made optional, for callers that will not run a backward pass (the
 * rollout side of the RL loop in the determinism section of "Kimi K3 on
 * Fireworks: Fast RL at frontier scale").  It runs the same one-workgroup-
 * per-token kernel as attnres_fwd, so every output is bitwise the one the
 * training forward gives for that token in any batch: rollout and training
 * see the same numbers.  A single token costs 5-7 us of kernel time on
 * MI355X (D = 7168, N = 9; sources in cache or in HBM).
 *   srcs, src_pitch, w, eps, N, T, D, out   as attnres_fwd_sources.
 *   rstd, alpha   [T][N] fp32 saved state as attnres_fwd, or both NULL: then
 *                 only out is written.  Exactly one of them NULL is
 *                 ATTNRES_ERR_INVALID_ARGUMENT.
 */
attnres_status attnres_fwd_decode(const uint16_t* const* srcs, int64_t src_pitch, const float* w, float eps,
                                  int32_t N, int64_t T, int32_t D, uint16_t* out, float* rstd, float* alpha,
                                  void* stream);

/*
 * Forward fused with the update of the current block's partial sum.  The
 * depth sources of a sub-layer are the embedding, the completed block sums
 * and the current block's partial sum -- the sum of the sub-layer outputs
 * already computed in the block (architecture figure of "Kimi K3
 * 模型结构（10）：RL 与服务中的状态管理").  After each sub-layer its output y is
 * added to that partial sum; this call does the addition while reading the
 * sources for the next sub-layer's operator, instead of in a separate pass:
 *   partial_out = bf16(partial + delta)   exact sum, rounded once to nearest
 *                                         even (also the completed block sum
 *                                         when delta is the block's last
 *                                         sub-layer output)
 *   then the forward of attnres_fwd_sources on {srcs[0..N-2], partial_out}.
 * Bytes per token drop from 2ND + 2D + 8N (+ 6D for a separate update pass)
 * to 2(N+1)D + 4D + 8N.
 *   srcs         host array of the N-1 other sources (device pointers); may
 *                be NULL when N == 1.
 *   src_pitch    as attnres_fwd_sources; it also applies to partial and
 *                partial_out (the partial sum is one of the sources).
 *   partial      partial sum before the update (rows of D bf16 values).
 *   delta        [T][D] bf16 (dense) sub-layer output to add.
 *   partial_out  updated partial sum; may be `partial` itself (in-place
 *                update), otherwise it must not overlap any input.
 *   out, rstd, alpha, w, eps, N (total sources, partial included), T, D
 *                as attnres_fwd_decode (rstd and alpha both NULL when no
 *                backward follows).
 * The backward is attnres_bwd_sources with partial_out as the last source;
 * the gradient of partial_out then flows unchanged to both partial and delta.
 */
attnres_status attnres_fwd_update(const uint16_t* const* srcs, int64_t src_pitch, const uint16_t* partial,
                                  const uint16_t* delta, const float* w, float eps, int32_t N, int64_t T, int32_t D,
                                  uint16_t* partial_out, uint16_t* out, float* rstd, float* alpha, void* stream);

/*
 * Backward with per-source row sets, writing or accumulating the source
 * gradients in bf16 or fp32.  A completed block sum is a source of every
 * later sub-layer's operator, so its gradient is the sum of those operators'
 * contributions:
 *   srcs, src_pitch   as attnres_fwd_sources.
 *   dsrcs       host array of N device pointers to the gradients, row t of
 *               gradient i at dsrcs[i] + t*dsrc_pitch elements (bf16 or
 *               fp32 as grad_mode says; the same choices of layout as the
 *               sources), pairwise disjoint and disjoint from every input.
 *   grad_mode   ATTNRES_GRAD_BF16 (0): dsrcs[i] = bf16(dx_i), bitwise what
 *                 attnres_bwd writes;
 *               ATTNRES_GRAD_ACCUMULATE (1): dsrcs[i] = bf16(dsrcs[i] + dx_i),
 *                 the sum formed in fp32 and rounded once to nearest even;
 *               ATTNRES_GRAD_F32 (2): dsrcs[i] = dx_i in fp32 (no rounding
 *                 to bf16);
 *               ATTNRES_GRAD_F32 | ATTNRES_GRAD_ACCUMULATE (3): fp32
 *                 gradients, dsrcs[i] += dx_i in fp32.
 *               Each gradient element is read (when accumulating) and
 *               written once.  Other values: ATTNRES_ERR_INVALID_ARGUMENT.
 * dw is always overwritten with this call's sum over the T tokens.  Other
 * arguments as attnres_bwd.  srcs and dsrcs may be NULL when T == 0.
 */
attnres_status attnres_bwd_sources(const uint16_t* dout, const uint16_t* const* srcs, int64_t src_pitch,
                                   const float* w, const float* rstd, const float* alpha, int32_t N, int64_t T,
                                   int32_t D, void* const* dsrcs, int64_t dsrc_pitch, int32_t grad_mode, float* dw,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-batched scores.  Every 12 layers form one AttnRes block, and the same
 * set of sources stands before every alpha of the block: the embedding and
 * the completed block sums do not change while the block runs (only the
 * current partial sum does), and each sub-layer has its own pseudo-query w_l
 * (architecture figure of "Kimi K3 模型结构（10）：RL 与服务中的状态管理").  For
 * those n sources this call forms, in one pass over them, their rstd and the
 * scores of all L pseudo-queries of the block:
 *     rstd[t][i]  = 1 / sqrt(mean_d x[i][t][d]^2 + eps)
 *     z[l][t][i]  = rstd[t][i] * sum_d W[l][d] x[i][t][d]
 * Each sub-layer's forward then takes its slice z[l] through
 * attnres_fwd_scored and reduces only the partial sum.  The product
 * [T*n x D] . [D x L] runs on the matrix cores (bf16 MFMA on an exact
 * three-part bf16 split of each fp32 pseudo-query, fp32 accumulation).
 *   srcs, src_pitch  the n sources as in attnres_fwd_sources (src_pitch <=
 *                    2^24 elements).
 *   W      [L][D] fp32   the block's pseudo-queries, 16-byte aligned
 *   L      1 .. ATTNRES_MAX_QUERIES
 *   eps, T, D        as attnres_fwd; n = 1 .. ATTNRES_MAX_SOURCES
 *   rstd   [T][n] fp32, z [L][T][n] fp32   outputs (4-byte aligned)
 *   workspace        at least ATTNRES_BLOCK_SCORES_WORKSPACE_BYTES(L, D)
 *                    bytes of device scratch, 16-byte aligned (the split
 *                    queries); contents on entry ignored, on exit unspecified.
 * Outputs and workspace must not overlap each other or any input.  T == 0:
 * nothing is enqueued.  Results are within fp32 rounding of the forward's own
 * rstd and scores (the summation order differs), not bitwise equal to them.
 */
#define ATTNRES_MAX_QUERIES 64
#define ATTNRES_BLOCK_SCORES_WORKSPACE_BYTES(L, D) \
  ((size_t)3 * (size_t)(((L) + 15) / 16 * 16) * (size_t)(((D) + 31) / 32 * 32) * 2)
attnres_status attnres_block_scores(const uint16_t* const* srcs, int64_t src_pitch, const float* W, int32_t L,
                                    float eps, int32_t n, int64_t T, int32_t D, float* rstd, float* z,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward of one sub-layer from block-batched scores: the first N-1 sources
 * are the block's shared sources, whose rstd and this sub-layer's scores come
 * from attnres_block_scores (rstd_given = its rstd, z_given = its z + l*T*(N-1)
 * for sub-layer l, both [T][N-1] fp32, 4-byte aligned); the last source is the
 * current block's partial sum, normalised and scored here with w.  Then the
 * softmax over all N scores and the weighted sum of all N raw sources, as
 * attnres_fwd_sources (same outputs; rstd[t][i] = rstd_given[t][i] for
 * i < N-1).  N = 2 .. ATTNRES_MAX_SOURCES; other arguments as
 * attnres_fwd_sources.  The backward is attnres_bwd_sources with these
 * outputs.
 */
attnres_status attnres_fwd_scored(const uint16_t* const* srcs, int64_t src_pitch, const float* z_given,
                                  const float* rstd_given, const float* w, float eps, int32_t N, int64_t T, int32_t D,
                                  uint16_t* out, float* rstd, float* alpha, void* stream);

/*
 * Block-batched shared sums.  The weighted sum is linear in the sources, and
 * while a block runs only its last source, the current partial sum, changes
 * from one sub-layer to the next (architecture figure of "Kimi K3
 * 模型结构（10）：RL 与服务中的状态管理").  So the part of sub-layer l's weighted
 * sum that the n shared sources contribute is formed here for all L
 * sub-layers in one pass over them, from the scores of attnres_block_scores,
 * up to the softmax normaliser:
 *     m[l][t]    = max_i z[l][t][i]
 *     U[l][t][d] = sum_i exp(z[l][t][i] - m[l][t]) x[i][t][d]       (fp32)
 * and each sub-layer's forward then runs attnres_fwd_merged, which reads its
 * U rows and the partial sum instead of all N source rows.
 * U is stored in one of two element formats (u_format):
 *   ATTNRES_U_F32  fp32, 4 bytes per element;
 *   ATTNRES_U_F24  the fp32 sum rounded to nearest even on a 16-bit
 *                  significand (fp32 exponent range), kept as the upper three
 *                  bytes of its fp32 bit pattern, little-endian, 3 bytes per
 *                  element: element k of a row occupies bytes 3k .. 3k+2 and
 *                  its value is the fp32 number whose bit pattern is
 *                  byte[3k] << 8 | byte[3k+1] << 16 | byte[3k+2] << 24.
 *                  A quarter less traffic for the sums and the merged
 *                  forward; the relative error of an element is at most
 *                  2^-16 (1/128 of a bf16 unit in the last place).
 *   srcs, src_pitch  the n shared sources as in attnres_block_scores
 *                    (n = 1 .. ATTNRES_MAX_SOURCES)
 *   z      [L][T][n] fp32, 4-byte aligned: attnres_block_scores' z (any
 *          finite scores)
 *   L      1 .. ATTNRES_MAX_QUERIES; T, D as attnres_fwd
 *   U      output, 16-byte (ATTNRES_U_F32) or 4-byte (ATTNRES_U_F24)
 *          aligned: row (l, t) of D elements at element offset
 *          l*u_lstride + t*u_pitch.  u_lstride and u_pitch are
 *          multiples of 4, at least D, and lay the rows out sub-layer-major
 *          (u_lstride >= (T-1)*u_pitch + D, e.g. u_lstride = T*D, u_pitch = D)
 *          or token-major (u_pitch >= (L-1)*u_lstride + D, e.g. u_lstride =
 *          D, u_pitch = L*D); other layouts are rejected.  L*T*D*4 (F32) or
 *          L*T*D*3 (F24) bytes in the dense layouts.
 *   u_format  ATTNRES_U_F32 or ATTNRES_U_F24; anything else is rejected.
 * U must not overlap the sources or z.  T == 0: nothing is enqueued.  The
 * weights are fp32 (exp on the hardware exp2), the sums fp32 in source order.
 */
#define ATTNRES_U_F32 0
#define ATTNRES_U_F24 1
attnres_status attnres_block_sums(const uint16_t* const* srcs, int64_t src_pitch, const float* z, int32_t L,
                                  int32_t n, int64_t T, int32_t D, void* U, int64_t u_lstride, int64_t u_pitch,
                                  int32_t u_format, void* stream);

/*
 * Forward of one sub-layer from its block-batched shared sum: U holds the
 * sub-layer's rows of attnres_block_sums in the format u_format (its element
 * offset l*u_lstride for sub-layer l; row t at a further t*u_pitch elements;
 * u_pitch a multiple of 4, >= D; base aligned as for attnres_block_sums),
 * partial [T][D] bf16 (row pitch partial_pitch, a multiple of
 * 8 elements, 16-byte aligned) the current partial sum, the last of the N
 * sources.  z_given and rstd_given ([T][N-1] fp32, 4-byte aligned) are the
 * shared sources' scores for this sub-layer and their rstd, as for
 * attnres_fwd_scored (z + l*T*(N-1) and rstd of attnres_block_scores).  The
 * partial sum is normalised and scored with w, the softmax runs over all N
 * scores as in attnres_fwd_scored (rstd and alpha within fp32 rounding of
 * that call's: the partial sum's dots are summed in another order), and with
 * m the largest given score and M the largest of all,
 *     out = exp(m - M) / den * U + alpha[N-1] * partial
 * which is the weighted sum of all N sources to within fp32 rounding.
 * N = 2 .. ATTNRES_MAX_SOURCES; w, eps, T, D, out, rstd, alpha as
 * attnres_fwd_sources.  Outputs must not overlap any input or each other.
 *   delta, partial_out  both NULL, or the fused partial-sum update of
 *               attnres_fwd_update: delta [T][D] bf16 (dense, 16-byte
 *               aligned) is added to the partial sum first, partial_out =
 *               bf16(partial + delta) (rounded once, ties to even; row pitch
 *               partial_pitch; may be `partial` itself, else disjoint from
 *               every input), and the forward then uses partial_out as the
 *               last source.
 * The backward is attnres_bwd_sources on all N sources (partial_out as the
 * last, when updated) with these outputs.
 */
attnres_status attnres_fwd_merged(const void* U, int64_t u_pitch, int32_t u_format, const uint16_t* partial,
                                  int64_t partial_pitch,
                                  const uint16_t* delta, uint16_t* partial_out, const float* z_given,
                                  const float* rstd_given, const float* w, float eps, int32_t N, int64_t T, int32_t D,
                                  uint16_t* out, float* rstd, float* alpha, void* stream);

/*
 * Backward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, contract and errors as attnres_bwd,
 * except that the dw partial rows live in a static device array of the
 * library (ATTNRES_DW_PARTIALS x ATTNRES_NOALLOC_MAX_D fp32 = 8 MiB on every
 * device the library runs on, held until the process ends), so this call
 * runs the one-token-per-workgroup backward, whose partial rows fit that
 * array, also where attnres_bwd splits tokens over workgroups: its dsrc and
 * dw equal attnres_bwd's to within fp32 rounding (another summation order),
 * not bit for bit.  The call allocates nothing (no hipMalloc, no library
 * routine that allocates).
 *   D > ATTNRES_NOALLOC_MAX_D   ATTNRES_ERR_WORKSPACE, nothing enqueued.
 * The first call on a device looks up that device's address of the array
 * (ATTNRES_ERR_HIP if the runtime refuses).  Every call on a device shares its
 * array: calls that overlap in time on one device (concurrent streams, or
 * host threads on different streams) race on it and may return wrong dw;
 * serialise them, or use attnres_bwd with a workspace per stream.  Nothing in
 * the array needs to start at zero: each call writes every partial row it
 * reads.
 */
#define ATTNRES_NOALLOC_MAX_D 8192
attnres_status attnres_bwd_noalloc(const uint16_t* dout, const uint16_t* src, const float* w, const float* rstd,
                                   const float* alpha, int32_t N, int64_t T, int32_t D, uint16_t* dsrc, float* dw,
                                   void* stream);

/*
 * Poll bound of the split backward (ATTNRES_BWD_SPLIT(N, D)): a workgroup
 * waiting for another slice's partial sums of a token reads that member's
 * ring word at most `polls` times, then recomputes the member's partial sums
 * from HBM itself, with the member's own arithmetic and reduction tree, so
 * dsrc and dw do not depend on which route was taken.  The route is taken
 * when the members of a token are not resident together (a device shared
 * with other work); polls = 0 takes it for every word, which makes the
 * backward slower (each slice workgroup then reads every slice of its
 * tokens) but still correct -- the way to exercise that route.
 * The bound applies to attnres_bwd / attnres_bwd_sources calls enqueued after
 * this call, in every thread; it returns the previous bound (default
 * ATTNRES_SPLIT_SPIN_DEFAULT).  It enqueues nothing and cannot fail.
 */
uint32_t attnres_set_split_spin(uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
