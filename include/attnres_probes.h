/*
 * libattnres_probes -- HBM bandwidth ceilings on MI355X (gfx950), measured
 * with access patterns and no arithmetic.  These kernels are not part of the
 * operator: the benchmark times them on the same device to state what the
 * memory system gives to (a) plain streams and (b) the operator's own access
 * patterns, so the operator's achieved bandwidth can be read against a
 * ceiling measured on the same box, next to the 8 TB/s peak.
 *
 * The Attention Residuals section of "Kimi K3 on Fireworks: Fast RL at
 * frontier scale" frames the operator's cost as data movement (normalisation,
 * weighting and gradient intermediates); these probes measure the data
 * movement alone.
 *
 * Conventions: device pointers owned by the caller, 16-byte aligned; sizes in
 * bytes, multiples of 16; all work is enqueued on `stream` (a hipStream_t,
 * NULL for the null stream) and the call returns once it is enqueued.  The
 * library allocates nothing.  Returns 0 on success, 1 for an invalid
 * argument (nothing enqueued), 3 when the HIP runtime refuses the launch.
 * Streaming accesses carry the nontemporal hint, as the operator's do.
 */
#ifndef ATTNRES_PROBES_H
#define ATTNRES_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from src, one 4 KiB chunk per 256-thread workgroup.  Nothing
 * is written except, never in practice, one word of `sink` (4 bytes), which
 * keeps the loads live. */
int attnres_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Write `bytes` of zeros to dst, one 4 KiB chunk per workgroup. */
int attnres_probe_write(void* dst, size_t bytes, void* stream);

/* Copy `bytes` from src to dst (disjoint), one 4 KiB chunk per workgroup. */
int attnres_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * The forward's access pattern without its arithmetic: token t reads row t of
 * each of the N row sets srcs[i] ([T][D] bf16, dense) and writes row t of out
 * ([T][D] bf16) -- one workgroup per token in the operator's forward launch
 * shape (D/8 16-byte vectors spread over whole waves, four per thread for
 * D <= 8192).  The written value is a bitwise OR of the token's rows, so the
 * loads stay live; it is not the operator's output.  1 <= N <= 9,
 * 8 <= D <= 8192 with D % 8 == 0, T >= 0.
 */
int attnres_probe_fwd_pattern(const uint16_t* const* srcs, int32_t N, int64_t T, int32_t D, uint16_t* out,
                              void* stream);

/*
 * The backward's access pattern without its arithmetic: token t reads row t
 * of the N row sets and of dout and writes row t of each of the N gradient
 * row sets dsrcs[i], in the backward's launch shape (256 persistent
 * workgroups of one 16-byte vector per thread, workgroup c taking tokens
 * c, c + 256, ...).  Row i's written value is row i OR dout's row.  Same
 * limits as attnres_probe_fwd_pattern.
 */
int attnres_probe_bwd_pattern(const uint16_t* const* srcs, const uint16_t* dout, int32_t N, int64_t T, int32_t D,
                              uint16_t* const* dsrcs, void* stream);

/*
 * The split backward's access pattern without its arithmetic or its exchange:
 * a workgroup of 4 x 128 threads reads one 1024-channel slice of 4
 * consecutive tokens' dout and N source rows and writes that slice of their N
 * gradient rows (row i's value: row i OR dout's row), and writes one fp32
 * partial row slice per 4 tokens into `partial` ([min(ceil(T/4), 8192)][D]
 * fp32, 16-byte aligned; rows reused every 8192 spans, as the operator's
 * chunked workspace is).  Same limits as attnres_probe_fwd_pattern.
 */
int attnres_probe_split_bwd_pattern(const uint16_t* const* srcs, const uint16_t* dout, int32_t N, int64_t T,
                                    int32_t D, uint16_t* const* dsrcs, float* partial, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_PROBES_H */
