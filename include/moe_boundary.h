/*
 * The two boundary steps either side of the routed-expert path in an
 * expert-parallel pipeline, in their one-GPU form ("kimi_k3 ... ep.comm"
 * page: EpDispatch, EpCombine, rms_rstd). Same library and error codes as
 * moe_decode.h; both calls enqueue one kernel on `stream` (a hipStream_t;
 * NULL is the default stream), allocate nothing and never synchronise.
 *
 * All pointers are device pointers; BF16 and e4m3 as in moe_decode.h, E8M0
 * is a byte b meaning 2^(b - 127).
 */
#ifndef MOE_BOUNDARY_H
#define MOE_BOUNDARY_H

#include <stdint.h>

#include "moe_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_BOUNDARY_MAX_D 16384 /* longest row either call takes */

/* Passage: "kimi_k3 ... ep.comm" page, EpDispatch (the sender quantises each
 * token's latent to MXFP8, one E8M0 scale per 32 values, before the copy).
 * MXFP8 quantisation of T BF16 rows of length D (EpDispatch: the latent is
 * quantised per 32 values before it is sent). Per 32-value block b of row t:
 * shared = floor(log2(max |x|)) - 8 kept within [-127, 127] (-127 for an
 * all-zero block), sf[t, b] = shared + 127, and q[t, 32b + i] =
 * e4m3(x * 2^-shared) rounded to nearest even, saturating at +-448 (the OCP
 * MX scale rule for e4m3 elements; the page names the rule's helpers without
 * showing them).
 *   x  [T, D] BF16, rows contiguous; 16-byte aligned
 *   q  [T, D] e4m3 out; 16-byte aligned
 *   sf [T, D / 32] E8M0 bytes out, one per block in block order (no swizzle)
 * D must be a positive multiple of 32, at most MOE_BOUNDARY_MAX_D
 * (UNSUPPORTED otherwise). T = 0 is a valid empty call whatever the other
 * arguments (nothing is read or written); otherwise T < 0 or a NULL or
 * misaligned pointer is INVALID_ARG. Nothing is enqueued on an error. */
int moe_mxfp8_quantize(const void* x, int32_t T, int32_t D, void* q, void* sf, void* stream);

/* Passage: "kimi_k3 ... ep.comm" page, EpCombine (the owner sums the ranks'
 * partial rows in FP32 in rank order, rounds once, then applies RMSNorm) and
 * rms_rstd (an IEEE divide by D, then the reciprocal square root).
 * The combine's reduce and RMSNorm (EpCombine, rms_rstd): for each token t,
 *   latent[t] = BF16(sum over n in 0..N-1, in that order, of partials[t, n])
 *               with the sum in FP32, rounded once;
 *   rstd      = 1 / sqrt(sum_i latent[t, i]^2 / D + eps), in FP32 with the
 *               division correctly rounded;
 *   out[t, i] = BF16(latent[t, i] * rstd * gamma[i]) (two FP32 products,
 *               one BF16 rounding).
 *   partials [T, N, D] BF16 (N per-rank partial rows of each token; on one
 *            GPU N = 1 and partials is the routed path's combined output)
 *   gamma    [D] BF16 gains
 *   latent   [T, D] BF16 out, or NULL to skip it
 *   out      [T, D] BF16 out
 * All arrays 16-byte aligned, rows contiguous. D a positive multiple of 8 up
 * to MOE_BOUNDARY_MAX_D and 1 <= N <= 64 (UNSUPPORTED otherwise); eps >= 0
 * and finite. T = 0 is a valid empty call. Errors as above. */
int moe_reduce_rmsnorm(const void* partials, int32_t T, int32_t N, int32_t D, const void* gamma, float eps,
                       void* latent, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BOUNDARY_H */
