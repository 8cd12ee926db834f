/*
 * moe_decode.h -- routed-expert FP8 block-scaled MoE decode on MI355X (gfx950).
 *
 * The operation (vLLM "mega_moe" page, module docstring and MegaExperts
 * __call__; slot semantics from the nvfp4-megamoe-kernel README, "slot
 * representation"): for each of M decode tokens
 *   1. biased sigmoid top-k routing from router logits: s = sigmoid(z),
 *      key = s + bias, top_k by key (ties to the lower expert), weights =
 *      s / sum(picked s) * routed_scale ("mega_moe" page, top_k_pick);
 *   2. the BF16 activation quantised to OCP FP8 e4m3 per 128 values with
 *      scale max(amax, 1e-10) / 448 (optionally rounded up to a power of two)
 *      ("mega_moe" page, epilogue);
 *   3. GEMM1 against the expert's FP8 W13 (rows 0..I-1 up, I..2I-1 gate)
 *      with FP32 128x128 block scales applied once per K block;
 *   4. clamped SwiGLU: gate = min(g, L), up = clamp(u, -L, L),
 *      act = gate / (1 + exp(-gate)) * up ("mega_moe" page, hidden_block);
 *   5. the hidden requantised to FP8 per 128 (scale amax / 448);
 *   6. GEMM2 against W2, written as an unweighted BF16 "slot" row per
 *      (token, expert) route, row t * top_k + j;
 *   7. combined[t] = BF16(sum_j weights[t, j] * slot[t * top_k + j]): the
 *      routing weights applied exactly once (nvfp4-megamoe-kernel README,
 *      bugs 6 and 7; FP32 sum rounded once as in the "kimi_k3 ... ep.comm"
 *      page's combine).
 * Optionally, the dense shared expert of the "shared_expert" page runs on the
 * same stream (FP8 gate_up GEMV with gate rows first, BF16 gate/up, clamped
 * SwiGLU rounded to BF16, FP8 per 128, down GEMV, BF16 out).
 *
 * Conventions
 *  - All tensor pointers are DEVICE pointers on the device that was current
 *    when moe_decode_create ran, row-major and contiguous, 16-byte aligned.
 *  - FP8 is OCP e4m3 ("e4m3fn": bias 7, max 448, no infinities), one byte per
 *    value; BF16 is a 16-bit brain float; FP32 is IEEE binary32.
 *  - Everything is enqueued on the HIP stream passed in (a hipStream_t, given
 *    as void* so that this header needs no HIP headers; NULL is the default
 *    stream). No call synchronises the host, and moe_decode_run allocates
 *    nothing, so it may be captured in a HIP graph: a replay reads the
 *    inputs and writes the outputs at the addresses captured, for the M
 *    captured, and replays of one handle's graph must be ordered like calls.
 *  - Return value: MOE_DECODE_OK (0) or a negative MOE_DECODE_ERR_* code.
 *    An argument error leaves the handle valid and enqueues nothing.
 *
 * Thread safety: one handle owns one workspace. Calls of moe_decode_run on
 * the same handle must be ordered (same stream, or synchronised); separate
 * handles are independent.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_OK 0
#define MOE_DECODE_ERR_INVALID_ARG (-1)     /* null or misaligned pointer, bad M, bad value */
#define MOE_DECODE_ERR_UNSUPPORTED (-2)     /* shape or option outside what the kernels take */
#define MOE_DECODE_ERR_TOO_MANY_TOKENS (-3) /* M > max_tokens of the handle */
#define MOE_DECODE_ERR_HIP (-4)             /* a HIP call or kernel launch failed */
#define MOE_DECODE_ERR_OUT_OF_MEMORY (-5)   /* workspace allocation failed */
#define MOE_DECODE_ERR_SCRATCH_TOO_SMALL (-6) /* moe_decode_run_noalloc: the step needs more
                                                 than MOE_DECODE_NOALLOC_SCRATCH_BYTES */

#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

/* Routed weight formats. */
#define MOE_WEIGHTS_FP8 0   /* OCP e4m3, FP32 128x128 block scales */
#define MOE_WEIGHTS_NVFP4 1 /* packed E2M1 (two per byte, low nibble first), a UE4M3 byte per 16 values along K */

#define MOE_SCALES_F32 0         /* FP32 [n/128, k/128] block scales */
#define MOE_SCALES_UE8M0_PACKED 1 /* int32 [n, ceil(k/512)]: byte g%4 of word g/4 = biased exponent of K group g */

/* GEMM kernels. All widen FP8 exactly to F16 and add exact products in FP32.
 * The split-K paths divide K among workgroups and sum FP32 partials in the
 * next kernel; MOE_GEMM_MFMA sums all of K inside one workgroup. */
#define MOE_GEMM_AUTO 0         /* MOE_GEMM_MFMA, with persistent workgroups where they apply */
#define MOE_GEMM_VALU_SPLITK 1  /* F16 dot2, split-K over workgroups */
#define MOE_GEMM_MFMA_SPLITK 2  /* v_mfma_f32_16x16x32_f16 (16 routes at once), split-K over workgroups */
#define MOE_GEMM_MFMA 3         /* v_mfma_f32_16x16x32_f16, K split among the waves of a workgroup;
                                   asked for by name: one workgroup per unit. Under AUTO, a GEMM
                                   without a shared expert, with at most 8 tokens or K <= 1024,
                                   and with K / 128 a multiple of 2 x its K parts (at most 64
                                   blocks) runs on resident workgroups that take the units in
                                   turn (bit-identical results) */
#define MOE_GEMM_FP4 4          /* the MOE_WEIGHTS_NVFP4 kernel (reported by moe_decode_plan; gemm_path stays AUTO) */

/* Launch shapes of run(). Every shape gives bit-identical results. */
#define MOE_LAUNCH_AUTO 0             /* the shape measured fastest: MOE_LAUNCH_ROUTE_IN_GEMM1 at
                                         one token where it applies, else MOE_LAUNCH_SEPARATE */
#define MOE_LAUNCH_SEPARATE 1         /* each step a launch of its own (five launches) */
#define MOE_LAUNCH_COMBINE_IN_GEMM2 2 /* MOE_GEMM_MFMA only: the combine inside the GEMM2 launch
                                         (the workgroup that completes a token's column tile
                                         combines it); other paths run MOE_LAUNCH_SEPARATE */
#define MOE_LAUNCH_SWIGLU_IN_GEMM1 3  /* when GEMM1 runs on persistent workgroups: the SwiGLU and
                                         requant inside the GEMM1 launch (the workgroup that
                                         completes a route's 128-column block finishes it);
                                         otherwise MOE_LAUNCH_SEPARATE */
#define MOE_LAUNCH_ROUTE_IN_GEMM1 4   /* when GEMM1 runs on persistent workgroups, M <= 2 and
                                         M * top_k <= 64: routing and the x quantisation inside
                                         the GEMM1 launch (every workgroup routes the tokens
                                         itself, the "mega_moe" page's per-warp routing, and
                                         workgroup 0 writes ids and weights); otherwise
                                         MOE_LAUNCH_SEPARATE */

/* Limits of this implementation. */
#define MOE_DECODE_MAX_EXPERTS 1024
#define MOE_DECODE_MAX_TOP_K 32
#define MOE_DECODE_MAX_TOKENS 256
/* hidden, inter and shared_inter are also bounded by the LDS the GEMM kernel
 * stages per workgroup: 13,376 + 80 * max(hidden, inter, shared_inter) / 128
 * bytes must not exceed 64 KiB, i.e. at most 83,456 (ERR_UNSUPPORTED). */

typedef struct moe_decode_config {
  /* Shapes. hidden (H) and inter (I) are multiples of 128; 1 <= top_k <=
   * min(experts, 32); experts <= 1024; 1 <= max_tokens <= 256. */
  int32_t hidden;
  int32_t inter;
  int32_t experts;
  int32_t top_k;
  int32_t max_tokens;
  int32_t logits_dtype; /* MOE_DTYPE_F32 or MOE_DTYPE_BF16 ([M, E] logits) */
  int32_t ue8m0_act;    /* nonzero: activation scales rounded up to powers of two */
  float limit;          /* SwiGLU clamp L > 0 */
  float routed_scale;   /* multiplies the renormalised routing weights */

  /* Routed expert weights (borrowed: they must outlive the handle), for the
   * El local experts (see local_begin below; El = experts when all are local).
   * MOE_WEIGHTS_FP8:
   *   w13       [El, 2I, H] e4m3, rows 0..I-1 "up", rows I..2I-1 "gate"
   *   w13_scale [El, 2I/128, H/128] FP32, any positive values
   *   w2        [El, H, I] e4m3
   *   w2_scale  [El, H/128, I/128] FP32
   * MOE_WEIGHTS_NVFP4 (nvfp4-megamoe-kernel README, "Data Formats"):
   *   w13       [El, 2I, H/2] packed E2M1, rows 0..I-1 "gate", I..2I-1 "up"
   *   w13_scale [El, 2I, H/16] UE4M3 bytes (e4m3 with the sign clear)
   *   w2        [El, H, I/2] packed E2M1
   *   w2_scale  [El, H, I/16] UE4M3 bytes
   *   H and I multiples of 256; activations are staged to E2M1 with a UE4M3
   *   scale of block_max / 6 per 16 values; GEMM outputs are rounded to BF16;
   *   no shared expert; ue8m0_act must be 0; splits1/splits2 are ignored
   *   (the FP4 GEMM spreads its work evenly over the resident workgroups).
   *   create copies the two scale arrays, reordered for the GEMM kernel, into
   *   memory the handle owns (an eighth of the weight bytes): later writes to
   *   the caller's scale buffers are not seen; the weights are read in place. */
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;

  /* Optional dense shared expert ("shared_expert" page); all zero/NULL when
   * absent. shared_inter (Is) is a multiple of 128. Its units run inside the
   * routed GEMM, SwiGLU and combine launches. The packed scales must repeat
   * one exponent over each 128-row block (INVALID_ARG from create if not).
   * sw13 [2Is, H] e4m3, rows 0..Is-1 gate, Is..2Is-1 up; sw2 [H, Is] e4m3.
   * Scales per shared_scale_format: FP32 [2Is/128, H/128] / [H/128, Is/128],
   * or MOE_SCALES_UE8M0_PACKED int32 [2Is, ceil(H/512)] / [H, ceil(Is/512)]
   * (converted once, in create, to FP32 owned by the handle). */
  int32_t shared_inter;
  int32_t shared_scale_format;
  int32_t shared_ue8m0_act; /* nonzero: the shared expert's activation scales are UE8M0 */
  float shared_limit;
  const void* sw13;
  const void* sw13_scale;
  const void* sw2;
  const void* sw2_scale;

  /* Tuning (0 = automatic). gemm_path: MOE_GEMM_*. splits1/splits2: K splits
   * of GEMM1/GEMM2: over workgroups on the split-K paths (a work unit is 64
   * weight rows x one K split of one touched expert), over the waves of a
   * workgroup on MOE_GEMM_MFMA (1, 2 or 4; a workgroup then owns 64, 32 or 16
   * weight rows). */
  int32_t gemm_path;
  int32_t splits1;
  int32_t splits2;

  /* Weight format (MOE_WEIGHTS_*), and the local experts: routing runs over
   * all `experts`, but only routes whose expert lies in
   * [local_begin, local_begin + local_experts) are computed (one GPU's share
   * under expert parallelism); the slot rows of the others are zero and they
   * add nothing to `combined`. local_experts = 0 means all experts. */
  int32_t weight_format;
  int32_t local_begin;
  int32_t local_experts;

  /* Launch shape (MOE_LAUNCH_*). */
  int32_t launch_mode;
} moe_decode_config;

typedef struct moe_decode_handle* moe_decode_t;

/* Passage: vLLM "mega_moe" page, MegaExperts.__init__ (the layer object holds
 * the expert weights and scales it was built with, and fixes hidden, inter,
 * experts, top_k, limit, routed scale and the UE8M0 flag) and
 * MegaExperts.prepare (all per-shape set-up happens before the first call, so
 * that calls can be captured in a graph); "shared_expert" page,
 * SharedExpert.__init__ (packed UE8M0 scales converted once, block_scales).
 * Ownership follows the nvfp4-megamoe-kernel README ("SFB ... NOT Cached"):
 * the handle keeps no cache keyed on caller memory that it might evict or
 * outlive; what it derives from the weights (FP32 shared scales, reordered
 * FP4 scales) it copies once, here, into memory it owns until destroy.
 *
 * Validates cfg, allocates the handle's workspace for cfg->max_tokens on the
 * current device, and converts packed shared-expert scales. Weight pointers
 * are borrowed, not copied. On success *out receives the handle.
 * Errors: INVALID_ARG (null cfg/out/weights, limit <= 0, max_tokens out of
 * range), UNSUPPORTED (shape limits above), OUT_OF_MEMORY, HIP. */
int moe_decode_create(const moe_decode_config* cfg, moe_decode_t* out);

/* Passage: vLLM "mega_moe" page, MegaExperts.__call__ (x [M, hidden] BF16,
 * logits [M, experts], bias [experts] FP32 in; BF16 [M * top_k, hidden] route
 * outputs, int32 [M, top_k] experts and FP32 [M, top_k] weights out) and the
 * nvfp4-megamoe-kernel README, "slot representation" (weights applied once,
 * in the final combine).
 *
 * One routed-expert decode step for M tokens, 0 <= M <= max_tokens.
 *   x          [M, H] BF16
 *   logits     [M, E] FP32 or BF16 (per logits_dtype)
 *   bias       [E] FP32 score-correction bias (selects, does not weigh)
 *   slots      [M*top_k, H] BF16 out: unweighted expert output of route
 *              t*top_k + j (token t, j-th pick)
 *   ids        [M, top_k] int32 out: picked experts, highest biased score first
 *   weights    [M, top_k] FP32 out: routing weights
 *   combined   [M, H] BF16 out: sum_j weights[t, j] * slots[t*top_k + j]
 *   shared_out [M, H] BF16 out of the shared expert, or NULL to skip it
 *              (must be NULL if the handle has no shared expert)
 *   stream     hipStream_t
 * M == 0 enqueues nothing and returns OK. Errors: INVALID_ARG (null handle or
 * pointer, misaligned pointer, M < 0), TOO_MANY_TOKENS, HIP (launch failure).
 * Numerics: ids and weights follow the FP32 rules above exactly; slot,
 * combined and shared rows carry FP32 accumulation-order differences. */
int moe_decode_run(moe_decode_t h, int32_t M, const void* x, const void* logits,
                   const float* bias, void* slots, int32_t* ids, float* weights,
                   void* combined, void* shared_out, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid allocation.
 *
 * moe_decode_run without a handle: the same launches and results as
 * moe_decode_run on a handle created from *cfg (bit-identical outputs), with
 * the workspace in a fixed device buffer of MOE_DECODE_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.
 * Nothing is allocated: no hipMalloc, no hipFree, no allocating library call.
 * The buffer's address is looked up once per device, on the first call made
 * with that device current. The call runs on the current device.
 *  - cfg as for moe_decode_create, except that max_tokens is not used (M
 *    sizes the workspace) and only what needs no handle-owned copy is taken:
 *    MOE_WEIGHTS_FP8 routed weights, and a shared expert only with
 *    MOE_SCALES_F32 scales (UNSUPPORTED otherwise).
 *  - Other arguments and errors as moe_decode_run; 0 <= M <= 256. A step
 *    whose workspace exceeds the buffer returns SCRATCH_TOO_SMALL and
 *    enqueues nothing (at DeepSeek-V3 shapes, H = 7168, I = 2048, top-8, up
 *    to 64 tokens fit).
 *  - Every call on one GPU shares that GPU's buffer, and the buffer keeps
 *    the last call's contents (the call clears the counters it needs at
 *    zero, with a kernel, before its other launches). Calls that overlap on
 *    one GPU (on different streams, or from different threads without
 *    ordering) race on the buffer and give undefined results. Handles
 *    created with moe_decode_create do not use it. */
#define MOE_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_decode_run_noalloc(const moe_decode_config* cfg, int32_t M, const void* x, const void* logits,
                           const float* bias, void* slots, int32_t* ids, float* weights, void* combined,
                           void* shared_out, void* stream);

/* Passage: the ownership rule of moe_decode_create (the pages' layer objects
 * release what they allocated when they go away; borrowed weights are left
 * to the caller).
 * Frees the workspace and the handle's own copies (after synchronising the
 * device). The caller's weights are untouched. NULL is a no-op. */
void moe_decode_destroy(moe_decode_t h);

/* The text of an error code (the pages report these conditions with Python
 * assertions, e.g. the "mega_moe" page's _MegaKernel checks of experts and
 * hidden; here they are return codes). Static storage; never NULL. */
const char* moe_decode_error_string(int code);

/* ---- Introspection (tests and benchmarks) ------------------------------ */

/* Test and benchmark introspection (no passage: it describes this library's
 * own launches). The launch plan run() uses for M tokens: out[0] = GEMM path used
 * (MOE_GEMM_*, never AUTO), out[1] / out[2] = partial-sum slices GEMM1 /
 * GEMM2 write (the K splits of the split-K paths; 1 on MOE_GEMM_MFMA),
 * out[3] / out[4] = 128-K blocks per split or per K part, out[5] / out[6] =
 * grids of GEMM1 / GEMM2 (including the shared expert's units when the
 * handle has one), out[7] / out[8] = on the split-K paths 64-row tiles
 * streamed per workgroup, on MOE_GEMM_MFMA weight rows per workgroup. With
 * n >= 15 also the shared expert's plan (zeros without one): out[9] /
 * out[10] = its partial-sum slices, out[11] / out[12] = blocks per split or
 * part, out[13] / out[14] = its work units in the GEMM1 / GEMM2 launches.
 * With n >= 17: out[15] / out[16] = K parts per workgroup in GEMM1 / GEMM2
 * (1 on the split-K paths). With n >= 18: out[17] = kernel launches of run()
 * (5, less one for each of routing, the SwiGLU and the combine that runs
 * inside a GEMM launch). With n >= 20:
 * out[18] / out[19] = workgroups of the persistent GEMM1 / GEMM2 launch on
 * MOE_GEMM_MFMA (0: one workgroup per unit). On MOE_GEMM_FP4: out[1] / out[2] = the most
 * partial slots a 64-row tile can have, out[3] / out[4] = 128-K blocks of
 * the whole K, out[5] / out[6] = launched workgroups (the resident ones, or
 * one per route when there are more routes). n is the capacity of out
 * (>= 9). */
int moe_decode_plan(moe_decode_t h, int32_t M, int32_t* out, int32_t n);

/* Passage: the intermediate results named by the "mega_moe" page's kernel
 * (routing picks, the FP8 activation and its scales, GEMM1 sums, the FP8
 * hidden and its scales, GEMM2 sums; epilogue and hidden_block) and by the
 * "shared_expert" page's _GateUpKernel and _DownKernel; for tests.
 * Stage read-back: copies workspace region `stage` of the last run into the
 * device buffer dst (bytes = capacity of dst) on stream. Stages:
 *  0 control words int32[3] (arrival counter, distinct experts U, jobs J)
 *  1 distinct experts, ascending int32[U]   2 their first index into stage 4
 *  3 their route counts int32[U]            4 routes grouped by expert int32[M*k]
 *  5 x_q [M, H] e4m3                        6 x_s [M, H/128] FP32
 *  7 GEMM1 split partials FP32 [splits1, M*k, 2I]
 *  8 h_q [M*k, I] e4m3                      9 h_s [M*k, I/128] FP32
 * 10 GEMM2 split partials FP32 [splits2, M*k, H]
 * Shared expert (handles with one; INVALID_ARG otherwise):
 * 11 its x_q [M, H] e4m3                   12 its x_s [M, H/128] FP32
 *    (the routed stages 5 and 6 when both use the same scale rule)
 * 13 gate_up split partials FP32 [splits, M, 2Is]
 * 14 h_q [M, Is] e4m3                      15 h_s [M, Is/128] FP32
 * 16 down split partials FP32 [splits, M, H]
 * 19 the shared expert's FP32 W13 block scales [2Is/128, H/128] as the kernels
 *    read them (for MOE_SCALES_UE8M0_PACKED, the conversion done by create:
 *    bit pattern byte << 23, so byte 0 is +0.0 and byte 255 +inf, the
 *    "shared_expert" page's block_scales)
 * 20 the same for W2 [H/128, Is/128]
 * MOE_WEIGHTS_NVFP4 handles: stages 5 / 8 hold packed E2M1 ([M, H/2],
 * [M*k, I/2]) and 6 / 9 UE4M3 bytes ([M, H/16], [M*k, I/16]); stages 7 / 10
 * hold the GEMMs' partial slots ([slots, M*k, N], out[1] / out[2] of
 * moe_decode_plan), and after a run slot 0 of stage 7 holds GEMM1's FP32
 * sums for the local routes; control word 2 is the job count J;
 * 17 job table int32[J][4] {local expert, first index into stage 4, route
 *    count (at most 4), 0}         18 job of each local route int32[M*k]
 * The size copied is min(bytes, size of the stage for the handle's maximum). */
int moe_decode_debug_stage(moe_decode_t h, int32_t stage, void* dst, size_t bytes,
                           void* stream);

/* Benchmark support (no passage: it times this library's own launches).
 * Per-kernel timing of subsequent runs (enable != 0; not for use under graph
 * capture): each kernel of the layer is launched with a pair of HIP events
 * that take its dispatch's own start and end timestamps (hipExtLaunchKernel),
 * so the time excludes the gaps between launches. After a run has completed,
 * moe_decode_last_timing writes the milliseconds of each kernel in order:
 * route+quant, GEMM1, SwiGLU+requant, GEMM2, combine (the shared expert, when
 * run, is part of the last four; when routing, the combine or the SwiGLU
 * runs inside a GEMM launch, its time is that GEMM's and its own entry is 0).
 * n is the capacity of ms (>= 5). */
int moe_decode_set_timing(moe_decode_t h, int32_t enable);
int moe_decode_last_timing(moe_decode_t h, float* ms, int32_t n);

/* Passage: the FP8 encode of the "mega_moe" page's epilogue and hidden_block
 * (pack_fp8 of scaled values; read here as OCP e4m3, nearest even,
 * saturating). For tests.
 * Codec self-check of the device code: q[i] = e4m3 encoding of in[i] with the
 * library's quantiser (nearest, ties to even, saturating), and dq[i] = the
 * value the GEMM inner products read for code (i & 255) through the path's
 * FP8 -> F16 conversion. in, q and dq are device buffers of n elements. */
int moe_decode_debug_codec(const float* in, uint8_t* q, float* dq, int32_t n, void* stream);

/* Passage: nvfp4-megamoe-kernel README, "Data Formats" (E2M1 values, two per
 * byte) and bug 2 (activation staging). For tests.
 * The same for E2M1: q[i] = the library's E2M1 code of in[i] (nearest, ties
 * to even, saturating at +-6), and dq[i] = the value the FP4 GEMM reads for
 * code (i & 15) through its FP4 -> F16 widening (with the code placed in
 * each nibble and byte position of a word in turn). */
int moe_decode_debug_codec_fp4(const float* in, uint8_t* q, float* dq, int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
