/*
 * decode_sampling_tail -- C ABI of the GPT-OSS decode sampling tail on one
 * MI355X (gfx950): final RMSNorm -> bf16 lm_head -> top-k -> sampler.
 *
 * The operations and their parameters follow the page "GPT-OSS Tail Chunked
 * Megakernel Kernel API Reference" (NKI library docs), cited below by the
 * name of the parameter whose paragraph defines them.  Everything runs on
 * one GPU with the whole vocabulary local, so the page's vocabulary shards,
 * collectives and rank maps have no counterpart here (V_s = V).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers, allocated, owned and freed by the
 *    caller.  The library allocates nothing, never synchronizes, and enqueues
 *    its kernels on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream).  Outputs are valid once the stream reaches that point.
 *    Its only global state is a set of per-device caches of device queries
 *    (compute-unit count, kernel occupancy, the raised LDS limit), each
 *    filled once, thread-safely, the first time a call runs on that device
 *    and never changed afterwards; no call's result depends on them beyond
 *    the launch shape.  tail_forward_noalloc alone also uses a static
 *    scratch array in each device's memory (see its declaration).
 *  - Arrays are C-contiguous (row-major) with the shapes given.
 *  - Every call validates its arguments on the host BEFORE any HIP call and
 *    returns a status code; on an error nothing is enqueued and no output is
 *    touched.  TAIL_ERR_HIP reports a launch error from the HIP runtime.
 *    Faults inside a kernel surface asynchronously, as for any HIP call.
 *  - Results are deterministic: the same inputs give the same bytes (no
 *    floating-point atomics).  Within one lm_head path a logit depends
 *    neither on the column's position nor on the other rows of the batch, so
 *    duplicated weight columns give bitwise-equal logits.  The path depends
 *    on the batch size: weight streaming with fp32 FMAs up to 3 rows, the
 *    16x16x32 matrix-core kernel from 4 to 64 rows, the 32x32x16 kernel
 *    above (from 65 to 128 rows only where the 16x16x32 kernel would not
 *    split K: V above 130560 columns, or fewer than 512 padded K lanes;
 *    otherwise it keeps those batches too, with K split); each sums in its
 *    own fixed order, so a row's logits may differ in the last bits when the
 *    batch crosses 3/4 or 64/65 rows (128/129 where K is split); each path
 *    meets the same accuracy bar.
 *  - Calls on different streams may run concurrently as long as they do not
 *    share output or workspace memory.
 */
#ifndef DECODE_SAMPLING_TAIL_H
#define DECODE_SAMPLING_TAIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TAIL_OK 0
#define TAIL_ERR_INVALID_ARG 1 /* a size, pointer, flag or dtype is out of its domain */
#define TAIL_ERR_UNSUPPORTED 2 /* valid, but outside what the library implements */
#define TAIL_ERR_WORKSPACE 3   /* workspace missing, misaligned or too small */
#define TAIL_ERR_HIP 4         /* the HIP runtime rejected a launch */
#define TAIL_ERR_SCRATCH_LIMIT 5 /* tail_forward_noalloc: more than TAIL_SCRATCH_BYTES needed */

/* storage dtype of hidden_states ("hidden_states": fp32, fp16 or bf16) */
#define TAIL_F32 0
#define TAIL_F16 1
#define TAIL_BF16 2

/* flags (run-time counterparts of the page's trace-time flags) */
#define TAIL_EMIT_LOGITS 1u  /* "emit_logits": write the fp32 [gbs,V] logits */
#define TAIL_ZERO_PAD 2u     /* "zero_interleaved_pad": skip the interleaved pad lanes */
#define TAIL_DEFERRED_RMS 4u /* "deferred_rms": apply the row's rms scale after the contraction */
#define TAIL_PAGE_PRECISION 8u /* the page's own numerics (below) */
#define TAIL_NAN_FOLD 16u      /* "skip_nan_fold" off: NaN logits rank (and return) as -inf */
/* Each entry point rejects (TAIL_ERR_INVALID_ARG) the bits it does not accept:
 * tail_rmsnorm, tail_lm_head and tail_rmsnorm_lm_head take the first four,
 * tail_forward all five, tail_topk_ex TAIL_PAGE_PRECISION and TAIL_NAN_FOLD. */

/* limits of the library */
#define TAIL_K_MAX 1024      /* largest k ("k": 256 in production) */
#define TAIL_GBS_MAX 4096    /* largest batch */
#define TAIL_H_MAX 65536     /* largest hidden width */

/*
 * Pad lanes ("zero_interleaved_pad", "hidden_actual").  With TAIL_ZERO_PAD and
 * H > H_u, the hidden is split into groups of s = H / (H - H_u) lanes and the
 * LAST lane of every group is a pad lane (H must be a multiple of H - H_u).
 * Pad lanes of hidden, gamma and of the weight's rows are never read, so any
 * value there (NaN included) cannot reach an output.  Without the flag all H
 * lanes are used and the caller guarantees that padding holds zeros.  The
 * mean square of the RMSNorm always divides by H_u (H_u = H when unpadded).
 */

/*
 * Precision ("deferred_rms", "skip_nan_fold", "emit_logits").  By default the
 * GEMM input keeps (at least) fp32 precision and the top-k ranks the fp32
 * logits.  TAIL_PAGE_PRECISION selects the page's own numerics instead: the
 * fp32 activation (x * gamma deferred, (x * r) * gamma in-chain) is rounded
 * to bf16 once per element (round to nearest, ties to even), the bf16 x bf16
 * products are summed in fp32, and the top-k ranks the bf16 mirror of the
 * fp32 logits (each logit rounded to bf16 the same way), returning the mirror
 * values.  The emitted logits stay fp32.
 */

/*
 * tail_rmsnorm -- final RMSNorm ("gamma", "eps", "hidden_actual",
 * "hidden_states", "deferred_rms").
 *
 *   hidden [gbs, H]  dtype TAIL_F32 / TAIL_F16 / TAIL_BF16 (bf16 as raw uint16
 *                    bits); widened exactly to fp32 (the page's 16-bit input
 *                    path), so a 16-bit input gives the same bytes as its
 *                    pre-widened fp32 copy.  Naturally aligned.
 *   gamma  [H]       fp32.
 *   eps              >= 0, added to the mean square inside the square root.
 *   out_y  [gbs, H]  fp32: x * r * gamma ("(x*rms)*gamma" order), or x * gamma
 *                    with TAIL_DEFERRED_RMS; pad lanes are written as 0.  With
 *                    TAIL_PAGE_PRECISION each value is rounded to bf16 (the
 *                    GEMM input of that mode), stored as fp32.
 *   out_r  [gbs]     fp32: r = 1/sqrt(mean_{H_u}(x^2) + eps); may be NULL
 *                    unless TAIL_DEFERRED_RMS is set.
 * TAIL_ZERO_PAD, TAIL_DEFERRED_RMS and TAIL_PAGE_PRECISION are meaningful in
 * `flags`.
 */
int tail_rmsnorm(const void* hidden, int dtype, const float* gamma, int gbs, int H, int H_u,
                 float eps, unsigned flags, float* out_y, float* out_r, void* stream);

/*
 * tail_lm_head -- the lm_head contraction ("lm_head_weight_t", "emit_logits").
 *
 *   y         [gbs, H] fp32 normalized hidden rows (the output of tail_rmsnorm).
 *   w_t       [H, V]   bf16 raw bits, ALREADY TRANSPOSED and C-contiguous (V is
 *                      the fast axis), 16-byte aligned; V must be a multiple
 *                      of 8 (TAIL_ERR_UNSUPPORTED otherwise), so that every
 *                      weight row starts 16-byte aligned for the 16-byte
 *                      loads and copies of all lm_head kernels (every entry
 *                      that takes V applies the same rule, and
 *                      tail_workspace_size returns 0 for such a V).
 *   row_scale [gbs]    fp32 per-row factor applied to the finished sum (the
 *                      deferred rms scale), or NULL for none.
 *   logits    [gbs, V] fp32, 16-byte aligned:
 *                      logits[b,v] = row_scale[b] * sum_h y[b,h] * W[h,v],
 *                      the sum in fp32 over the real (non-pad) lanes.  By
 *                      default the activations are never rounded to a single
 *                      bf16: the weight-streaming path (gbs <= 3) uses them
 *                      as fp32; the matrix-core path (gbs > 3) splits each
 *                      into two bf16 terms whose sum keeps it to 2^-17
 *                      relative.  With TAIL_PAGE_PRECISION each y[b,h] is
 *                      first rounded to bf16.
 *   ws, ws_bytes       workspace of at least tail_workspace_size() bytes,
 *                      256-byte aligned (may be NULL when that size is 0).
 * TAIL_ZERO_PAD and TAIL_PAGE_PRECISION are meaningful in `flags`.
 */
int tail_lm_head(const float* y, const uint16_t* w_t, const float* row_scale, int gbs, int H,
                 int H_u, int V, unsigned flags, float* logits, void* ws, size_t ws_bytes,
                 void* stream);

/*
 * tail_rmsnorm_lm_head -- the final RMSNorm and the lm_head in one call
 * ("hidden_states", "gamma", "eps", "hidden_actual", "zero_interleaved_pad",
 * "deferred_rms", "lm_head_weight_t"): the logits of tail_rmsnorm followed by
 * tail_lm_head, with the row's rms scale applied after the contraction under
 * TAIL_DEFERRED_RMS (the page's default) or inside the activations without it.
 * On small batches the normalization runs in the prologue of the
 * weight-streaming kernel; on larger ones it writes the activations that the
 * matrix-core kernel reads.
 *
 *   hidden, dtype, gamma, gbs, H, H_u, eps, w_t, V: as above.
 *   logits [gbs, V] fp32, 16-byte aligned.
 *   out_r  [gbs] fp32 or NULL: the per-row rms scale r.
 *   ws, ws_bytes: workspace of at least tail_workspace_size() bytes.
 * TAIL_ZERO_PAD, TAIL_DEFERRED_RMS and TAIL_PAGE_PRECISION are meaningful in
 * `flags`.
 */
int tail_rmsnorm_lm_head(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t,
                         int gbs, int H, int H_u, int V, float eps, unsigned flags, float* logits,
                         float* out_r, void* ws, size_t ws_bytes, void* stream);

/*
 * tail_topk -- global top-k of every row over the full vocabulary ("k",
 * Background: the global top-k computed locally over the full vocabulary).
 *
 *   logits [gbs, V] fp32, finite (NaN ordering is unspecified), 16-byte aligned.
 *   vals   [gbs, k] fp32: the k largest logits of the row, descending.
 *   idx    [gbs, k] int32: their column indices.  Equal values are listed in
 *                   ascending index order, so ties at the k-th place keep the
 *                   lower indices; -0.0 and +0.0 are equal.
 *   1 <= k <= min(V, TAIL_K_MAX).
 */
int tail_topk(const float* logits, int gbs, int V, int k, float* vals, int32_t* idx, void* ws,
              size_t ws_bytes, void* stream);

/*
 * tail_topk_ex -- tail_topk with the page's top-k options ("emit_logits",
 * "skip_nan_fold", "debug_taps").  Arguments and workspace as for tail_topk;
 * infinities always order as numbers.
 *   flags: TAIL_PAGE_PRECISION ranks the bf16 mirror of the logits (each logit
 *          rounded to bf16, nearest, ties to even) and returns the rounded
 *          values (fp32 with zero low 16 bits); distinct logits that round to
 *          one bf16 tie, and ties keep the lower indices.
 *          TAIL_NAN_FOLD ranks a NaN logit (either sign) as -inf and returns
 *          -inf for it (without it, NaN ordering is unspecified).  Any other
 *          bit is TAIL_ERR_INVALID_ARG.
 *   taps:  [gbs, 4] u32 or NULL ("debug_taps": the page does not list its
 *          taps; these are this top-k's stage-1 diagnostics): per row, the
 *          lower bound t0 of the k-th largest group maximum as an
 *          order-preserving key (key(f) = bits | 0x80000000 for f >= +0,
 *          ~bits for f < 0, -0.0 as +0.0; the same transform applies to the
 *          mirrored and folded values the row is ranked by), the number of
 *          candidate groups (gs consecutive columns, gs the largest power of
 *          two <= 64 that leaves at least k groups, doubled while there are
 *          more than 8192) whose maximum key is >= t0, the number of elements
 *          with key >= t0, and 1 if that number exceeded 4096 (the exact
 *          multi-pass path ran) or 0.
 */
int tail_topk_ex(const float* logits, int gbs, int V, int k, unsigned flags, float* vals,
                 int32_t* idx, uint32_t* taps, void* ws, size_t ws_bytes, void* stream);

/*
 * tail_sample -- per-row sampler over the k candidates ("sampling_params").
 *
 *   vals, idx  [gbs, k] as produced by tail_topk (descending).
 *   params     [gbs, ncols] fp32, ncols 3 = [top_k, top_p, temperature] with
 *              the deterministic draw u = 0.5, or 4 = [.., u] with u in [0,1).
 *   tokens     [gbs] int32: the sampled column index.
 * Per row: kk = trunc(top_k), and kk = k when top_k is not in [1, k+1);
 * temperature <= 0 (or NaN) is greedy: tokens = idx[0].  Otherwise, in fp64,
 * e_i = exp((vals_i - vals_0) / T) for i < kk, S_i = e_0 + .. + e_i; the
 * nucleus keeps m = 1 + min{i : S_i >= top_p * S_{kk-1}} candidates (kk when
 * none); the token is idx[j] with j = min{i < m : S_i > u * S_{m-1}} (m-1 when
 * none), i.e. candidate i owns [S_{i-1}, S_i) / S_{m-1}.  u < 0 acts as 0.
 */
int tail_sample(const float* vals, const int32_t* idx, int gbs, int k, const float* params,
                int ncols, int32_t* tokens, void* stream);

/*
 * tail_forward -- the whole tail in one call (the page's
 * gpt_oss_tail_chunked_megakernel on one GPU): RMSNorm -> lm_head -> top-k ->
 * sampler, all enqueued on `stream`.
 *
 *   hidden, dtype, gamma, w_t, gbs, H, H_u, V, k, eps: as above.
 *   flags:  TAIL_EMIT_LOGITS (write `logits`), TAIL_ZERO_PAD, TAIL_DEFERRED_RMS,
 *           TAIL_PAGE_PRECISION (bf16 GEMM input, and the top-k ranks the bf16
 *           mirror as tail_topk_ex does), TAIL_NAN_FOLD (the top-k folds NaN
 *           logits to -inf as tail_topk_ex does; NaN-free logits give the same
 *           outputs either way).  A row with no finite logit has no defined token.
 *   params: [gbs, ncols] or NULL; NULL skips the sampler and leaves `tokens`
 *           untouched (tokens may then be NULL).
 *   logits: [gbs, V] fp32, required only with TAIL_EMIT_LOGITS.
 *   vals, idx: [gbs, k] top-k outputs (always written).
 *   ws:     workspace of at least tail_workspace_size(...) bytes, 256-byte aligned.
 *
 * From 65 rows the lm_head kernel can also run the top-k and sampler itself,
 * after a grid barrier, so that the step is the producer and one kernel (the
 * page's fused tail; GPT-OSS tail API page, Background): the environment
 * variable TAIL_FUSED_SELECT=1, read at every call, selects that, for
 * batches whose top-k groups are the lm_head's 64-column groups and without
 * TAIL_NAN_FOLD (and up to 128 rows in the page-precision mode).  The outputs
 * are bitwise the same either way; it is not the default because it measured
 * slower.  Its barrier waits a bounded time (TAIL_FUSED_SPIN polls, 4096 by
 * default), after which a workgroup leaves its share of the rows to the
 * others, so a call ends with every row done even where the GPU is shared.
 */
int tail_forward(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t, int gbs,
                 int H, int H_u, int V, int k, float eps, unsigned flags, const float* params,
                 int ncols, float* logits, float* vals, int32_t* idx, int32_t* tokens, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * tail_forward_noalloc -- tail_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments and outputs without `ws`/`ws_bytes`.
 * The workspace is a static array of TAIL_SCRATCH_BYTES inside the library,
 * one per device, held from the library's first use on that device until
 * the process ends; the call allocates and frees nothing.
 *   - A call whose workspace (tail_workspace_size(...) bounds it) exceeds
 *     TAIL_SCRATCH_BYTES returns TAIL_ERR_SCRATCH_LIMIT and enqueues nothing.
 *     With the logits not emitted the workspace holds them, so at H = 2880
 *     and V = 201088 the limit admits up to 79 rows; with TAIL_EMIT_LOGITS
 *     (the logits in the caller's buffer) up to 1882.
 *   - Every call on a device uses that device's one array: calls that may run
 *     at the same time on one device (different streams, or threads without
 *     ordering) race on it and must not overlap.  Nothing in it has to start
 *     cleared: every call writes what it reads.
 *   - TAIL_ERR_HIP if the array's device address cannot be obtained.
 */
#define TAIL_SCRATCH_BYTES (64u << 20)
int tail_forward_noalloc(const void* hidden, int dtype, const float* gamma, const uint16_t* w_t,
                         int gbs, int H, int H_u, int V, int k, float eps, unsigned flags,
                         const float* params, int ncols, float* logits, float* vals, int32_t* idx,
                         int32_t* tokens, void* stream);

/*
 * Workspace bytes needed by tail_forward, tail_rmsnorm_lm_head, tail_lm_head
 * and tail_topk for these sizes and flags (one buffer of this size serves any
 * of them).  Returns 0
 * for arguments that the calls would reject.  Pure host function.
 */
size_t tail_workspace_size(int gbs, int H, int H_u, int V, int k, unsigned flags);

/* Static description of a status code (never NULL). */
const char* tail_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_SAMPLING_TAIL_H */
