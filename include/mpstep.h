/*
 * mpstep -- the mixed-precision optimizer step on AMD Instinct MI355X (gfx950).
 *
 * One logical update of a mixed-precision training run, entirely on the GPU
 * and stream-ordered (no host synchronisation on the hot path):
 *
 *   for each micro-batch i:  mp_accumulate        acc += (n_i/N) * widen(g16_i)
 *   mp_unscale_check_norm                         g = acc / S, overflow flag,
 *                                                 global L2 norm, clip coefficient
 *   mp_adamw_step                                 AdamW on fp32 master, m, v;
 *                                                 RNE cast master -> 16-bit weight;
 *                                                 nothing is written on overflow
 *   mp_scaler_update                              dynamic loss-scale decision
 *
 * The method is the one described on these pages (cited by title and section):
 *  - "Mixed precision, loss scaling, gradient accumulation, and activation
 *    checkpointing", section 2 "Principles" (16-bit formats, fp32 masters,
 *    loss scaling, dynamic scaling, gradient accumulation) and section 4
 *    "The interface" (scaler, grad_accumulate, train_step_mixed);
 *  - "Megatron Internals III: Mixed Precision, Loss Scaling, and Grad
 *    Clipping", sections 4-9 (unscale, controller, global overflow decision,
 *    optimizer wrapper, fused gradient copy, global-norm clipping and the
 *    order of operations);
 *  - "Accumulate gradients and recompute activations", section "Weight each
 *    mean by the targets it represents" (token-weighted accumulation) and
 *    "Discard a failed partial logical update" (what a skip preserves);
 *  - "Your weights fit on one device but Adam's moments do not", section "Why
 *    the optimizer state is the thing that overflows" (the Adam update);
 *  - "Chapter 41 Training at Scale", section 41.1, equation (41.1) (memory).
 *
 * Conventions shared by every entry point:
 *  - Pointers named in a plan or gradset are device pointers into memory the
 *    CALLER owns (e.g. PyTorch allocations).  The library never frees them;
 *    they must stay valid until the stream work that uses them has finished.
 *    Every such pointer must be 16-byte aligned.  Starting every tensor on a
 *    whole 128-byte line (256 bytes for fp32) is faster: the AdamW pass then
 *    writes no partial lines at tensor edges (10% on 4096 ragged tensors).
 *  - The library owns plans, gradsets and states.  It allocates device memory
 *    only in the *_create calls, never in the hot calls.
 *  - Objects are bound to the HIP device that was current at creation; make it
 *    current before calling a hot entry point (else MP_ERR_INVALID).
 *  - `stream` is a hipStream_t passed as void* (NULL: the null stream).  Hot
 *    calls only enqueue work on it and return; results reach the host through
 *    mp_state_read.
 *  - Structural errors (bad arguments, wrong call order) are returned before
 *    anything is enqueued.  Numeric overflow is NOT an error: it is a device
 *    flag and the update is skipped on the device.
 *  - A plan and a state are used by one stream at a time (not thread-safe).
 */
#ifndef MPSTEP_H
#define MPSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MPSTEP_ABI_VERSION 1

/* The two enumerations span every int32 value (the _RANGE_ enumerators are not
 * values of the ABI): a C caller may pass any int32 where one is expected, and
 * the library refuses what is not a listed value without undefined behaviour. */
typedef enum {
    MP_OK = 0,
    MP_ERR_INVALID = 1,   /* an argument is out of range or NULL */
    MP_ERR_ALIGN = 2,     /* a buffer is not 16-byte aligned */
    MP_ERR_NOMEM = 3,     /* a device or host allocation failed */
    MP_ERR_HIP = 4,       /* the HIP runtime reported an error */
    MP_ERR_ORDER = 5,     /* calls out of the documented order */
    MP_STATUS_RANGE_MIN_ = -2147483647 - 1,
    MP_STATUS_RANGE_MAX_ = 2147483647
} mp_status;

/* The 16-bit model format ("Mixed precision ...", section 2, "Two 16-bit
 * formats"): bf16 = 8 significant bits and fp32's exponent range; fp16 = 11
 * significant bits, largest finite 65504, smallest subnormal 2^-24. */
typedef enum {
    MP_BF16 = 0,
    MP_FP16 = 1,
    MP_DTYPE16_RANGE_MIN_ = -2147483647 - 1,
    MP_DTYPE16_RANGE_MAX_ = 2147483647
} mp_dtype16;

typedef struct mp_plan mp_plan;        /* tensor list + chunk table (device) */
typedef struct mp_gradset mp_gradset;  /* one micro-batch's gradient pointers (device) */
typedef struct mp_state mp_state;      /* loss scale, optimizer clock, step results (device) */
typedef struct mp_fp8set mp_fp8set;    /* per-tensor FP8 outputs of the fused AdamW (device) */
typedef void* mp_stream;               /* hipStream_t */

/* Dynamic loss scaler ("Mixed precision ...", section 2 "Dynamic scaling";
 * "Megatron Internals III", section 5).  init_scale, growth, backoff,
 * min_scale and max_scale must be positive powers of two with growth >= 1,
 * backoff <= 1 and min_scale <= init_scale <= max_scale; interval >= 1.
 * enabled = 0 keeps S fixed at init_scale (bf16 needs no scaler). */
typedef struct {
    float init_scale;
    float growth;
    float backoff;
    float min_scale;
    float max_scale;
    int32_t interval;
    int32_t enabled;
} mp_scaler_cfg;

/* AdamW hyper-parameters: lr >= 0, 0 <= beta1, beta2 < 1, eps > 0,
 * weight_decay >= 0 (all finite). */
typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
} mp_adamw_hparams;

/* What the device knows after a step (read with mp_state_read). */
typedef struct {
    int32_t found_inf;      /* the last unscale/check saw an inf or NaN */
    int32_t skipped;        /* the last scaler update recorded a skipped step */
    int32_t good_steps;     /* clean steps since the scale last changed */
    int32_t reserved0;
    int64_t step;           /* committed optimizer steps t */
    int64_t skipped_total;  /* skipped steps so far */
    double sumsq;           /* sum of squares of the unscaled gradient (fp64) */
    double beta1_pow;       /* beta1^t */
    double beta2_pow;       /* beta2^t */
    float scale;            /* the loss scale S the next step uses */
    float grad_norm;        /* fp32(sqrt(sumsq)) */
    float clip_coef;        /* min(1, max_norm / (grad_norm + 1e-6)), or 1 */
    float reserved1;
} mp_stats;

/* Human-readable name of a status code (static storage). */
const char* mp_status_string(mp_status status);

/* Detail of the last error returned to the calling thread ("" if none). */
const char* mp_last_error(void);

int32_t mp_abi_version(void);

/* Token weights ("Accumulate gradients and recompute activations", "Weight
 * each mean by the targets it represents"; counts validated as in "Extend the
 * existing update and reverse owners"): weights_out[i] = fp32(n_i / N) with
 * N = sum of counts, computed in binary64 then rounded once.  Host-only.
 * MP_ERR_INVALID if k < 1, any n_i <= 0, or N > 2^53. */
mp_status mp_token_weights(int32_t k, const int64_t* counts, float* weights_out);

/* mp_token_weights on the device, for counts that the data pipeline leaves in
 * device memory: no host round trip, and a captured graph reads the counts of
 * each replay.  `counts` (k int64, 8-byte aligned) and `weights_out` (k fp32,
 * 4-byte aligned) are device pointers owned by the caller; one small kernel on
 * `stream` writes weights_out[i] = fp32(n_i / N) with the same binary64
 * division as the host call, so both give the same bits.  Counts the host call
 * would refuse (any n_i <= 0, N > 2^53) cannot be refused here without a
 * sync: every weight is then NaN, the gradient they scale is non-finite, and
 * the step is skipped and the scale backed off exactly as on an overflow.
 * MP_ERR_INVALID if k < 1 or a pointer is NULL, MP_ERR_ALIGN if misaligned. */
mp_status mp_token_weights_dev(int32_t k, const int64_t* counts, float* weights_out,
                               mp_stream stream);

/* Model-state bytes per parameter ("Chapter 41 Training at Scale", equation
 * (41.1)): 16-bit weight 2 + 16-bit gradient 2 + fp32 master 4 + m 4 + v 4 =
 * 16, plus 4 for the fp32 accumulation buffer when with_accumulator != 0.
 * The 16-bit weight and gradient are 2 bytes in both formats. */
size_t mp_state_bytes_per_param(mp_dtype16 dtype, int32_t with_accumulator);

/* Describe the parameter tensors of one model.  For tensor i (1 <= numel[i]
 * <= 2^40 elements, contiguous; at most 2^48 in all): acc[i] fp32
 * accumulation buffer, master[i] fp32
 * master weight, m[i] and v[i] fp32 Adam moments, w16[i] the 16-bit model
 * weight.  `acc` may be NULL when the model is never accumulated (one
 * micro-batch per update: pass it as the last micro-batch with
 * last_is_first = 1).  wd_mult[i] >= 0 multiplies weight_decay for tensor i
 * (NULL: all 1).  Builds the chunk table and uploads it (synchronously).
 * On success *out owns device memory until mp_plan_destroy. */
mp_status mp_plan_create(int32_t n_tensors, const int64_t* numel, mp_dtype16 dtype,
                         void* const* acc, void* const* master, void* const* m,
                         void* const* v, void* const* w16, const float* wd_mult,
                         mp_plan** out);
mp_status mp_plan_destroy(mp_plan* plan);

/* Tensor and chunk counts of a plan (any output may be NULL). */
mp_status mp_plan_info(const mp_plan* plan, int32_t* n_tensors, int64_t* total_params,
                       int64_t* n_chunks, int32_t* chunk_elems);

/* The chunk table mp_plan_create builds for `numel` on a device with n_cus
 * compute units, computed on the host (no device needed).  Every tensor is cut
 * into contiguous chunks of at most *chunk_elems elements (a power-of-two
 * multiple of 2048; the last chunk of a tensor is ragged), tensor by tensor.
 * Writes *n_chunks and up to `capacity` entries of (tensor index, start
 * element, length) into the optional output arrays. */
mp_status mp_chunk_layout(int32_t n_tensors, const int64_t* numel, int32_t n_cus,
                          int32_t* chunk_elems, int64_t* n_chunks, int32_t* tensor_out,
                          int64_t* start_out, int32_t* len_out, int64_t capacity);

/* One micro-batch's 16-bit gradients: g16[i] points at numel[i] elements of
 * the plan's 16-bit format, in the caller's device memory.  The pointer list
 * is uploaded once (synchronously), so a gradset can be reused every step.
 * Destroy a gradset only after the stream work that uses it has finished. */
mp_status mp_gradset_create(const mp_plan* plan, void* const* g16, mp_gradset** out);
mp_status mp_gradset_destroy(mp_gradset* set);

/* Point an existing gradset at other gradient buffers (same plan, same rules
 * as mp_gradset_create), for callers whose gradient tensors move between
 * steps (e.g. freed and reallocated by the framework).  Allocates nothing: the
 * new pointer list is written into one of 4 pinned host slots owned by the
 * gradset and copied to the device on `stream`, so work enqueued on `stream`
 * after this call sees the new buffers and work enqueued before it the old
 * ones.  Before rewriting a slot the call waits until the copy that last read
 * it has run, so the host can run at most 4 updates ahead of the device.
 * Refused (MP_ERR_INVALID) while `stream` is being captured into a graph: a
 * replay would copy whatever the slot holds at replay time.  A norm measured
 * (mp_unscale_check_norm, mp_norm_partial and their group forms) with this
 * gradset folded in no longer describes it: the AdamW step that would follow
 * returns MP_ERR_ORDER until the norm is measured again. */
mp_status mp_gradset_update(mp_gradset* set, void* const* g16, mp_stream stream);

/* Device state: S = init_scale, no good steps, t = 0, beta powers 1. */
mp_status mp_state_create(const mp_scaler_cfg* cfg, mp_state** out);
mp_status mp_state_destroy(mp_state* state);

/* Save and restore the device state: loss scale, clean-step count, scaler
 * configuration, optimizer step t and the beta powers ("Mixed precision ...",
 * section 4 "The interface": state_dict / load_state_dict; section 5, pitfall
 * 16: a resume that loses the count grows S late).  The fp32 masters, moments
 * and 16-bit weights are the caller's buffers and are saved by the caller.
 * A blob is MP_STATE_BLOB_BYTES bytes of host memory.
 *  - export: writes the header at once and enqueues the copy of the device
 *    state; the blob is complete once `stream` has reached this point.
 *  - import: checks the header and every field on the host (MP_ERR_INVALID
 *    for a foreign blob, another version, or out-of-range fields, leaving the
 *    state untouched), then copies it to the device and waits for `stream`.
 *    Call it between steps. */
#define MP_STATE_BLOB_BYTES 256
mp_status mp_state_export(const mp_state* state, void* blob, size_t blob_bytes, mp_stream stream);
mp_status mp_state_import(mp_state* state, const void* blob, size_t blob_bytes, mp_stream stream);

/* Enqueue a copy of the state into *out (host memory; pinned memory keeps the
 * call asynchronous).  *out is valid once `stream` has reached this point. */
mp_status mp_state_read(const mp_state* state, mp_stats* out, mp_stream stream);

/* Device address of S (fp32), so the caller can scale its loss on the device
 * ("Megatron Internals III", section 4: scaled_loss = S * loss). */
mp_status mp_state_scale_ptr(const mp_state* state, const float** dev_scale);

/* Accumulate one micro-batch ("Mixed precision ...", section 2 "Gradient
 * accumulation"; "Megatron Internals III", section 8): for every element,
 *   first != 0:  acc = fl(weight * widen(g16))
 *   first == 0:  acc = fl(acc + fl(weight * widen(g16)))
 * where widen is the exact 16-bit -> fp32 conversion and weight = n_i/N from
 * mp_token_weights (finite, > 0).  `first` starts a new logical update and
 * discards whatever the buffer held (the gradients of a skipped step).
 * MP_ERR_INVALID if the plan has no accumulators.  The call changes the
 * gradient a preceding mp_unscale_check_norm / mp_norm_partial measured, so the
 * next mp_adamw_step on this plan returns MP_ERR_ORDER until the norm is
 * measured again. */
mp_status mp_accumulate(mp_plan* plan, const mp_gradset* g16, float weight, int32_t first,
                        mp_stream stream);

/* Accumulate n resident micro-batches (1 <= n <= 4) in one pass, for a caller
 * that keeps several micro-batch gradients in device memory at once.  The
 * result is bit for bit that of n mp_accumulate calls in array order (the
 * first with `first`, the rest with first = 0), since every term is added with
 * the same two roundings, in the same order, while the running sum stays in a
 * register.  The accumulator is read once (not at all when first != 0) and
 * written once, so the pass moves 2n + 8 bytes per parameter (2n + 4 when
 * first) instead of 10n (10n - 4).
 *   sets:    n gradsets of this plan, in micro-batch order (host array);
 *   weights: n weights, a host array, or when weights_on_device != 0 a device
 *            array of n fp32 (4-byte aligned, e.g. part of the output of
 *            mp_token_weights_dev), read when the kernel runs.
 * MP_ERR_INVALID if n is out of range, an argument is NULL, a gradset belongs
 * to another plan or the plan has no accumulators. */
mp_status mp_accumulate_group(mp_plan* plan, const mp_gradset* const* sets, const float* weights,
                              int32_t n, int32_t weights_on_device, int32_t first,
                              mp_stream stream);

/* The token weights ("Accumulate gradients and recompute activations", "Weight
 * each mean by the targets it represents") computed inside the first
 * accumulation of an update: one launch instead of two, with the same results,
 * bit for bit, as
 *   mp_token_weights_dev(k, counts, weights_out);
 *   mp_accumulate_group(plan, sets, weights_out, n, 1, first = 1);
 * Every block of the pass computes the weights of micro-batches 0..n-1 from
 * the k counts itself (k int64 scalar reads), and one block writes all k
 * weights to weights_out, where the later passes of the update read them
 * (group calls with weights_on_device).
 *   sets:        the n gradsets of micro-batches 0..n-1 (host array, 1 <= n <= 4);
 *   counts:      k int64 in device memory (8-byte aligned), n <= k <= 64;
 *   weights_out: k fp32 in device memory (4-byte aligned);
 * both device arrays are the caller's.  Counts that mp_token_weights would
 * refuse give NaN weights, as in mp_token_weights_dev.  MP_ERR_INVALID if n or
 * k is out of range, a pointer is NULL, a gradset belongs to another plan or
 * the plan has no accumulators; MP_ERR_ALIGN if a device array is misaligned. */
mp_status mp_accumulate_first_counts(mp_plan* plan, const mp_gradset* const* sets, int32_t n,
                                     int32_t k, const int64_t* counts, float* weights_out,
                                     mp_stream stream);

/* Unscale, check and measure ("Megatron Internals III", sections 4, 6 and 9;
 * "Mixed precision ...", section 2 "Dynamic scaling").  The gradient of each
 * element is g_eff = acc (last == NULL), fl(w_last * widen(last))
 * (last_is_first != 0), or fl(acc + fl(w_last * widen(last))) -- the last
 * micro-batch folded in exactly as mp_accumulate would add it.  Then
 *   g = fl(g_eff * (1/S));  found_inf = any g is inf or NaN;
 *   sumsq = sum g^2 in binary64 (a fixed-order reduction: per block of
 *           chunks -- one chunk, or sixteen when the pass reads a single
 *           16-bit stream and no accumulator -- then 256 contiguous range
 *           sums, then one total; the same bits on every run);
 *   grad_norm = fp32(sqrt(sumsq));
 *   clip_coef = min(1, fl(max_norm / fl(grad_norm + 1e-6))) if max_norm > 0
 *               and !found_inf, else 1.
 * Results stay on the device for mp_adamw_step and mp_state_read. */
mp_status mp_unscale_check_norm(mp_plan* plan, mp_state* state, const mp_gradset* last,
                                float w_last, int32_t last_is_first, float max_norm,
                                mp_stream stream);

/* The two halves of mp_unscale_check_norm, for a model whose parameters are
 * sharded over ranks (ZeRO-1/2: each rank's plan covers its slice).  The norm
 * must cover every shard ("Megatron Internals III", section 9: local squared
 * norms reduced over the owning ranks; "Your weights fit on one device...",
 * "Operational sharp edges: Gradient clipping"), and every rank must take the
 * same skip decision (section 6).  One all-reduce of one binary64 value does
 * both: an inf/NaN anywhere makes the sum non-finite.
 *  - mp_norm_partial: writes this plan's fixed-order binary64 sum of squares
 *    of g = g_eff/S (same g_eff as mp_unscale_check_norm) to partial_out, one
 *    double in device memory.
 *  - mp_norm_finish: from *sumsq (device; the sum over ranks, reduced in a
 *    fixed rank order by the caller) sets found_inf = !isfinite(sumsq),
 *    grad_norm and clip_coef exactly as mp_unscale_check_norm does.  Must
 *    follow mp_norm_partial on the same plan and state (else MP_ERR_ORDER);
 *    mp_adamw_step may follow it as it follows mp_unscale_check_norm. */
mp_status mp_norm_partial(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                          int32_t last_is_first, double* partial_out, mp_stream stream);
mp_status mp_norm_finish(mp_plan* plan, mp_state* state, const double* sumsq, float max_norm,
                         mp_stream stream);

/* AdamW + RNE cast ("Your weights fit on one device...", the Adam update;
 * "Accumulate gradients...", decoupled decay; "Mixed precision ...", section 2
 * "Why the weights stay float32"; "Megatron Internals III", section 9 steps
 * 5-7).  Must follow mp_unscale_check_norm on the same plan and state with the
 * same last/w_last/last_is_first (else MP_ERR_ORDER).  If found_inf: nothing
 * is written and t, beta powers stay (the skipped step of "Discard a failed
 * partial logical update").  Otherwise, with t' = t + 1, p_j = beta_j^t',
 * bc_j = fp32(1 - p_j), scale = fl((1/S) * clip_coef), lambda = weight_decay
 * * wd_mult[tensor], every element takes, each operation rounded to fp32:
 *   gs = g_eff*scale;  m = b1*m + (1-b1)*gs;  v = b2*v + (1-b2)*(gs*gs);
 *   u = (m/bc1) / (sqrt(v/bc2) + eps);  w = w - lr*(u + lambda*w);
 *   w16 = round-to-nearest-even(w) in the plan's 16-bit format
 * (NaN -> the format's quiet NaN with the sign kept). */
mp_status mp_adamw_step(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                        int32_t last_is_first, const mp_adamw_hparams* hp, mp_stream stream);

/* Loss-scale decision after the step ("Mixed precision ...", section 2
 * "Dynamic scaling"; "Megatron Internals III", section 5): skipped = found_inf;
 * on overflow S = max(S*backoff, min_scale) and the count restarts; on a clean
 * step the count grows and, on reaching `interval`, S = min(S*growth,
 * max_scale) and the count restarts.  A disabled scaler keeps S.  Exactly one
 * call per measurement: it must follow mp_unscale_check_norm (or
 * mp_norm_finish) on this state, with no mp_scaler_update in between, else
 * MP_ERR_ORDER (a second call would count the same clean step twice).
 * mp_state_import leaves no measurement pending. */
mp_status mp_scaler_update(mp_state* state, mp_stream stream);

/* The whole update after the last micro-batch in one call: mp_unscale_check_norm,
 * mp_adamw_step and mp_scaler_update with the same arguments, enqueued in that
 * order on `stream` -- the scaler's step of "Mixed precision ...", section 4
 * "The interface" (check, unscale, clip, optimizer step, update S).  Every
 * structural check of the three calls is made before anything is enqueued.
 * Here the norm's finishing block also advances the optimizer clock and takes
 * the scaler's decision (both depend only on the overflow flag), so the call
 * enqueues the norm pass, its finish and the AdamW pass and nothing else. */
mp_status mp_update_step(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                         int32_t last_is_first, float max_norm, const mp_adamw_hparams* hp,
                         mp_stream stream);

/* mp_update_step for callers that cannot allocate device memory while they
 * run: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, checks, order rules and results as
 * mp_update_step, but the norm pass keeps its partial sums in a static device
 * array of the library (MP_NOALLOC_MAX_NORM_BLOCKS + 256 doubles, about 2 MB,
 * one copy per device held until the process ends) instead of the plan's own
 * buffer, and the call allocates nothing.  The norm's first stage takes one
 * partial per block; a plan whose norm pass takes more than
 * MP_NOALLOC_MAX_NORM_BLOCKS blocks is refused with MP_ERR_INVALID before
 * anything is enqueued (one block per chunk of 2048 elements, or per 16 chunks
 * when the pass reads the last micro-batch alone: plans of up to about 537M
 * parameters, or 8.6G with last_is_first).  Each launch writes every partial it
 * later reads, so nothing needs clearing between calls.  All calls on one
 * device share that one array: calls that may overlap on a device (two streams,
 * two threads) race and must be serialised by the caller.  The plan's device
 * address of the array is looked up when the plan is created. */
#define MP_NOALLOC_MAX_NORM_BLOCKS 262144
mp_status mp_update_step_noalloc(mp_plan* plan, mp_state* state, const mp_gradset* last,
                                 float w_last, int32_t last_is_first, float max_norm,
                                 const mp_adamw_hparams* hp, mp_stream stream);

/* mp_update_step with the last n micro-batches (1 <= n <= 4) resident and all
 * folded into the norm pass and the AdamW pass, as `last` is folded in for
 * n = 1.  The gradient of each element is the accumulator (skipped when
 * last_is_first != 0, so that with k <= 4 micro-batches no accumulator is
 * needed at all) followed by the n terms in array order, each added with the
 * roundings of mp_accumulate: bit for bit the gradient mp_update_step sees
 * after accumulating all but the last micro-batch one by one.  Per parameter,
 * the norm pass reads 4 + 2n bytes (2n with last_is_first) and AdamW 30 + 2n
 * (26 + 2n) bytes, so k = 4 micro-batches cost 42 bytes in all, against 64 for
 * the one-at-a-time schedule.  sets and weights as in mp_accumulate_group.
 * Same checks, order and results as mp_update_step. */
mp_status mp_update_step_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                               const float* weights, int32_t n, int32_t weights_on_device,
                               int32_t last_is_first, float max_norm, const mp_adamw_hparams* hp,
                               mp_stream stream);

/* The two halves of mp_update_step_group before the scaler, for callers that
 * time or interleave them: mp_unscale_check_norm and mp_adamw_step over the
 * same group (same sets, weights and last_is_first, else MP_ERR_ORDER, as for
 * the single-`last` forms).  With n = 1 and weights_on_device these are the
 * single-`last` calls with the weight read on the device. */
mp_status mp_unscale_check_norm_group(mp_plan* plan, mp_state* state,
                                      const mp_gradset* const* sets, const float* weights,
                                      int32_t n, int32_t weights_on_device, int32_t last_is_first,
                                      float max_norm, mp_stream stream);
mp_status mp_adamw_step_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                              const float* weights, int32_t n, int32_t weights_on_device,
                              int32_t last_is_first, const mp_adamw_hparams* hp, mp_stream stream);

/* mp_norm_partial over a group of resident micro-batches, for a sharded model
 * (ZeRO-1/2) whose ranks fold their micro-batches in groups: the partial sum
 * of squares of the same gradient mp_unscale_check_norm_group measures.  Then
 * mp_norm_finish, and mp_adamw_step_group with the same group. */
mp_status mp_norm_partial_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                                const float* weights, int32_t n, int32_t weights_on_device,
                                int32_t last_is_first, double* partial_out, mp_stream stream);

/* Elementwise casts with the step's conversions: dst = round-to-nearest-even
 * of src into the 16-bit format (as in mp_adamw_step), and dst = exact fp32
 * value of a 16-bit pattern (as in mp_accumulate).  Useful to initialise the
 * 16-bit weights from the masters.  n >= 0; buffers 16-byte aligned. */
mp_status mp_cast_to_16(const float* src, uint16_t* dst, int64_t n, mp_dtype16 dtype,
                        mp_stream stream);
mp_status mp_widen_16(const uint16_t* src, float* dst, int64_t n, mp_dtype16 dtype,
                      mp_stream stream);

/* Fine-grained FP8 cast ("Chapter 41 Training at Scale", section 41.5,
 * listing 41.5), e.g. of the updated fp32 masters for an FP8 forward pass.
 * For each block of `block` consecutive values (block a multiple of 16 in
 * [16, 1024]; n a multiple of block, else MP_ERR_INVALID):
 *   scales[b] = fl(max|x| / 448), or 1 for an all-zero block; the maximum
 *   propagates NaN as the listing's NumPy maximum does, so a block holding a
 *   NaN gets the quiet NaN 0x7FC00000 as its scale;
 *   codes[i]  = E4M3(fl(x_i / scales[b])): 1 sign, 4 exponent bits (bias 7),
 *   3 mantissa bits, round to nearest even, saturating at 448 (E4M3 has no
 *   infinity), NaN -> S.1111.111.  A NaN quotient (every value of a NaN-scale
 *   block, or inf / inf in a block whose maximum is infinite) takes the sign
 *   bit of x_i, IEEE 754 leaving the sign of a NaN result open.
 * Dequantisation is value(codes[i]) * scales[b].  src and codes 16-byte
 * aligned, scales 4-byte aligned; n/block scales are written. */
mp_status mp_cast_fp8_blocks(const float* src, uint8_t* codes, float* scales, int64_t n,
                             int32_t block, mp_stream stream);

/* FP8 outputs for chosen tensors of a plan, for mp_adamw_step_fp8 ("Chapter
 * 41 Training at Scale", section 41.5: FP8 copies kept for storage or
 * transfer, each block of values with its own scale).  For tensor i either both
 * codes[i] (numel[i] bytes, 16-byte aligned) and scales[i] (numel[i]/16
 * floats, 4-byte aligned) are device pointers the caller owns, or both are
 * NULL and the tensor is not cast.  A cast tensor needs numel[i] % 16 == 0;
 * at least one tensor must be cast (else MP_ERR_INVALID). */
mp_status mp_fp8set_create(const mp_plan* plan, void* const* codes, void* const* scales,
                           mp_fp8set** out);
mp_status mp_fp8set_destroy(mp_fp8set* set);

/* mp_adamw_step with the FP8 cast of the new weights fused into the same pass:
 * everything mp_adamw_step writes, bit for bit, and for every cast tensor of
 * `fp8` the codes and scales that mp_cast_fp8_blocks with block = 16 would
 * write for the new fp32 masters.  The masters are cast while they are in
 * registers, so the cast costs its 1.25 bytes/param of writes, not a second
 * 4-byte read.  Same order rules as mp_adamw_step; on a skipped step
 * (found_inf) nothing is written, the FP8 outputs included. */
mp_status mp_adamw_step_fp8(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                            int32_t last_is_first, const mp_adamw_hparams* hp,
                            const mp_fp8set* fp8, mp_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MPSTEP_H */
