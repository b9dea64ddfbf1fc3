/*
 * Oracle for the mixed-precision update step -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU implementation of what the step computes, written
 * from the pages' definitions.  It exists so that tests, the smoke check and
 * the CPU-baseline leg of the benchmark have something independent to compare
 * the HIP library against.  No product code may link, load or call it, and it
 * shares no source with the HIP library.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math (x86-64 SSE math,
 * so every float operation below is one IEEE-754 round-to-nearest-even
 * operation in binary32, and every double operation one in binary64).
 *
 * Sources (the text of the pages, cited by title and section):
 *  [MP]  "Mixed precision, loss scaling, gradient accumulation, and activation
 *        checkpointing" (course module L11.1): section 2 "Principles"
 *        (Two 16-bit formats; Why the weights stay float32; Loss scaling;
 *        Dynamic scaling; Gradient accumulation), section 3 "Worked example by
 *        hand", section 4 "The interface".
 *  [MEG] "Megatron Internals III: Mixed Precision, Loss Scaling, and Grad
 *        Clipping": section 4 (loss scaling equation), section 5 (dynamic loss
 *        scaling controller), section 8 (copying gradients), section 9
 *        (global-norm clipping and the order of operations).
 *  [ZQ]  "Your weights fit on one device but Adam's moments do not -- how do
 *        you shard the optimizer state?": "Why the optimizer state is the
 *        thing that overflows" (the Adam update in words).
 *  [RS]  "Accumulate gradients and recompute activations" (Practical LLM in
 *        Rust, chapter 13): "Weight each mean by the targets it represents"
 *        (token-weighted accumulation equations), "Extend the existing update
 *        and reverse owners" (count validation), "Discard a failed partial
 *        logical update" (what a skipped update preserves).
 *  [TS]  "Chapter 41 Training at Scale": section 41.1, equation (41.1);
 *        section 41.5, fine-grained FP8 scaling (listing 41.5).
 *
 * Readings where the pages are silent, ambiguous or leave a detail open:
 *  - AdamW: the pages describe it only in words ([ZQ]); the per-element
 *    sequence in or_adamw_tensor is the standard decoupled AdamW with the bias
 *    corrections applied to m and v, epsilon added after the square root, and
 *    decay lr*lambda*w on the pre-update weight.
 *  - Backoff multiplies S by the backoff factor 1/2 ([MP] "Dynamic scaling");
 *    [MEG] section 5 prints a division, which only agrees if its factor is 2.
 *  - Clip coefficient min(1, c/(norm + 1e-6)); [MEG] section 9 leaves eps open.
 *  - bias corrections use running products of beta in binary64, advanced only
 *    on committed steps ([RS]: a skipped attempt keeps the "beta powers").
 *  - NaN inputs to the 16-bit rounding give the format's quiet NaN with the
 *    sign kept; the payload is not specified by the pages.
 *  - FP8: the chapter's E4M3 emulator is not printed; or_e4m3 rounds to
 *    nearest, ties to even, saturates at the largest finite value 448 (E4M3
 *    has no infinity), and maps NaN to S.1111.111.
 *  - FP8 blocks holding a NaN: the listing's maximum propagates NaN, so the
 *    block's scale is NaN (the quiet NaN 0x7FC00000) and each of its codes is
 *    the NaN code with the sign bit of its value; a NaN quotient of inf / inf
 *    takes the value's sign too.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* 16-bit formats ([MP] section 2 "Two 16-bit formats").                     */
/* p = significant bits, bias = exponent bias; emin = 1 - bias is the        */
/* exponent of the smallest normal number, emax = bias the largest.          */
/* ------------------------------------------------------------------------ */
enum { OR_BF16 = 0, OR_FP16 = 1 };

typedef struct {
    int p;      /* precision in bits: 8 for bf16, 11 for fp16 */
    int ebits;  /* exponent field width: 8 for bf16, 5 for fp16 */
    int bias;   /* 127 for bf16, 15 for fp16 */
} or_format;

static or_format or_fmt(int dtype)
{
    or_format f;
    if (dtype == OR_BF16) { f.p = 8;  f.ebits = 8; f.bias = 127; }
    else                  { f.p = 11; f.ebits = 5; f.bias = 15;  }
    return f;
}

/* Largest finite value: (2 - 2^(1-p)) * 2^emax. */
static double or_max_finite(or_format f)
{
    return ldexp(2.0 - ldexp(1.0, 1 - f.p), f.bias);
}

/* Encode a value that is exactly representable in the format (or +-inf). */
static uint16_t or_encode(or_format f, double y, int negative)
{
    uint16_t sign = negative ? (uint16_t)(1u << 15) : 0;
    int mbits = f.p - 1;
    uint16_t emask = (uint16_t)(((1u << f.ebits) - 1u) << mbits);
    double a = fabs(y);
    if (isinf(a)) return (uint16_t)(sign | emask);
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);                 /* a = fr * 2^E, fr in [0.5, 1) */
    int e = E - 1;                /* a in [2^e, 2^(e+1)) */
    int emin = 1 - f.bias;
    if (e >= emin) {
        double frac = a / ldexp(1.0, e) - 1.0;           /* in [0, 1) */
        uint32_t mant = (uint32_t)(frac * ldexp(1.0, mbits));
        uint32_t efield = (uint32_t)(e + f.bias);
        return (uint16_t)(sign | (efield << mbits) | mant);
    }
    /* subnormal: value = mant * 2^(emin - mbits) */
    uint32_t mant = (uint32_t)(a / ldexp(1.0, emin - mbits));
    return (uint16_t)(sign | mant);
}

/*
 * rd16: round an fp32 value to the nearest value of the 16-bit format, ties to
 * even ([MP] section 2, the symbol rd16; section 3 "A bf16 matmul" shows the
 * tie 1 + 2^-8 -> 1 and 1.01 -> 1.0078125).  Written from the definition: the
 * representable numbers around |x| are the integer multiples of the quantum
 * 2^(e - p + 1) of x's binade (fixed at the subnormal quantum below the normal
 * range); pick the nearest multiple, ties to an even multiple, and overflow to
 * infinity when the nearest value is beyond the largest finite number.
 */
uint16_t or_rd16(float x, int dtype)
{
    or_format f = or_fmt(dtype);
    int negative = signbit(x) != 0;
    int mbits = f.p - 1;
    if (isnan(x)) {
        uint16_t emask = (uint16_t)(((1u << f.ebits) - 1u) << mbits);
        uint16_t quiet = (uint16_t)(1u << (mbits - 1));
        return (uint16_t)((negative ? 0x8000u : 0u) | emask | quiet);
    }
    double X = (double)x;                  /* exact */
    if (isinf(X) || X == 0.0) return or_encode(f, X, negative);
    int E;
    frexp(fabs(X), &E);
    int e = E - 1;
    int emin = 1 - f.bias;
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - mbits);
    double r = nearbyint(X / quantum);     /* default mode: nearest, ties to even */
    double Y = r * quantum;                /* exact */
    if (fabs(Y) > or_max_finite(f)) Y = negative ? -INFINITY : INFINITY;
    return or_encode(f, Y, negative);
}

/*
 * widen: the exact fp32 value of a 16-bit pattern (every bf16 and fp16 value,
 * subnormals included, is an fp32 value).  Decoded from the fields:
 * (-1)^s * 1.m * 2^(E - bias) for normals, 0.m * 2^emin for subnormals.
 * A NaN keeps its sign and its payload at the top of the fp32 mantissa.
 */
float or_widen16(uint16_t h, int dtype)
{
    or_format f = or_fmt(dtype);
    int mbits = f.p - 1;
    uint32_t s = (h >> 15) & 1u;
    uint32_t E = (h >> mbits) & ((1u << f.ebits) - 1u);
    uint32_t M = h & ((1u << mbits) - 1u);
    if (E == (1u << f.ebits) - 1u) {
        if (M == 0) return s ? -INFINITY : INFINITY;
        uint32_t bits = (s << 31) | (0xFFu << 23) | (M << (23 - mbits));
        float out;
        memcpy(&out, &bits, sizeof out);
        return out;
    }
    double v;
    if (E == 0) v = ldexp((double)M, 1 - f.bias - mbits);
    else        v = ldexp(1.0 + ldexp((double)M, -mbits), (int)E - f.bias);
    return (float)(s ? -v : v);            /* exact: v has <= 11 significant bits */
}

void or_rd16_array(const float* x, uint16_t* y, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) y[i] = or_rd16(x[i], dtype);
}

void or_widen16_array(const uint16_t* h, float* y, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) y[i] = or_widen16(h[i], dtype);
}

/* ------------------------------------------------------------------------ */
/* Token weights ([RS] "Weight each mean by the targets it represents":       */
/* N = sum n_i, weight n_i / N; "Extend the existing update and reverse       */
/* owners": every micro-batch has targets, the total is positive and at most  */
/* 2^53 so it converts to binary64 exactly).                                  */
/* Returns 0 on success, -1 when the counts are refused.                      */
/* ------------------------------------------------------------------------ */
int or_token_weights(int32_t k, const int64_t* n, float* w)
{
    if (k <= 0) return -1;
    int64_t total = 0;
    for (int32_t i = 0; i < k; ++i) {
        if (n[i] <= 0) return -1;
        if (n[i] > ((int64_t)1 << 53) - total) return -1;
        total += n[i];
    }
    for (int32_t i = 0; i < k; ++i)
        w[i] = (float)((double)n[i] / (double)total);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Accumulation ([MP] "Gradient accumulation": the gradient of the batch is   */
/* sum_i (n_i/N) grad L_i, added into the gradient buffer without zeroing in  */
/* between; [MEG] section 8: the 16-bit gradient is cast to fp32 and placed   */
/* in the fp32 main-gradient buffer).                                         */
/* first != 0: acc = w * widen(g16); otherwise acc = acc + w * widen(g16).    */
/* ------------------------------------------------------------------------ */
void or_accumulate_tensor(const uint16_t* g16, float* acc, int64_t n, int dtype,
                          float w, int first)
{
    for (int64_t j = 0; j < n; ++j) {
        float a = or_widen16(g16[j], dtype);
        float contribution = w * a;
        if (first) acc[j] = contribution;
        else       acc[j] = acc[j] + contribution;
    }
}

/*
 * The gradient one element carries into the update, when the last micro-batch
 * is still in 16-bit form: the same two operations as or_accumulate_tensor,
 * so that folding the last micro-batch into the later passes and running the
 * accumulation first give the same fp32 gradient.
 *   mode 0: acc[j]               (every micro-batch already accumulated)
 *   mode 1: w * widen(g16[j])    (the last micro-batch is the only one)
 *   mode 2: acc[j] + w * widen(g16[j])
 */
static float or_effective_grad(const float* acc, const uint16_t* g16, int64_t j,
                               int dtype, float w, int mode)
{
    if (mode == 0) return acc[j];
    float contribution = w * or_widen16(g16[j], dtype);
    if (mode == 1) return contribution;
    return acc[j] + contribution;
}

/* ------------------------------------------------------------------------ */
/* Unscale, overflow check and the tensor's squared norm                     */
/* ([MEG] section 4: grad = scaled_grad / S; [MP] "Loss scaling": S is a     */
/* power of two, so dividing by it is exact; [MP] "Dynamic scaling": any     */
/* non-finite gradient poisons the step; [MEG] section 9: the global norm is  */
/* sqrt(sum_i ||grad_i||^2)).                                                 */
/* g = acc * (1/S).  The squares are formed in binary64 (exact for fp32       */
/* inputs) and summed with Neumaier's compensated summation, which is         */
/* accurate to a few binary64 roundings regardless of length.                 */
/* Writes the tensor's sum of squares; returns 1 if any g is inf or NaN.      */
/* ------------------------------------------------------------------------ */
typedef struct { double sum, comp; } or_ksum;

static void or_ksum_add(or_ksum* k, double t)
{
    double s = k->sum + t;
    if (!isfinite(s)) { k->sum = s; return; }      /* inf/NaN just propagate */
    if (fabs(k->sum) >= fabs(t)) k->comp += (k->sum - s) + t;
    else                         k->comp += (t - s) + k->sum;
    k->sum = s;
}

static double or_ksum_value(const or_ksum* k)
{
    return isfinite(k->sum) ? k->sum + k->comp : k->sum;
}

int or_unscale_sumsq_tensor(const float* acc, const uint16_t* g16, int64_t n, int dtype,
                            float w_last, int mode, float inv_scale, double* sumsq_out)
{
    or_ksum k = {0.0, 0.0};
    int found_inf = 0;
    for (int64_t j = 0; j < n; ++j) {
        float g = or_effective_grad(acc, g16, j, dtype, w_last, mode) * inv_scale;
        if (!isfinite(g)) found_inf = 1;
        double gd = (double)g;
        or_ksum_add(&k, gd * gd);
    }
    *sumsq_out = or_ksum_value(&k);
    return found_inf;
}

/* 1/S, exact for a power-of-two S ([MP] "Loss scaling"). */
float or_unscale_factor(float scale)
{
    return 1.0f / scale;
}

/* The factor applied to each fp32 gradient before the moments: (1/S) * coef
 * ([MEG] section 9, steps 3 and 5: unscale, then clip with the global
 * coefficient). */
float or_update_scale(float scale, float coef)
{
    return (1.0f / scale) * coef;
}

/* Per-tensor decoupled weight decay lambda_t = weight_decay * multiplier. */
float or_decay(float weight_decay, float multiplier)
{
    return weight_decay * multiplier;
}

/* Combine per-tensor (or per-segment) sums of squares in the order given. */
double or_sum_in_order(const double* parts, int64_t count)
{
    or_ksum k = {0.0, 0.0};
    for (int64_t i = 0; i < count; ++i) or_ksum_add(&k, parts[i]);
    return or_ksum_value(&k);
}

/*
 * Global norm and clip coefficient ([MEG] section 9: clip_coef =
 * max_norm / (global_norm + eps); [MP] "Dynamic scaling": clipping comes after
 * unscaling, so the bound is in true gradient units).
 * norm = fp32(sqrt(sumsq)); when max_norm > 0 and no overflow,
 * coef = min(1, max_norm / (norm + 1e-6)); otherwise coef = 1.
 */
void or_norm_and_coef(double sumsq, int found_inf, float max_norm,
                      float* norm_out, float* coef_out)
{
    float norm = (float)sqrt(sumsq);
    float coef = 1.0f;
    if (max_norm > 0.0f && !found_inf) {
        float q = max_norm / (norm + 1e-6f);
        coef = q < 1.0f ? q : 1.0f;
    }
    *norm_out = norm;
    *coef_out = coef;
}

/* ------------------------------------------------------------------------ */
/* Optimizer step bookkeeping: t and the running beta powers.                */
/* ------------------------------------------------------------------------ */
typedef struct {
    int64_t t;      /* committed optimizer steps */
    double  p1;     /* beta1^t */
    double  p2;     /* beta2^t */
} or_adam_clock;

/* Bias corrections of the step about to be taken (t + 1). */
void or_bias_corrections(const or_adam_clock* c, float beta1, float beta2,
                         float* bc1, float* bc2)
{
    double p1 = c->p1 * (double)beta1;
    double p2 = c->p2 * (double)beta2;
    *bc1 = (float)(1.0 - p1);
    *bc2 = (float)(1.0 - p2);
}

void or_clock_advance(or_adam_clock* c, float beta1, float beta2)
{
    c->t += 1;
    c->p1 = c->p1 * (double)beta1;
    c->p2 = c->p2 * (double)beta2;
}

/*
 * AdamW on one tensor's fp32 master, m and v, then the RNE cast back to the
 * 16-bit model weight ([ZQ]: the update divides the bias-corrected first moment
 * by the square root of the bias-corrected second moment plus a small
 * constant; [RS]: decoupled weight decay; [MP] "Why the weights stay float32":
 * the master, the moments and the update are fp32 and only the model copy is
 * rounded; [MEG] section 9 steps 5-7: the clip coefficient scales the
 * unscaled gradient before the master step, then the master is copied back to
 * model precision).
 * Per element, every operation rounded to fp32:
 *   gs = g_eff * scale                      (scale = (1/S) * coef)
 *   m  = beta1*m + (1-beta1)*gs
 *   v  = beta2*v + (1-beta2)*(gs*gs)
 *   mh = m / bc1,  vh = v / bc2
 *   u  = mh / (sqrt(vh) + eps)
 *   w  = w - lr * (u + lambda*w)
 *   w16 = rd16(w)
 */
void or_adamw_tensor(const float* acc, const uint16_t* g16_last, int64_t n, int dtype,
                     float w_last, int mode, float scale,
                     float* master, float* m, float* v, uint16_t* w16,
                     float lr, float beta1, float beta2, float eps, float lambda,
                     float bc1, float bc2)
{
    float ob1 = 1.0f - beta1;
    float ob2 = 1.0f - beta2;
    for (int64_t j = 0; j < n; ++j) {
        float gs = or_effective_grad(acc, g16_last, j, dtype, w_last, mode) * scale;
        float mj = beta1 * m[j] + ob1 * gs;
        float vj = beta2 * v[j] + ob2 * (gs * gs);
        float mh = mj / bc1;
        float vh = vj / bc2;
        float den = sqrtf(vh) + eps;
        float u = mh / den;
        float w = master[j];
        w = w - lr * (u + lambda * w);
        m[j] = mj;
        v[j] = vj;
        master[j] = w;
        w16[j] = or_rd16(w, dtype);
    }
}

/* ------------------------------------------------------------------------ */
/* Dynamic loss scaler ([MP] "Dynamic scaling" and section 3 "Loss scaling"   */
/* table; [MEG] section 5 controller).                                       */
/* ------------------------------------------------------------------------ */
typedef struct {
    float   scale;         /* S */
    int32_t good_steps;    /* consecutive clean steps since the last change */
    float   growth, backoff, min_scale, max_scale;
    int32_t interval;
    int32_t enabled;       /* 0: S stays fixed (bf16 needs no scaler) */
    int32_t skipped;       /* the last step was skipped */
    int64_t skipped_total;
} or_scaler;

/*
 * After the step: an overflow skips it, multiplies S by the backoff (not below
 * min_scale) and restarts the count; a clean step counts, and after
 * `interval` clean steps S is multiplied by the growth factor (not above
 * max_scale) and the count restarts.
 */
void or_scaler_update(or_scaler* s, int found_inf)
{
    s->skipped = found_inf ? 1 : 0;
    if (found_inf) s->skipped_total += 1;
    if (!s->enabled) return;
    if (found_inf) {
        float next = s->scale * s->backoff;
        s->scale = next > s->min_scale ? next : s->min_scale;
        s->good_steps = 0;
    } else {
        s->good_steps += 1;
        if (s->good_steps == s->interval) {
            float next = s->scale * s->growth;
            s->scale = next < s->max_scale ? next : s->max_scale;
            s->good_steps = 0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Memory accounting ([TS] equation (41.1); [MEG] section 1 table; [MP] "Why  */
/* the weights stay float32"): 16-bit weight 2 + 16-bit gradient 2 + fp32    */
/* master 4 + fp32 m 4 + fp32 v 4 bytes per parameter.                        */
/* ------------------------------------------------------------------------ */
int64_t or_model_state_bytes(int64_t params)
{
    return params * (2 + 2 + 4 + 4 + 4);
}

/* ------------------------------------------------------------------------ */
/* Fine-grained FP8 scaling ([TS] section 41.5, listing 41.5): per block of  */
/* `block` values, scale = max|x| / 448 in fp32 (a zero block takes scale    */
/* 1), then every value x / scale is rounded to E4M3.                          */
/* E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities; the  */
/* largest finite value is 1.75 * 2^8 = 448 (S.1111.111 is NaN), the smallest */
/* normal 2^-6, the smallest subnormal 2^-9.                                   */
/* ------------------------------------------------------------------------ */
uint8_t or_e4m3(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    if (isnan(x)) return (uint8_t)(sign | 0x7F);
    double X = fabs((double)x);
    if (X == 0.0) return sign;
    double Y;
    if (isinf(X)) {
        Y = 448.0;
    } else {
        int E;
        frexp(X, &E);
        int e = E - 1;
        if (e < -6) e = -6;                       /* subnormal quantum below 2^-6 */
        double quantum = ldexp(1.0, e - 3);
        Y = nearbyint(X / quantum) * quantum;     /* nearest, ties to even */
        if (Y > 448.0) Y = 448.0;                 /* saturate */
    }
    if (Y == 0.0) return sign;
    int E;
    frexp(Y, &E);
    int e = E - 1;
    if (e >= -6) {
        uint32_t mant = (uint32_t)((Y / ldexp(1.0, e) - 1.0) * 8.0);
        return (uint8_t)(sign | (uint32_t)((e + 7) << 3) | mant);
    }
    return (uint8_t)(sign | (uint32_t)(Y / ldexp(1.0, -9)));
}

void or_e4m3_array(const float* x, uint8_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = or_e4m3(x[i]);
}

float or_e4m3_value(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 0xF, M = c & 7;
    if (E == 0xF && M == 7) return NAN;
    double v = E == 0 ? ldexp((double)M, -9) : ldexp(1.0 + M / 8.0, E - 7);
    return (float)(s ? -v : v);
}

/* x / scale for the cast.  The quotient is NaN when the block's scale is NaN
 * or for inf / inf; IEEE 754 leaves the sign of a NaN result open, and this
 * reading gives it the sign of x (the sign rule of division, scales being
 * positive), so that the code does not depend on a machine's default NaN. */
static float or_fp8_quotient(float x, float scale)
{
    float q = x / scale;
    if (isnan(q)) q = copysignf(NAN, x);
    return q;
}

/* Returns 0, or -1 when n is not a multiple of block (the listing refuses a
 * last dimension that the block size does not divide).
 * The block maximum is the listing's np.max of |x|: a NaN anywhere in the block
 * makes it NaN, so the block's scale is NaN (written as the quiet NaN
 * 0x7FC00000, NumPy fixing no payload) and every quotient, hence every code of
 * the block, is NaN. */
int or_fp8_block_cast(const float* x, int64_t n, int32_t block, uint8_t* codes, float* scales)
{
    if (block <= 0 || n % block != 0) return -1;
    for (int64_t b = 0; b < n / block; ++b) {
        const float* xb = x + b * block;
        float amax = 0.0f;
        for (int32_t i = 0; i < block; ++i) {
            float a = fabsf(xb[i]);
            if (isnan(a) || a > amax) amax = a;
        }
        float scale = amax / 448.0f;
        if (isnan(scale)) {
            const uint32_t quiet_nan = 0x7FC00000u;
            memcpy(&scale, &quiet_nan, sizeof scale);
        }
        if (scale == 0.0f) scale = 1.0f;
        scales[b] = scale;
        for (int32_t i = 0; i < block; ++i)
            codes[b * block + i] = or_e4m3(or_fp8_quotient(xb[i], scale));
    }
    return 0;
}
