/*
 * Seeded synthetic inputs for the mixed-precision update step.
 *
 * One counter-based generator, compiled twice: by gcc for the host fill
 * (gen_host.c) and by hipcc for the device fill (gen_dev.hip).  Both sides get
 * bit-identical values because everything below is integer arithmetic plus
 * single, correctly rounded binary64 multiplications and the binary64 -> binary32
 * conversion; no transcendental function is used.  This module holds none of
 * the update step's arithmetic: 16-bit gradient patterns are produced by
 * truncation toward zero, not by the step's round-to-nearest-even cast.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to
 * key + (index + 1) * golden-gamma, so element i of a stream is computed
 * independently of every other element.
 */
#ifndef MPGEN_H
#define MPGEN_H

#include <stdint.h>

#if defined(__HIPCC__)
#define MPGEN_FN __host__ __device__ static inline
#else
#define MPGEN_FN static inline
#endif

#define MPGEN_GAMMA 0x9E3779B97F4A7C15ull

enum {
    MPGEN_NORMAL = 0,        /* sigma * z */
    MPGEN_NORMAL_TAIL = 1,   /* sigma * z, times tail_mult with probability tail_prob */
    MPGEN_LOGUNIF_MIX = 2,   /* with probability tail_prob: +-2^e * (1 + m), e uniform in
                                [lo_exp, hi_exp); otherwise sigma * z */
    MPGEN_CONST = 3          /* the constant sigma */
};

enum { MPGEN_BF16 = 0, MPGEN_FP16 = 1 };

typedef struct {
    uint64_t key;
    int32_t kind;
    int32_t lo_exp, hi_exp;
    int32_t pad;
    double sigma;
    double scale;       /* applied last: the loss scale S for scaled gradients (a power of 2) */
    double tail_prob;
    double tail_mult;
} mpgen_recipe;

MPGEN_FN uint64_t mpgen_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

MPGEN_FN uint64_t mpgen_draw(uint64_t key, uint64_t index)
{
    return mpgen_mix(key + (index + 1ull) * MPGEN_GAMMA);
}

/* Stream key from a seed and up to four labels (config, purpose, step, tensor ...). */
MPGEN_FN uint64_t mpgen_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d)
{
    uint64_t k = mpgen_mix(seed + MPGEN_GAMMA);
    k = mpgen_mix(k ^ (a + 1ull * MPGEN_GAMMA));
    k = mpgen_mix(k ^ (b + 2ull * MPGEN_GAMMA));
    k = mpgen_mix(k ^ (c + 3ull * MPGEN_GAMMA));
    k = mpgen_mix(k ^ (d + 4ull * MPGEN_GAMMA));
    return k;
}

/* Uniform in [0, 1) with 53 random bits. */
MPGEN_FN double mpgen_uniform(uint64_t z)
{
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

/* Normal-like draw: Irwin-Hall sum of the four 16-bit fields of z (each field
 * plus 1/2, over 2^16, is uniform on (0,1)), centred and scaled to unit
 * variance.  The centring is exact; one multiplication rounds. */
MPGEN_FN double mpgen_normal(uint64_t z)
{
    int64_t s = (int64_t)(z & 0xFFFFull) + (int64_t)((z >> 16) & 0xFFFFull)
              + (int64_t)((z >> 32) & 0xFFFFull) + (int64_t)(z >> 48);
    double centred = (double)(s + 2 - 131072) * (1.0 / 65536.0);
    return centred * 1.7320508075688772;      /* sqrt(12 / 4) */
}

MPGEN_FN double mpgen_pow2(int e)
{
    union { uint64_t u; double d; } v;
    v.u = (uint64_t)(1023 + e) << 52;
    return v.d;
}

/* Element `index` of the stream described by r, as binary64. */
MPGEN_FN double mpgen_value(const mpgen_recipe* r, uint64_t index)
{
    uint64_t z1 = mpgen_draw(r->key, 2ull * index);
    double x;
    if (r->kind == MPGEN_CONST) {
        x = r->sigma;
    } else if (r->kind == MPGEN_NORMAL) {
        x = mpgen_normal(z1) * r->sigma;
    } else {
        uint64_t z2 = mpgen_draw(r->key, 2ull * index + 1ull);
        int tail = mpgen_uniform(z2) < r->tail_prob;
        if (r->kind == MPGEN_NORMAL_TAIL) {
            x = mpgen_normal(z1) * r->sigma;
            if (tail) x = x * r->tail_mult;
        } else if (tail) {
            int span = r->hi_exp - r->lo_exp;
            int e = r->lo_exp + (int)((z2 & 0x7FFull) % (uint64_t)span);
            double mant = 1.0 + (double)(z1 & 0x7FFFFFull) * (1.0 / 8388608.0);
            x = mant * mpgen_pow2(e);
            if (z1 >> 63) x = -x;
        } else {
            x = mpgen_normal(z1) * r->sigma;
        }
    }
    return x * r->scale;
}

MPGEN_FN uint32_t mpgen_f32_bits(float f)
{
    union { float f; uint32_t u; } v;
    v.f = f;
    return v.u;
}

/* bf16 pattern of an fp32 value, truncated toward zero. */
MPGEN_FN uint16_t mpgen_bf16_trunc(float f)
{
    return (uint16_t)(mpgen_f32_bits(f) >> 16);
}

/* fp16 pattern of a finite fp32 value, truncated toward zero; magnitudes
 * beyond the largest finite fp16 value saturate to it. */
MPGEN_FN uint16_t mpgen_fp16_trunc(float f)
{
    uint32_t b = mpgen_f32_bits(f);
    uint16_t s = (uint16_t)((b >> 16) & 0x8000u);
    int E = (int)((b >> 23) & 0xFFu) - 127;
    uint32_t m = b & 0x7FFFFFu;
    if (E > 15) return (uint16_t)(s | 0x7BFFu);
    if (E >= -14) return (uint16_t)(s | (uint32_t)((E + 15) << 10) | (m >> 13));
    if (E >= -24) return (uint16_t)(s | ((m | 0x800000u) >> (uint32_t)(-1 - E)));
    return s;
}

MPGEN_FN uint16_t mpgen_u16(const mpgen_recipe* r, uint64_t index, int dtype)
{
    float f = (float)mpgen_value(r, index);
    return dtype == MPGEN_BF16 ? mpgen_bf16_trunc(f) : mpgen_fp16_trunc(f);
}

MPGEN_FN float mpgen_f32(const mpgen_recipe* r, uint64_t index)
{
    return (float)mpgen_value(r, index);
}

#endif /* MPGEN_H */
