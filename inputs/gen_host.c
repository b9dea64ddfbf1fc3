/*
 * Host fill of the seeded synthetic inputs (twin of gen_dev.hip; both include
 * mpgen.h).  OpenMP splits the index range; every element depends only on
 * (recipe, offset + i), so the result does not depend on the thread count.
 */
#include <omp.h>

#include "mpgen.h"

/* threads <= 0: OpenMP's default team; 1: the calling thread only. */
void mpgen_fill_f32_host(float* out, int64_t n, int64_t offset, const mpgen_recipe* r,
                         int threads)
{
    mpgen_recipe rc = *r;
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) out[i] = mpgen_f32(&rc, (uint64_t)(offset + i));
}

void mpgen_fill_u16_host(uint16_t* out, int64_t n, int64_t offset, const mpgen_recipe* r,
                         int dtype, int threads)
{
    mpgen_recipe rc = *r;
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; ++i) out[i] = mpgen_u16(&rc, (uint64_t)(offset + i), dtype);
}

uint64_t mpgen_key_host(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d)
{
    return mpgen_key(seed, a, b, c, d);
}

uint64_t mpgen_draw_host(uint64_t key, uint64_t index)
{
    return mpgen_draw(key, index);
}

double mpgen_uniform_host(uint64_t key, uint64_t index)
{
    return mpgen_uniform(mpgen_draw(key, index));
}
