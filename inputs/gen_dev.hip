/*
 * Device fill of the seeded synthetic inputs (twin of gen_host.c; both
 * include mpgen.h).  Grid-stride loop over the index range; the caller's
 * buffer must hold n elements.
 */
#include <hip/hip_runtime.h>

#include "mpgen.h"

__global__ void mpgen_fill_f32_kernel(float* out, int64_t n, int64_t offset, mpgen_recipe r)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = mpgen_f32(&r, (uint64_t)(offset + i));
}

__global__ void mpgen_fill_u16_kernel(uint16_t* out, int64_t n, int64_t offset, mpgen_recipe r,
                                      int dtype)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = mpgen_u16(&r, (uint64_t)(offset + i), dtype);
}

static unsigned mpgen_grid(int64_t n)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

extern "C" int mpgen_fill_f32_dev(float* out, int64_t n, int64_t offset, const mpgen_recipe* r,
                                  void* stream)
{
    if (n <= 0) return 0;
    if (out == nullptr || r == nullptr) return 1;
    mpgen_fill_f32_kernel<<<mpgen_grid(n), 256, 0, (hipStream_t)stream>>>(out, n, offset, *r);
    return (int)hipGetLastError();
}

extern "C" int mpgen_fill_u16_dev(uint16_t* out, int64_t n, int64_t offset, const mpgen_recipe* r,
                                  int dtype, void* stream)
{
    if (n <= 0) return 0;
    if (out == nullptr || r == nullptr) return 1;
    mpgen_fill_u16_kernel<<<mpgen_grid(n), 256, 0, (hipStream_t)stream>>>(out, n, offset, *r,
                                                                          dtype);
    return (int)hipGetLastError();
}
