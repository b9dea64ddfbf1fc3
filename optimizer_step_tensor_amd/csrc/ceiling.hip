// Bandwidth probes for the benchmark (not part of the library's API): kernels
// that move exactly the bytes of the update step's passes, with trivial
// arithmetic, in the launch shape the library uses -- one 256-lane block per
// 2048 consecutive elements, each lane two groups of 4 elements 256 apart, the
// blocks renumbered so that each XCD takes runs of consecutive chunks, the
// nontemporal hint on every streamed access, and an optional cap on resident
// blocks per CU.  They measure what the memory system delivers for each access
// pattern, so that each pass of the step can be rated against the speed of its
// own pattern as well as against the published peak.
//
// All arrays are flat, n elements long.  The AdamW-pattern probe reads and
// writes the caller's optimizer state but leaves it as it was: it writes back
// master, m and v plus 0 * (a finite value), and the 16-bit weight as the
// round-to-nearest-even of the master (which is what the step leaves there).
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MPC_GLOBAL __attribute__((address_space(1)))

namespace {

constexpr int kBlock = 256;
constexpr int kWave = 64;
constexpr int kChunk = 2048;
constexpr int kXcds = 8;
constexpr int kLdsPerCu = 160 * 1024;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// chunk of block b of a G-block grid: each XCD takes runs of `span` chunks
__device__ __forceinline__ int64_t chunk_of(int64_t b, int64_t G, int span)
{
    const int64_t turn = int64_t(span) * kXcds;
    if (span <= 1 || b >= (G / turn) * turn) return b;
    const int64_t t = b / turn, within = b % turn;
    return t * turn + (within % kXcds) * span + within / kXcds;
}

// first element of group h (0, 1) of this lane in a chunk
__device__ __forceinline__ int lane_elem(int h)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    return wave * 512 + h * 256 + lane * 4;
}

__device__ __forceinline__ f32x4 ld4(const float* p)
{
    return __builtin_nontemporal_load((const MPC_GLOBAL f32x4*)p);
}

__device__ __forceinline__ void st4(float* p, f32x4 v)
{
    __builtin_nontemporal_store(v, (MPC_GLOBAL f32x4*)p);
}

__device__ __forceinline__ u32x2 ld2(const uint16_t* p)
{
    return __builtin_nontemporal_load((const MPC_GLOBAL u32x2*)p);
}

__device__ __forceinline__ void st2(uint16_t* p, u32x2 v)
{
    __builtin_nontemporal_store(v, (MPC_GLOBAL u32x2*)p);
}

__device__ __forceinline__ uint32_t bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t fp16_rne(float x)
{
    if (x != x) return ((__float_as_uint(x) >> 16) & 0x8000u) | 0x7E00u;
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Whether group h of this lane's chunk is whole (the probes skip a partial tail
// group, which moves a negligible number of bytes).
__device__ __forceinline__ bool whole(int64_t e, int64_t n)
{
    return e + 4 <= n;
}

// AdamW's traffic: read acc, g16, master, m, v; write master, m, v, w16.
template <bool FP16>
__global__ __launch_bounds__(kBlock) void k_adamw_pattern(const float* acc, const uint16_t* g16,
                                                          float* master, float* m, float* v,
                                                          uint16_t* w16, int64_t n, float zero,
                                                          int span)
{
    const int64_t c = chunk_of(blockIdx.x, gridDim.x, span);
    const int64_t base = c * kChunk;
    f32x4 a[2], w[2], mm[2], vv[2];
    u32x2 g[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        ok[h] = whole(e, n);
        if (ok[h]) {
            a[h] = ld4(acc + e);
            g[h] = ld2(g16 + e);
            w[h] = ld4(master + e);
            mm[h] = ld4(m + e);
            vv[h] = ld4(v + e);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!ok[h]) continue;
        const int64_t e = base + lane_elem(h);
        const float gw = __uint_as_float(g[h].x << 16);
        const f32x4 z = a[h] * zero;
        w[h] = w[h] + z;
        mm[h] = mm[h] + z;
        vv[h] = vv[h] + gw * zero;
        uint32_t r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = FP16 ? fp16_rne(w[h][k]) : bf16_rne(w[h][k]);
        st4(master + e, w[h]);
        st4(m + e, mm[h]);
        st4(v + e, vv[h]);
        u32x2 o;
        o.x = r[0] | (r[1] << 16);
        o.y = r[2] | (r[3] << 16);
        st2(w16 + e, o);
    }
}

// The norm's traffic with the last micro-batch folded in: read acc and g16.
// One float per block is written so that the loads stay live.
__global__ __launch_bounds__(kBlock) void k_read_pattern(const float* acc, const uint16_t* g16,
                                                         int64_t n, float* sink, int span)
{
    const int64_t c = chunk_of(blockIdx.x, gridDim.x, span);
    const int64_t base = c * kChunk;
    // every load of the block is issued before the first is used, as in the norm pass
    f32x4 a[2];
    u32x2 g[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        ok[h] = whole(e, n);
        if (ok[h]) {
            a[h] = ld4(acc + e);
            g[h] = ld2(g16 + e);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (ok[h])
            s += a[h].x + a[h].y + a[h].z + a[h].w + __uint_as_float(g[h].x << 16) +
                 __uint_as_float(g[h].y << 16);
    if (s == 1.2345f) sink[blockIdx.x] = s;   // practically never: keeps the loads
}

// The accumulations' traffic.  First (acc = w * widen(g16)): read g16, write
// acc.  Later (acc += w * widen(g16)): read acc and g16, write acc.  The
// accumulator is dead between steps, so the probes may leave any finite value in it.
template <bool LATER>
__global__ __launch_bounds__(kBlock) void k_accumulate_pattern(float* acc, const uint16_t* g16,
                                                               int64_t n, int span)
{
    const int64_t c = chunk_of(blockIdx.x, gridDim.x, span);
    const int64_t base = c * kChunk;
    f32x4 a[2];
    u32x2 g[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        if (!whole(e, n)) continue;
        g[h] = ld2(g16 + e);
        if (LATER) a[h] = ld4(acc + e);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        if (!whole(e, n)) continue;
        f32x4 x = {__uint_as_float(g[h].x << 16), __uint_as_float(g[h].x & 0xFFFF0000u),
                   __uint_as_float(g[h].y << 16), __uint_as_float(g[h].y & 0xFFFF0000u)};
        if (LATER) x = a[h] + x;
        st4(acc + e, x);
    }
}

// Plain copy (one fp32 read, one fp32 write) and fill (one fp32 write).
__global__ __launch_bounds__(kBlock) void k_copy_pattern(const float* src, float* dst, int64_t n,
                                                         int span)
{
    const int64_t c = chunk_of(blockIdx.x, gridDim.x, span);
    const int64_t base = c * kChunk;
    f32x4 x[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        if (whole(e, n)) x[h] = ld4(src + e);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        if (whole(e, n)) st4(dst + e, x[h]);
    }
}

__global__ __launch_bounds__(kBlock) void k_fill_pattern(float* dst, int64_t n, float value,
                                                         int span)
{
    const int64_t c = chunk_of(blockIdx.x, gridDim.x, span);
    const int64_t base = c * kChunk;
    const f32x4 x = {value, value, value, value};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t e = base + lane_elem(h);
        if (whole(e, n)) st4(dst + e, x);
    }
}

unsigned lds_bytes(int blocks_per_cu)
{
    return blocks_per_cu > 0 ? static_cast<unsigned>(kLdsPerCu / blocks_per_cu) & ~1023u : 0u;
}

bool grid_of(int64_t n, unsigned* grid)
{
    const int64_t g = (n + kChunk - 1) / kChunk;
    if (n <= 0 || g > (int64_t(1) << 31) - 1) return false;
    *grid = static_cast<unsigned>(g);
    return true;
}

bool shape_ok(int blocks_per_cu, int span)
{
    return blocks_per_cu >= 0 && blocks_per_cu <= 8 && span >= 1 && span <= 4096;
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

}  // namespace

// Each returns 0 on success, 1 for invalid arguments (nothing launched), 2 for a
// launch error.  blocks_per_cu: 0 = no cap, else 1..8; span: consecutive chunks
// per XCD turn (1 = the dispatcher's own order), 1..4096.
extern "C" {

int mpc_adamw_pattern(const float* acc, const uint16_t* g16, float* master, float* m, float* v,
                      uint16_t* w16, int64_t n, int32_t fp16, int32_t blocks_per_cu, int32_t span,
                      void* stream)
{
    unsigned grid;
    if (!grid_of(n, &grid) || !shape_ok(blocks_per_cu, span)) return 1;
    if (!aligned16(acc) || !aligned16(g16) || !aligned16(master) || !aligned16(m) ||
        !aligned16(v) || !aligned16(w16))
        return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fp16)
        k_adamw_pattern<true><<<grid, kBlock, lds_bytes(blocks_per_cu), s>>>(acc, g16, master, m,
                                                                            v, w16, n, 0.0f, span);
    else
        k_adamw_pattern<false><<<grid, kBlock, lds_bytes(blocks_per_cu), s>>>(acc, g16, master, m,
                                                                             v, w16, n, 0.0f, span);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// sink: one float per 2048 elements, device memory
int mpc_read_pattern(const float* acc, const uint16_t* g16, int64_t n, float* sink,
                     int32_t blocks_per_cu, int32_t span, void* stream)
{
    unsigned grid;
    if (!grid_of(n, &grid) || !shape_ok(blocks_per_cu, span)) return 1;
    if (!aligned16(acc) || !aligned16(g16) || sink == nullptr) return 1;
    k_read_pattern<<<grid, kBlock, lds_bytes(blocks_per_cu), static_cast<hipStream_t>(stream)>>>(
        acc, g16, n, sink, span);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// later: 0 = the first accumulation's pattern, 1 = a later one's
int mpc_accumulate_pattern(float* acc, const uint16_t* g16, int64_t n, int32_t later,
                           int32_t blocks_per_cu, int32_t span, void* stream)
{
    unsigned grid;
    if (!grid_of(n, &grid) || !shape_ok(blocks_per_cu, span)) return 1;
    if (!aligned16(acc) || !aligned16(g16)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (later)
        k_accumulate_pattern<true><<<grid, kBlock, lds_bytes(blocks_per_cu), s>>>(acc, g16, n, span);
    else
        k_accumulate_pattern<false><<<grid, kBlock, lds_bytes(blocks_per_cu), s>>>(acc, g16, n, span);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mpc_copy_pattern(const float* src, float* dst, int64_t n, int32_t blocks_per_cu, int32_t span,
                     void* stream)
{
    unsigned grid;
    if (!grid_of(n, &grid) || !shape_ok(blocks_per_cu, span)) return 1;
    if (!aligned16(src) || !aligned16(dst)) return 1;
    k_copy_pattern<<<grid, kBlock, lds_bytes(blocks_per_cu), static_cast<hipStream_t>(stream)>>>(
        src, dst, n, span);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mpc_fill_pattern(float* dst, int64_t n, float value, int32_t blocks_per_cu, int32_t span,
                     void* stream)
{
    unsigned grid;
    if (!grid_of(n, &grid) || !shape_ok(blocks_per_cu, span)) return 1;
    if (!aligned16(dst)) return 1;
    k_fill_pattern<<<grid, kBlock, lds_bytes(blocks_per_cu), static_cast<hipStream_t>(stream)>>>(
        dst, n, value, span);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
