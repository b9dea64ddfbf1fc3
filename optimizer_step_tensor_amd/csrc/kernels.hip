// HIP kernels of the mixed-precision update step, written for CDNA4 (gfx950).
//
// All element passes share one layout: a block of 256 lanes (4 wave64s) walks
// its chunks of the plan's chunk table; within a chunk each pass covers 2048
// elements, each wave a contiguous 512-element slab, and each lane two groups
// of 4 consecutive elements 256 elements apart, so every fp32 load or store
// instruction of a wave moves one contiguous 1 KiB line run (16 B per lane)
// and every 16-bit one a contiguous 512 B run.  Only the last partial group
// of a tensor takes the scalar path.  Every block's share of chunks is fixed by
// its index and the grid, so the assignment of elements to lanes is fixed,
// which makes the norm's reduction order -- and its bits -- the same on every
// run.
//
// Arithmetic: compiled with -ffp-contract=off and correctly rounded fp32
// division and square root, so every operation below is one IEEE-754 binary32
// (or binary64) round-to-nearest-even step, in the order written.
#include <type_traits>

#include "internal.h"

namespace mpk {
namespace {

// ---------------------------------------------------------------------------
// 16-bit formats ("Mixed precision, loss scaling, gradient accumulation, and
// activation checkpointing", section 2 "Two 16-bit formats").
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float widen16(uint32_t h);

template <>
__device__ __forceinline__ float widen16<MP_BF16>(uint32_t h)
{
    return __uint_as_float(h << 16);                     // bf16 is the top half of fp32
}

template <>
__device__ __forceinline__ float widen16<MP_FP16>(uint32_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Round to nearest, ties to even.  NaN -> the format's quiet NaN, sign kept.
template <int DT>
__device__ __forceinline__ uint32_t round16(float x);

template <>
__device__ __forceinline__ uint32_t round16<MP_BF16>(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    // Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
    // when the dropped half is above one half, or equal to it with an odd kept
    // half; a carry out of the largest finite value lands on infinity.
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <>
__device__ __forceinline__ uint32_t round16<MP_FP16>(float x)
{
    if (x != x) return ((__float_as_uint(x) >> 16) & 0x8000u) | 0x7E00u;
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));   // v_cvt_f16_f32, RNE
}

// ---------------------------------------------------------------------------
// Memory access.  Pointers are cast to the global address space so the
// compiler emits global_load/global_store (not flat) instructions; full groups
// move 16 bytes (fp32) or 8 bytes (16-bit) per lane in one instruction.
// nv = number of valid elements of a group (<= 0: none, >= 4: all).
// ---------------------------------------------------------------------------
#define MPK_GLOBAL __attribute__((address_space(1)))

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct F4 {
    float v[4];
};

struct H4 {
    uint32_t v[4];
};

template <bool FULL>
__device__ __forceinline__ F4 load_f4(const float* p, int nv)
{
    F4 r;
    if (FULL || nv >= kGroup) {
        const MPK_GLOBAL f32x4* q = (const MPK_GLOBAL f32x4*)(p);
        const f32x4 t = MPK_NT_LOADS ? __builtin_nontemporal_load(q) : *q;
        r.v[0] = t.x; r.v[1] = t.y; r.v[2] = t.z; r.v[3] = t.w;
    } else {
        const MPK_GLOBAL float* g = (const MPK_GLOBAL float*)(p);
#pragma unroll
        for (int k = 0; k < kGroup; ++k) r.v[k] = k < nv ? g[k] : 0.0f;
    }
    return r;
}

template <bool FULL>
__device__ __forceinline__ void store_f4(float* p, const F4& r, int nv)
{
    if (FULL || nv >= kGroup) {
        f32x4 t;
        t.x = r.v[0]; t.y = r.v[1]; t.z = r.v[2]; t.w = r.v[3];
        MPK_GLOBAL f32x4* q = (MPK_GLOBAL f32x4*)(p);
        if (MPK_NT_STORES) __builtin_nontemporal_store(t, q);
        else *q = t;
    } else {
        MPK_GLOBAL float* g = (MPK_GLOBAL float*)(p);
#pragma unroll
        for (int k = 0; k < kGroup; ++k)
            if (k < nv) g[k] = r.v[k];
    }
}

template <bool FULL>
__device__ __forceinline__ H4 load_h4(const uint16_t* p, int nv)
{
    H4 r;
    if (FULL || nv >= kGroup) {
        const MPK_GLOBAL u32x2* q = (const MPK_GLOBAL u32x2*)(p);
        const u32x2 t = MPK_NT_LOADS ? __builtin_nontemporal_load(q) : *q;
        r.v[0] = t.x & 0xFFFFu; r.v[1] = t.x >> 16; r.v[2] = t.y & 0xFFFFu; r.v[3] = t.y >> 16;
    } else {
        const MPK_GLOBAL uint16_t* g = (const MPK_GLOBAL uint16_t*)(p);
#pragma unroll
        for (int k = 0; k < kGroup; ++k) r.v[k] = k < nv ? static_cast<uint32_t>(g[k]) : 0u;
    }
    return r;
}

template <bool FULL>
__device__ __forceinline__ void store_h4(uint16_t* p, const H4& r, int nv)
{
    if (FULL || nv >= kGroup) {
        u32x2 t;
        t.x = r.v[0] | (r.v[1] << 16);
        t.y = r.v[2] | (r.v[3] << 16);
        MPK_GLOBAL u32x2* q = (MPK_GLOBAL u32x2*)(p);
        if (MPK_NT_STORES) __builtin_nontemporal_store(t, q);
        else *q = t;
    } else {
        MPK_GLOBAL uint16_t* g = (MPK_GLOBAL uint16_t*)(p);
#pragma unroll
        for (int k = 0; k < kGroup; ++k)
            if (k < nv) g[k] = static_cast<uint16_t>(r.v[k]);
    }
}

// The chunk block b of a G-block grid starts at.  Workgroup b runs on XCD
// b mod 8; this renumbering gives each XCD SPAN consecutive chunks per turn of
// 8 * SPAN blocks.  It permutes 0..G-1: blocks of the last, incomplete turn
// keep their own number.
template <int SPAN = MPK_XCD_SPAN>
__device__ __forceinline__ int64_t xcd_first_chunk(int64_t b, int64_t G)
{
    constexpr int64_t span = SPAN;
    constexpr int64_t turn = span * kXcds;
    if (span <= 1 || b >= (G / turn) * turn) return b;
    const int64_t t = b / turn, within = b % turn;
    return t * turn + (within % kXcds) * span + within / kXcds;
}

// Run pass(full, base) over a chunk of `len` elements: every complete
// 2048-element block pass with full = true_type (no bounds checks at all),
// then the one partial pass, if any, with full = false_type.
template <class Pass>
__device__ __forceinline__ void for_each_pass(int len, Pass&& pass)
{
    int base = 0;
    for (; base + kBlockSlab <= len; base += kBlockSlab) pass(std::true_type{}, base);
    if (base < len) pass(std::false_type{}, base);
}

// Element offset of group h of this lane inside one 2048-element block pass.
__device__ __forceinline__ int lane_offset(int h)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    return wave * kWaveSlab + h * (kWave * kGroup) + lane * kGroup;
}

__device__ __forceinline__ int valid_count(int len, int e)
{
    int r = len - e;
    return r > kGroup ? kGroup : r;
}

// A read from a table that nothing writes while the pass runs: the plan's chunk
// and tensor tables, a gradset's pointer table, the FP8 output table, a weight
// written by an earlier launch.  Through the constant address space, a load at
// a uniform address becomes one scalar load served by the scalar cache; as a
// plain load in a pass that also stores, the compiler must assume the stores
// may change the table and issues a vector load from every wave instead, all
// of the grid's waves then hitting the same few L2 lines (the accumulations
// ran 3-7% slower reading a device-resident weight that way).
#define MPK_CONST __attribute__((address_space(4)))
// A struct is read as 8-byte words (a struct copy would bind a reference in
// the generic address space and lose the constant one).
template <class T, bool SCALAR = MPK_SCALAR_TABLES>
__device__ __forceinline__ T read_table(const T* p)
{
    if constexpr (!SCALAR) {
        return *p;
    } else if constexpr (sizeof(T) <= 8) {
        return *(const MPK_CONST T*)(p);
    } else {
        static_assert(sizeof(T) % 8 == 0 && alignof(T) >= 8, "a table entry of 8-byte words");
        struct Words {
            uint64_t w[sizeof(T) / 8];
        } x;
        const MPK_CONST uint64_t* q = (const MPK_CONST uint64_t*)(p);
#pragma unroll
        for (int i = 0; i < int(sizeof(T) / 8); ++i) x.w[i] = q[i];
        return __builtin_bit_cast(T, x);
    }
}

__device__ __forceinline__ float weight_of(const Weight& w)
{
    return w.ptr != nullptr ? read_table(w.ptr) : w.value;
}

// The fp32 gradient of one element ("Megatron Internals III", section 8;
// "Mixed precision ...", section 2 "Gradient accumulation"): the accumulator
// (ACC) followed by NG micro-batches in order, each added with the two
// roundings of one accumulation step, x = fl(x + fl(w_i * widen(g_i))).
// Without the accumulator the first term is fl(w_1 * widen(g_1)) itself, as
// in a first accumulation (so a -0 stays -0).
template <int DT, bool ACC, int NG>
__device__ __forceinline__ float grad_sum(float acc, const uint32_t (&h)[kMaxGroup],
                                          const float (&w)[kMaxGroup])
{
    static_assert(ACC || NG > 0, "a gradient needs at least one term");
    float x = acc;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const float t = w[i] * widen16<DT>(h[i]);
        x = (ACC || i > 0) ? x + t : t;
    }
    return x;
}

// Token weights ("Accumulate gradients and recompute activations", "Weight each
// mean by the targets it represents"): w_i = fp32(n_i / N) with N = sum of the k
// counts, in binary64 then rounded once -- the host helper's arithmetic.  Counts
// the host helper would refuse (n_i <= 0, N > 2^53) give NaN weights, so that the
// step they feed overflows and is skipped.  Returns N, or -1 for refused counts.
// The running sum stops growing once a count is refused or the sum passes 2^53,
// so it never leaves int64; the loads do not depend on it and can all be in
// flight at once.
__device__ __forceinline__ double count_total(const int64_t* __restrict__ counts, int k)
{
    const int64_t limit = int64_t(1) << 53;
    int64_t n = 0;
    bool bad = false;
#pragma unroll 8
    for (int i = 0; i < k; ++i) {
        const int64_t c = read_table(counts + i);
        bad |= c <= 0 || c > limit;
        n += bad ? 0 : c;
        bad |= n > limit;
    }
    return bad ? -1.0 : static_cast<double>(n);
}

__device__ __forceinline__ float token_weight(const int64_t* __restrict__ counts, int i,
                                              double total)
{
    return total > 0.0 ? static_cast<float>(static_cast<double>(read_table(counts + i)) / total)
                       : __builtin_nanf("");
}

// The group's weights, each read once per block.  With token counts (the first
// accumulation of an update), every block computes the weights of micro-batches
// 0..NG-1 from the k counts itself, and block 0 also writes all k weights to
// weights_out, where the later passes of the update read them.
template <int NG>
__device__ __forceinline__ void group_weights(const Grads& g, float (&w)[kMaxGroup])
{
    if (g.counts != nullptr) {
        const double total = count_total(g.counts, g.k);
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i)
            w[i] = i < NG ? token_weight(g.counts, i, total) : 0.0f;
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < g.k; i += kBlock)
                g.weights_out[i] = token_weight(g.counts, i, total);
        return;
    }
#pragma unroll
    for (int i = 0; i < kMaxGroup; ++i) w[i] = i < NG ? weight_of(g.w[i]) : 0.0f;
}

// Element k of group j of every set, in micro-batch order.
template <int NG>
__device__ __forceinline__ void element_terms(const H4 (&h)[kMaxGroup][kGroupsPerLane], int j, int k,
                                              uint32_t (&out)[kMaxGroup])
{
#pragma unroll
    for (int i = 0; i < kMaxGroup; ++i) out[i] = i < NG ? h[i][j].v[k] : 0u;
}

// Deterministic block sum of one double per lane (result valid in lane 0).
__device__ __forceinline__ double block_sum(double x)
{
    __shared__ double wave_sums[kBlock / kWave];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) wave_sums[threadIdx.x / kWave] = x;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0) {
        total = wave_sums[0];
#pragma unroll
        for (int w = 1; w < kBlock / kWave; ++w) total += wave_sums[w];
    }
    return total;
}

// ---------------------------------------------------------------------------
// Accumulation of one micro-batch.
// ---------------------------------------------------------------------------
template <int DT, bool FIRST, int NG>
__global__ __launch_bounds__(kBlock) void k_accumulate(PlanView p, Grads g)
{
    // the weights are read after a pass's loads are issued, so that a weight in
    // device memory is read while the loads are in flight
    float w[kMaxGroup];
    bool have_w = false;
    for (int64_t c = xcd_first_chunk<MPK_ACC_XCD_SPAN>(blockIdx.x, gridDim.x); c < p.n_chunks;
         c += gridDim.x) {
        const Chunk ch = read_table(p.chunks + c);
        float* acc = read_table(&p.tensors[ch.tensor].acc) + ch.start;
        const uint16_t* gp[kMaxGroup];
#pragma unroll
        for (int i = 0; i < NG; ++i) gp[i] = read_table(g.set[i] + ch.tensor) + ch.start;
        for_each_pass(ch.len, [&](auto full, int base) {
            constexpr bool F = decltype(full)::value;
            int e[kGroupsPerLane], nv[kGroupsPerLane];
            H4 h[kMaxGroup][kGroupsPerLane];
            F4 a[kGroupsPerLane];
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
                e[j] = base + lane_offset(j);
                nv[j] = F ? kGroup : valid_count(ch.len, e[j]);
#pragma unroll
                for (int i = 0; i < NG; ++i) h[i][j] = load_h4<F>(gp[i] + e[j], nv[j]);
                if (!FIRST) a[j] = load_f4<F>(acc + e[j], nv[j]);
            }
            if (!have_w) {
                group_weights<NG>(g, w);
                have_w = true;
            }
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
                F4 out;
#pragma unroll
                for (int k = 0; k < kGroup; ++k) {
                    uint32_t hk[kMaxGroup];
                    element_terms<NG>(h, j, k, hk);
                    out.v[k] = grad_sum<DT, !FIRST, NG>(FIRST ? 0.0f : a[j].v[k], hk, w);
                }
                store_f4<F>(acc + e[j], out, nv[j]);
            }
        });
    }
}

// ---------------------------------------------------------------------------
// Unscale + sum of squares, first stage: one binary64 partial per block.  Block
// b takes the CPB consecutive chunks of "super-chunk" b (renumbered for the XCDs
// like the chunks of the other passes).  When all of them are whole 2048-element
// chunks, every descriptor is read first and then every data load is issued
// before the first square is summed, so that the latency of the descriptor
// reads and of one block's loads is paid once per CPB chunks; a block with a
// ragged or missing chunk walks its chunks one by one.  The order of the sum is
// fixed by the grid either way.  An inf or NaN gradient makes the sum inf or
// NaN; finite fp32 squares cannot overflow binary64 for any element count a
// device can hold, so the overflow flag is exactly "the sum is not finite".
// ---------------------------------------------------------------------------
template <int DT, bool ACC, int NG>
__device__ __forceinline__ void add_squares(const F4& a, const u32x2 (&h)[kMaxGroup],
                                            const float (&w)[kMaxGroup], float inv, double& s)
{
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        uint32_t hk[kMaxGroup];
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i)
            hk[i] = i < NG ? ((k & 1) ? (h[i][k >> 1] >> 16) : (h[i][k >> 1] & 0xFFFFu)) : 0u;
        const float gv = grad_sum<DT, ACC, NG>(ACC ? a.v[k] : 0.0f, hk, w) * inv;
        const double d = static_cast<double>(gv);
        // the square of an fp32 value is exact in binary64, so this fma is the
        // same as a rounded add of the exact square; the zeros loaded for
        // elements past a tail add exactly 0
        s = __builtin_fma(d, d, s);
    }
}

template <int DT, bool ACC, int NG, int CPB>
__global__ __launch_bounds__(kBlock) void k_norm_partial(PlanView p, Grads g,
                                                         const DevState* __restrict__ st,
                                                         double* __restrict__ partials)
{
    float w[kMaxGroup];
    group_weights<NG>(g, w);
    const float inv = st->inv_scale;
    double s = 0.0;
    const int64_t c0 = xcd_first_chunk<MPK_NORM_XCD_SPAN>(blockIdx.x, gridDim.x) * CPB;
    bool whole = c0 + CPB <= p.n_chunks;
    Chunk ch[CPB] = {};
#pragma unroll
    for (int q = 0; q < CPB; ++q) {
        if (c0 + q < p.n_chunks) ch[q] = read_table(p.chunks + c0 + q);
        whole = whole && ch[q].len == kBlockSlab;
    }
    if (whole) {
        F4 a[CPB][kGroupsPerLane];
        u32x2 h[CPB][kGroupsPerLane][kMaxGroup];
#pragma unroll
        for (int q = 0; q < CPB; ++q) {
            const float* acc =
                ACC ? read_table(&p.tensors[ch[q].tensor].acc) + ch[q].start : nullptr;
            const uint16_t* gp[kMaxGroup];
#pragma unroll
            for (int i = 0; i < NG; ++i) gp[i] = read_table(g.set[i] + ch[q].tensor) + ch[q].start;
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
                const int e = lane_offset(j);
                if (ACC) a[q][j] = load_f4<true>(acc + e, kGroup);
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const MPK_GLOBAL u32x2* x = (const MPK_GLOBAL u32x2*)(gp[i] + e);
                    h[q][j][i] = MPK_NT_LOADS ? __builtin_nontemporal_load(x) : *x;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < CPB; ++q)
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) add_squares<DT, ACC, NG>(a[q][j], h[q][j], w, inv, s);
    } else {
        for (int q = 0; q < CPB && c0 + q < p.n_chunks; ++q) {
            // (ch[] is indexed by constants only)
            const Chunk c = read_table(p.chunks + c0 + q);
            const float* acc = ACC ? read_table(&p.tensors[c.tensor].acc) + c.start : nullptr;
            const uint16_t* gp[kMaxGroup];
#pragma unroll
            for (int i = 0; i < NG; ++i) gp[i] = read_table(g.set[i] + c.tensor) + c.start;
            for_each_pass(c.len, [&](auto full, int base) {
                constexpr bool F = decltype(full)::value;
#pragma unroll
                for (int j = 0; j < kGroupsPerLane; ++j) {
                    const int e = base + lane_offset(j);
                    const int nv = F ? kGroup : valid_count(c.len, e);
                    const F4 a = ACC ? load_f4<F>(acc + e, nv) : F4{};
                    u32x2 h[kMaxGroup];
#pragma unroll
                    for (int i = 0; i < NG; ++i) {
                        const H4 x = load_h4<F>(gp[i] + e, nv);
                        h[i][0] = x.v[0] | (x.v[1] << 16);
                        h[i][1] = x.v[2] | (x.v[3] << 16);
                    }
                    add_squares<DT, ACC, NG>(a, h, w, inv, s);
                }
            });
        }
    }
    const double total = block_sum(s);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

// Sum of x[lo..hi) by one block in a fixed order: lane t adds x[lo + t],
// x[lo + t + 256], ... in increasing index, then the block tree.  Valid in
// thread 0.  The loads are issued 32 at a time, those past hi replaced by
// +0.0, which leaves a sum of squares (>= +0, inf or NaN) exactly as it was:
// up to 8192 partials cost one memory latency instead of a chain of them.
constexpr int kSumBatch = 32;
__device__ __forceinline__ double block_sum_range(const double* __restrict__ x, int64_t lo,
                                                  int64_t hi)
{
    double s = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kSumBatch * kBlock) {
        double v[kSumBatch];
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) {
            const int64_t j = i + static_cast<int64_t>(u) * kBlock;
            v[u] = j < hi ? x[j] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) s += v[u];
    }
    return block_sum(s);
}

// Second stage: block j sums the j-th of `gridDim.x` contiguous ranges of the n
// first-stage partials.
__global__ __launch_bounds__(kBlock) void k_norm_stage2(const double* __restrict__ partials,
                                                        int64_t n, double* __restrict__ out)
{
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    const double total = block_sum_range(partials, lo, hi);
    if (threadIdx.x == 0) out[blockIdx.x] = total;
}

// The optimizer clock advances only on a committed step ("Accumulate gradients
// and recompute activations", "Discard a failed partial logical update").
__device__ void advance_clock(DevState* __restrict__ st, float beta1, float beta2)
{
    if (st->s.found_inf) return;
    st->s.step += 1;
    st->s.beta1_pow = st->s.beta1_pow * static_cast<double>(beta1);
    st->s.beta2_pow = st->s.beta2_pow * static_cast<double>(beta2);
}

// Dynamic loss-scale controller ("Mixed precision ...", section 2 "Dynamic
// scaling"; "Megatron Internals III", section 5).
__device__ void scaler_decision(DevState* __restrict__ st)
{
    const int found_inf = st->s.found_inf;
    st->s.skipped = found_inf;
    if (found_inf) st->s.skipped_total += 1;
    if (!st->enabled) return;
    float scale = st->s.scale;
    if (found_inf) {
        const float next = scale * st->backoff;
        scale = next > st->min_scale ? next : st->min_scale;
        st->s.good_steps = 0;
    } else {
        int good = st->s.good_steps + 1;
        if (good == st->interval) {
            const float next = scale * st->growth;
            scale = next < st->max_scale ? next : st->max_scale;
            good = 0;
        }
        st->s.good_steps = good;
    }
    st->s.scale = scale;
    st->inv_scale = 1.0f / scale;
}

// Overflow flag, norm and clip coefficient from the total sum of squares
// ("Megatron Internals III", section 9).
__device__ void apply_norm(double total, float max_norm, DevState* __restrict__ st)
{
    const int found_inf = !__builtin_isfinite(total);
    const float norm = static_cast<float>(__builtin_sqrt(total));
    float coef = 1.0f;
    if (max_norm > 0.0f && !found_inf) {
        const float q = max_norm / (norm + 1e-6f);
        coef = q < 1.0f ? q : 1.0f;
    }
    st->s.found_inf = found_inf;
    st->s.sumsq = total;
    st->s.grad_norm = norm;
    st->s.clip_coef = coef;
    st->update_scale = st->inv_scale * coef;
}

// Last stage: the fixed-order sum of n partial sums, then either the norm into
// the state (out == NULL) or the total into *out.  With a tail (the whole
// update enqueued by one call), the optimizer clock and the scaler's decision
// follow in the same thread: both depend only on the overflow flag, and the
// AdamW pass then reads the advanced clock.
__global__ __launch_bounds__(kBlock) void k_norm_finish(const double* __restrict__ partials,
                                                        int64_t n, float max_norm,
                                                        DevState* __restrict__ st,
                                                        double* __restrict__ out, Tail tail)
{
    const double total = block_sum_range(partials, 0, n);
    if (threadIdx.x != 0) return;
    if (out != nullptr) {
        out[0] = total;
        return;
    }
    apply_norm(total, max_norm, st);
    if (tail.on) {
        advance_clock(st, tail.beta1, tail.beta2);
        scaler_decision(st);
    }
}

// The finish from a sum of squares reduced across ranks.
__global__ void k_norm_apply(const double* __restrict__ sumsq, float max_norm,
                             DevState* __restrict__ st)
{
    if (threadIdx.x == 0) apply_norm(sumsq[0], max_norm, st);
}

// ---------------------------------------------------------------------------
// Fine-grained FP8 ("Chapter 41 Training at Scale", section 41.5): blocks of
// consecutive values; scale = max|x| / 448 (a zero block takes 1); each value
// x / scale rounded to E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no
// infinity: saturate at 448; NaN -> S.1111.111).  The maximum propagates NaN
// as the section's NumPy maximum does: a block holding a NaN gets the quiet
// NaN 0x7FC00000 as its scale and the NaN code for every value.  A NaN
// quotient (NaN scale, or inf / inf) takes the sign bit of its value.
// ---------------------------------------------------------------------------
constexpr uint32_t kQuietNan = 0x7FC00000u;

// max(amax, a) for the block maximum: a NaN wins, and stays.
__device__ __forceinline__ float nan_max(float amax, float a)
{
    return (a > amax || a != a) ? a : amax;
}

__device__ __forceinline__ float block_scale_of(float amax)
{
    float scale = amax / 448.0f;
    if (scale != scale) scale = __uint_as_float(kQuietNan);
    if (scale == 0.0f) scale = 1.0f;
    return scale;
}
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;                  // NaN
    if (a >= 0x43E80000u) return sign | 0x7Eu;                 // >= 464 (incl. inf): 448
    if (a >= 0x3C800000u) {                                    // >= 2^-6: normal
        // round the 23-bit mantissa to 3 bits, ties to even, then rebias 127 -> 7
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        return sign | ((r >> 20) - (120u << 3));
    }
    // subnormal: the nearest multiple of 2^-9 (ties to even); 8 * 2^-9 is the
    // smallest normal, whose code is 8 as well
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);
}

// The codes of x[0..3] / scale.  The quotients go through gfx950's fp32 -> fp8
// pack instruction, which rounds to nearest even into E4M3 exactly as e4m3_code
// does for every finite input below 464 in magnitude (subnormals and zeros
// included); it was compared with e4m3_code on all 2^32 fp32 patterns.  At and
// above 464, for infinities and for NaN it returns a NaN code instead, so those
// quotients take e4m3_code (saturation to 448), and a NaN quotient the NaN code
// with the sign bit of its value.  A block's quotients stay at or below 448
// unless its maximum is infinite or NaN.
__device__ __forceinline__ uint32_t pack_e4m3(const F4& x, float scale)
{
    float q[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) q[k] = x.v[k] / scale;
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    uint32_t packed = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true));
    bool special = false;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) special |= (__float_as_uint(q[k]) & 0x7FFFFFFFu) >= 0x43E80000u;
    if (special) {
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
            const uint32_t a = __float_as_uint(q[k]) & 0x7FFFFFFFu;
            if (a >= 0x43E80000u) {
                const uint32_t code = a > 0x7F800000u
                                          ? ((__float_as_uint(x.v[k]) >> 24) & 0x80u) | 0x7Fu
                                          : e4m3_code(q[k]);
                packed = (packed & ~(0xFFu << (8 * k))) | (code << (8 * k));
            }
        }
    }
    return packed;
}

// Scale of the 16-value block held by lanes 4q..4q+3 (4 consecutive values
// each): the lanes' maxima combined with two butterfly shuffles.  Every lane
// of the wave must call it.
__device__ __forceinline__ float block16_scale(const F4& x)
{
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) amax = nan_max(amax, __builtin_fabsf(x.v[k]));
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) amax = nan_max(amax, __shfl_xor(amax, off, kWave));
    return block_scale_of(amax);
}

__device__ __forceinline__ void store_codes4(uint8_t* p, uint32_t packed)
{
    MPK_GLOBAL uint32_t* q = (MPK_GLOBAL uint32_t*)(p);
    if (MPK_NT_STORES) __builtin_nontemporal_store(packed, q);
    else *q = packed;
}

__device__ __forceinline__ void store_scale(float* p, float scale)
{
    MPK_GLOBAL float* q = (MPK_GLOBAL float*)(p);
    if (MPK_NT_STORES) __builtin_nontemporal_store(scale, q);
    else *q = scale;
}

// ---------------------------------------------------------------------------
// AdamW on fp32 master/m/v and the RNE cast to the 16-bit weight.  With FP8,
// the new weights of every tensor that has FP8 outputs are also cast in blocks
// of 16 exactly as k_fp8_blocks16 casts them, in the same pass.
// ---------------------------------------------------------------------------
template <int DT, bool ACC, int NG, bool FP8>
__global__ __launch_bounds__(kBlock) void k_adamw(PlanView p, Grads g, AdamArgs a,
                                                  const Fp8Out* __restrict__ fp8,
                                                  const DevState* __restrict__ st)
{
    if (st->s.found_inf) return;                  // skipped step: write nothing
    float gw[kMaxGroup];
    group_weights<NG>(g, gw);
    const float scale = st->update_scale;
    // beta^(t+1): the clock advances after this pass, or (a.clock_advanced) the
    // norm's finish already advanced it -- the same binary64 product either way
    const double p1 = a.clock_advanced ? st->s.beta1_pow : st->s.beta1_pow * static_cast<double>(a.beta1);
    const double p2 = a.clock_advanced ? st->s.beta2_pow : st->s.beta2_pow * static_cast<double>(a.beta2);
    const float bc1 = static_cast<float>(1.0 - p1);
    const float bc2 = static_cast<float>(1.0 - p2);
    const float b1 = a.beta1, b2 = a.beta2;
    const float ob1 = 1.0f - b1, ob2 = 1.0f - b2;
    const float eps = a.eps, lr = a.lr;
    for (int64_t c = xcd_first_chunk<MPK_ADAMW_XCD_SPAN>(blockIdx.x, gridDim.x); c < p.n_chunks;
         c += gridDim.x) {
        // AdamW's long blocks measured 0-3% faster with these as vector loads
        constexpr bool S = MPK_ADAMW_SCALAR_TABLES;
        const Chunk ch = read_table<Chunk, S>(p.chunks + c);
        const TensorDesc td = read_table<TensorDesc, S>(p.tensors + ch.tensor);
        const float lam = a.weight_decay * td.wd_mult;
        const float* acc = ACC ? td.acc + ch.start : nullptr;
        const uint16_t* gp[kMaxGroup];
#pragma unroll
        for (int i = 0; i < NG; ++i)
            gp[i] = read_table<const uint16_t*, S>(g.set[i] + ch.tensor) + ch.start;
        float* mw = td.master + ch.start;
        float* mm = td.m + ch.start;
        float* mv = td.v + ch.start;
        uint16_t* w16 = td.w16 + ch.start;
        // a cast tensor has numel % 16 == 0, so with chunk starts on 2048 every
        // group of 4 is wholly inside or wholly past its tensor's end
        uint8_t* codes = nullptr;
        float* scales = nullptr;
        if (FP8) {
            const Fp8Out o = read_table<Fp8Out, S>(fp8 + ch.tensor);
            if (o.codes != nullptr) {
                codes = o.codes + ch.start;
                scales = o.scales + ch.start / 16;
            }
        }
        for_each_pass(ch.len, [&](auto full, int base) {
            constexpr bool F = decltype(full)::value;
            int e[kGroupsPerLane], nv[kGroupsPerLane];
            F4 ga[kGroupsPerLane], wv[kGroupsPerLane], m[kGroupsPerLane], v[kGroupsPerLane];
            H4 h[kMaxGroup][kGroupsPerLane];
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
                e[j] = base + lane_offset(j);
                nv[j] = F ? kGroup : valid_count(ch.len, e[j]);
            }
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
                if (ACC) ga[j] = load_f4<F>(acc + e[j], nv[j]);
#pragma unroll
                for (int i = 0; i < NG; ++i) h[i][j] = load_h4<F>(gp[i] + e[j], nv[j]);
                wv[j] = load_f4<F>(mw + e[j], nv[j]);
                m[j] = load_f4<F>(mm + e[j], nv[j]);
                v[j] = load_f4<F>(mv + e[j], nv[j]);
            }
            H4 out16[kGroupsPerLane];
#pragma unroll
            for (int j = 0; j < kGroupsPerLane; ++j) {
#pragma unroll
                for (int k = 0; k < kGroup; ++k) {
                    uint32_t hk[kMaxGroup];
                    element_terms<NG>(h, j, k, hk);
                    const float gr = grad_sum<DT, ACC, NG>(ACC ? ga[j].v[k] : 0.0f, hk, gw);
                    const float gs = gr * scale;
                    const float mj = b1 * m[j].v[k] + ob1 * gs;
                    const float vj = b2 * v[j].v[k] + ob2 * (gs * gs);
                    const float mh = mj / bc1;
                    const float vh = vj / bc2;
                    const float den = __builtin_sqrtf(vh) + eps;
                    const float u = mh / den;
                    float w = wv[j].v[k];
                    w = w - lr * (u + lam * w);
                    m[j].v[k] = mj;
                    v[j].v[k] = vj;
                    wv[j].v[k] = w;
                    out16[j].v[k] = round16<DT>(w);
                }
                store_f4<F>(mw + e[j], wv[j], nv[j]);
                store_f4<F>(mm + e[j], m[j], nv[j]);
                store_f4<F>(mv + e[j], v[j], nv[j]);
                store_h4<F>(w16 + e[j], out16[j], nv[j]);
                if (FP8 && codes != nullptr) {          // uniform over the block
                    const float scale = block16_scale(wv[j]);
                    if (F || nv[j] >= kGroup) {
                        store_codes4(codes + e[j], pack_e4m3(wv[j], scale));
                        if ((threadIdx.x & 3) == 0) store_scale(scales + e[j] / 16, scale);
                    }
                }
            }
        });
    }
}

__global__ void k_adam_clock(DevState* __restrict__ st, float beta1, float beta2)
{
    if (threadIdx.x == 0) advance_clock(st, beta1, beta2);
}

__global__ void k_scaler(DevState* __restrict__ st)
{
    if (threadIdx.x == 0) scaler_decision(st);
}

// Both, in that order, in one launch: the tail of a whole update enqueued by one
// call, where nothing can run between them.
__global__ void k_clock_scaler(DevState* __restrict__ st, float beta1, float beta2)
{
    if (threadIdx.x != 0) return;
    advance_clock(st, beta1, beta2);
    scaler_decision(st);
}

// Token weights on the device (count_total, token_weight above).
__global__ __launch_bounds__(kBlock) void k_token_weights(const int64_t* __restrict__ counts, int k,
                                                          float* __restrict__ weights)
{
    const double total = count_total(counts, k);
    for (int i = threadIdx.x; i < k; i += kBlock) weights[i] = token_weight(counts, i, total);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_cast_to_16(const float* __restrict__ src,
                                                       uint16_t* __restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = static_cast<uint16_t>(round16<DT>(src[i]));
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_widen_16(const uint16_t* __restrict__ src,
                                                     float* __restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = widen16<DT>(src[i]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Block of 16 (the listing's default): a wave covers 1024 consecutive values,
// lane l holding values 4l..4l+3 of each 256-value slab, so every load and
// store instruction of the wave is contiguous; the four lanes that hold one
// block combine their maxima with two butterfly shuffles.
__global__ __launch_bounds__(kBlock) void k_fp8_blocks16(const float* __restrict__ src,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         int64_t n)
{
    constexpr int kSlab = kWave * kGroup;                  // 256 values
    constexpr int kWaveValues = 4 * kSlab;                 // 1024 values per wave pass
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kBlock / kWave) + threadIdx.x / kWave;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (kBlock / kWave);
    for (int64_t base = wave * kWaveValues; base < n; base += waves * kWaveValues) {
        F4 v[4];
        bool live[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {                          // all four loads in flight first
            const int64_t e = base + j * kSlab + lane * kGroup;   // n is a multiple of 16
            live[j] = e < n;
            if (live[j]) v[j] = load_f4<true>(src + e, kGroup);
            else v[j].v[0] = v[j].v[1] = v[j].v[2] = v[j].v[3] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t e = base + j * kSlab + lane * kGroup;
            const float scale = block16_scale(v[j]);
            if (live[j]) {
                *(MPK_GLOBAL uint32_t*)(codes + e) = pack_e4m3(v[j], scale);
                if ((lane & 3) == 0) scales[e / 16] = scale;
            }
        }
    }
}

// Other block sizes (multiples of 16): one lane per block, two passes; the
// second re-reads the block from cache.
__global__ __launch_bounds__(kBlock) void k_fp8_blocks(const float* __restrict__ src,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       int64_t nblocks, int block)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; b < nblocks;
         b += stride) {
        const float* x = src + b * block;
        uint8_t* out = codes + b * block;
        float amax = 0.0f;
        for (int i = 0; i < block; i += kGroup) {
            const F4 v = load_f4<true>(x + i, kGroup);
#pragma unroll
            for (int k = 0; k < kGroup; ++k) amax = nan_max(amax, __builtin_fabsf(v.v[k]));
        }
        const float scale = block_scale_of(amax);
        for (int i = 0; i < block; i += 16) {
            u32x4 w;
            w.x = pack_e4m3(load_f4<true>(x + i, kGroup), scale);
            w.y = pack_e4m3(load_f4<true>(x + i + 4, kGroup), scale);
            w.z = pack_e4m3(load_f4<true>(x + i + 8, kGroup), scale);
            w.w = pack_e4m3(load_f4<true>(x + i + 12, kGroup), scale);
            *(MPK_GLOBAL u32x4*)(out + i) = w;
        }
        scales[b] = scale;
    }
}

unsigned elementwise_grid(int64_t n)
{
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 8192) blocks = 8192;
    return static_cast<unsigned>(blocks < 1 ? 1 : blocks);
}

// Calls fn(dt, acc, ng) with the three as compile-time constants, for the
// plan's 16-bit format, whether the accumulator is a term, and the group size.
template <int DT, bool ACC, class Fn>
bool with_count(int n, Fn&& fn)
{
    using std::integral_constant;
    switch (n) {
    case 0:
        if constexpr (ACC) {
            fn(integral_constant<int, DT>{}, std::bool_constant<ACC>{}, integral_constant<int, 0>{});
            return true;
        }
        return false;
    case 1: fn(integral_constant<int, DT>{}, std::bool_constant<ACC>{}, integral_constant<int, 1>{}); return true;
    case 2: fn(integral_constant<int, DT>{}, std::bool_constant<ACC>{}, integral_constant<int, 2>{}); return true;
    case 3: fn(integral_constant<int, DT>{}, std::bool_constant<ACC>{}, integral_constant<int, 3>{}); return true;
    case 4: fn(integral_constant<int, DT>{}, std::bool_constant<ACC>{}, integral_constant<int, 4>{}); return true;
    default: return false;
    }
}

template <class Fn>
hipError_t with_group(int dtype, const Grads& g, Fn&& fn)
{
    bool ok;
    if (dtype == MP_BF16) ok = g.acc ? with_count<MP_BF16, true>(g.n, fn) : with_count<MP_BF16, false>(g.n, fn);
    else                  ok = g.acc ? with_count<MP_FP16, true>(g.n, fn) : with_count<MP_FP16, false>(g.n, fn);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// First stage of the norm.  One block per chunk, except when the pass reads a
// single 16-bit stream (one micro-batch, no accumulator): a chunk is then only
// 4 KiB, and giving each block kNormChunks16 chunks (64 KiB) made the pass 30-38%
// faster on the 124M, ragged, 1.3B and 8B lists (timed against 1, 4, 8 and 32).
// With two 16-bit streams the lists disagreed (8B faster with 4 chunks, 1.3B
// slower), and from 6 bytes per element up one chunk per block was fastest.
// *used: the blocks launched, i.e. the number of first-stage partials.
// Chunks per norm block: kNormChunks16 when the pass reads a single 16-bit
// stream (no accumulator, one micro-batch), else kNormChunks.
int norm_chunks_per_block(const Grads& g)
{
    return (!g.acc && g.n == 1) ? kNormChunks16 : kNormChunks;
}

hipError_t launch_norm_blocks(const PlanView& p, int grid, const Grads& g, int dtype,
                              double* partials, const DevState* st, hipStream_t s, int* used)
{
    const int blocks = norm_blocks(grid, g);
    *used = blocks;
    const bool single = norm_chunks_per_block(g) == kNormChunks16;
    return with_group(dtype, g, [&](auto dt, auto acc, auto ng) {
        constexpr int D = decltype(dt)::value, N = decltype(ng)::value;
        constexpr bool A = decltype(acc)::value;
        const unsigned lds = lds_for_blocks_per_cu(MPK_NORM_BLOCKS_PER_CU);
        if (single) {
            if constexpr (!A && N == 1)
                k_norm_partial<D, A, N, kNormChunks16><<<blocks, kBlock, lds, s>>>(p, g, st, partials);
        } else {
            k_norm_partial<D, A, N, kNormChunks><<<blocks, kBlock, lds, s>>>(p, g, st, partials);
        }
    });
}

}  // namespace

int norm_blocks(int grid, const Grads& g)
{
    const int cpb = norm_chunks_per_block(g);
    return (grid + cpb - 1) / cpb;
}

hipError_t launch_accumulate(const PlanView& p, int grid, const Grads& g, int first, int dtype,
                             hipStream_t s)
{
    if (g.n < 1 || g.acc) return hipErrorInvalidValue;
    // the accumulator is read unless this is the first accumulation
    Grads gg = g;
    gg.acc = first ? 0 : 1;
    return with_group(dtype, gg, [&](auto dt, auto acc, auto ng) {
        if constexpr (decltype(ng)::value > 0)
            k_accumulate<decltype(dt)::value, !decltype(acc)::value, decltype(ng)::value>
                <<<grid, kBlock,
                   lds_for_blocks_per_cu(first ? MPK_ACC_FIRST_BLOCKS_PER_CU : MPK_ACC_BLOCKS_PER_CU),
                   s>>>(p, gg);
    });
}

// After the first stage: up to kNormDirect partials are summed by the finishing
// block itself, more go through kNormStage2 range sums first.
hipError_t launch_norm_rest(double* partials, int np, float max_norm, DevState* st, double* out,
                            const Tail& tail, hipStream_t s)
{
    if (np <= kNormDirect) {
        k_norm_finish<<<1, kBlock, 0, s>>>(partials, np, max_norm, st, out, tail);
    } else {
        k_norm_stage2<<<kNormStage2, kBlock, 0, s>>>(partials, np, partials + np);
        k_norm_finish<<<1, kBlock, 0, s>>>(partials + np, kNormStage2, max_norm, st, out, tail);
    }
    return hipGetLastError();
}

hipError_t launch_norm(const PlanView& p, int grid, const Grads& g, int dtype, double* partials,
                       float max_norm, DevState* st, const Tail& tail, hipStream_t s)
{
    int np = 0;
    hipError_t err = launch_norm_blocks(p, grid, g, dtype, partials, st, s, &np);
    if (err != hipSuccess) return err;
    return launch_norm_rest(partials, np, max_norm, st, nullptr, tail, s);
}

hipError_t launch_norm_partial(const PlanView& p, int grid, const Grads& g, int dtype,
                               double* partials, const DevState* st, double* out, hipStream_t s)
{
    int np = 0;
    hipError_t err = launch_norm_blocks(p, grid, g, dtype, partials, st, s, &np);
    if (err != hipSuccess) return err;
    return launch_norm_rest(partials, np, 0.0f, nullptr, out, Tail{}, s);
}

hipError_t launch_norm_apply(const double* sumsq, float max_norm, DevState* st, hipStream_t s)
{
    k_norm_apply<<<1, 64, 0, s>>>(sumsq, max_norm, st);
    return hipGetLastError();
}

hipError_t launch_adamw(const PlanView& p, int grid, const Grads& g, int dtype, const AdamArgs& a,
                        const Fp8Out* fp8, DevState* st, bool with_scaler, hipStream_t s)
{
    hipError_t err;
    if (fp8 != nullptr) {
        // the fused FP8 cast is built for a single last micro-batch
        if (g.n > 1) return hipErrorInvalidValue;
        err = with_group(dtype, g, [&](auto dt, auto acc, auto ng) {
            if constexpr (decltype(ng)::value <= 1)
                k_adamw<decltype(dt)::value, decltype(acc)::value, decltype(ng)::value, true>
                    <<<grid, kBlock, lds_for_blocks_per_cu(MPK_ADAMW_BLOCKS_PER_CU), s>>>(
                        p, g, a, fp8, st);
        });
    } else {
        err = with_group(dtype, g, [&](auto dt, auto acc, auto ng) {
            k_adamw<decltype(dt)::value, decltype(acc)::value, decltype(ng)::value, false>
                <<<grid, kBlock, lds_for_blocks_per_cu(MPK_ADAMW_BLOCKS_PER_CU), s>>>(p, g, a, fp8, st);
        });
    }
    if (err != hipSuccess) return err;
    if (a.clock_advanced) return hipSuccess;      // the norm's finish ran the tail
    if (with_scaler) k_clock_scaler<<<1, 64, 0, s>>>(st, a.beta1, a.beta2);
    else             k_adam_clock<<<1, 64, 0, s>>>(st, a.beta1, a.beta2);
    return hipGetLastError();
}

hipError_t launch_scaler(DevState* st, hipStream_t s)
{
    k_scaler<<<1, 64, 0, s>>>(st);
    return hipGetLastError();
}

hipError_t launch_token_weights(const int64_t* counts, int k, float* weights, hipStream_t s)
{
    k_token_weights<<<1, kBlock, 0, s>>>(counts, k, weights);
    return hipGetLastError();
}

hipError_t launch_cast_to_16(const float* src, uint16_t* dst, int64_t n, int dtype, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    if (dtype == MP_BF16) k_cast_to_16<MP_BF16><<<elementwise_grid(n), kBlock, 0, s>>>(src, dst, n);
    else                  k_cast_to_16<MP_FP16><<<elementwise_grid(n), kBlock, 0, s>>>(src, dst, n);
    return hipGetLastError();
}

hipError_t launch_fp8_blocks(const float* src, uint8_t* codes, float* scales, int64_t n, int block,
                             hipStream_t s)
{
    const int64_t nblocks = n / block;
    if (nblocks == 0) return hipSuccess;
    if (block == 16) {
        // one wave pass per wave (timed best on MI355X, like the one-block-per-chunk passes)
        int64_t waves = (n + 1023) / 1024;
        int64_t grid = (waves + kBlock / kWave - 1) / (kBlock / kWave);
        if (grid > (int64_t(1) << 30)) grid = int64_t(1) << 30;
        k_fp8_blocks16<<<static_cast<unsigned>(grid), kBlock, 0, s>>>(src, codes, scales, n);
    } else {
        k_fp8_blocks<<<elementwise_grid(nblocks), kBlock, 0, s>>>(src, codes, scales, nblocks, block);
    }
    return hipGetLastError();
}

hipError_t launch_widen_16(const uint16_t* src, float* dst, int64_t n, int dtype, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    if (dtype == MP_BF16) k_widen_16<MP_BF16><<<elementwise_grid(n), kBlock, 0, s>>>(src, dst, n);
    else                  k_widen_16<MP_FP16><<<elementwise_grid(n), kBlock, 0, s>>>(src, dst, n);
    return hipGetLastError();
}

}  // namespace mpk
