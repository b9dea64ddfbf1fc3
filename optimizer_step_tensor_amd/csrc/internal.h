// Internal layout shared by the C-ABI layer (api.hip) and the kernels (kernels.hip).
//
// Device-resident tables of one plan:
//   TensorDesc[n_tensors]  -- the caller's buffers of each parameter tensor
//   Chunk[n_chunks]        -- contiguous element ranges of at most chunk_elems
//                             elements, never crossing a tensor; every element of
//                             every tensor lies in exactly one chunk
//   double[grid]           -- per-block partial sums of squares of the norm pass
// A gradset is a device array uint16_t*[n_tensors].
// The state is one DevState (the public mp_stats first, so mp_state_read copies
// a prefix).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mpstep.h"

namespace mpk {

// Launch shape (compile-time).  The defaults were chosen by timing variants on
// MI355X with the 1.3B, ragged 4096-tensor and 8B-parameter lists resident:
// chunks of one block pass (2048 elements) with one block per chunk for every
// streaming pass -- the blocks resident at any moment then sweep a compact
// window of memory instead of thousands of separate streams, and the
// dispatcher balances ragged chunks -- and the nontemporal hint on every
// streamed load and store (each byte is touched once per pass).  The
// dispatcher hands consecutive workgroups to the 8 XCDs in turn; the passes
// renumber their blocks so that each XCD takes runs of 64 consecutive chunks
// (512 KiB of every fp32 array) rather than every 8th chunk, which made the
// accumulate and AdamW passes 2-3.5% faster and the norm pass 2-8% faster.
#ifndef MPK_XCD_SPAN
#define MPK_XCD_SPAN 64            // consecutive chunks per XCD turn; 1: no renumbering
#endif
// The passes that write (accumulate, AdamW) take runs of 128 chunks per XCD
// together with the cap on resident blocks below; the read-only norm keeps 64.
#ifndef MPK_ACC_XCD_SPAN
#define MPK_ACC_XCD_SPAN 128
#endif
#ifndef MPK_NORM_XCD_SPAN
#define MPK_NORM_XCD_SPAN MPK_XCD_SPAN
#endif
#ifndef MPK_ADAMW_XCD_SPAN
#define MPK_ADAMW_XCD_SPAN 128
#endif
#ifndef MPK_GROUPS_PER_LANE
#define MPK_GROUPS_PER_LANE 2      // groups of 4 elements per lane per block pass
#endif
#ifndef MPK_ELEM_BLOCKS_PER_CU
#define MPK_ELEM_BLOCKS_PER_CU 0   // grid cap per CU of the streaming passes; 0: one block per chunk
#endif
#ifndef MPK_MAX_CHUNK
#define MPK_MAX_CHUNK 2048         // largest chunk (elements); chunks are powers of two
#endif
#ifndef MPK_CHUNKS_PER_SLOT
#define MPK_CHUNKS_PER_SLOT 4      // chunk size target: total / (this * 8 blocks per CU * CUs)
#endif
#ifndef MPK_NT_LOADS
#define MPK_NT_LOADS 1             // nontemporal hint on streamed loads
#endif
#ifndef MPK_NT_STORES
#define MPK_NT_STORES 1            // nontemporal hint on streamed stores
#endif
// Resident blocks per CU of each streaming pass (0: as many as registers allow,
// 7 for AdamW, 8 for the others).  The cap is imposed by reserving a share of
// the CU's LDS per block.  Timed in alternation on the 8B, 1.3B and ragged
// lists, 4 blocks per CU (with runs of 128 chunks per XCD) made AdamW 2-4% and
// the accumulate passes 1-2% faster on all three, while the read-only norm pass
// only lost from any cap.  Fewer blocks in flight keep fewer DRAM pages open
// at once; the mix of reads and writes is what suffers from too many.
#ifndef MPK_ADAMW_BLOCKS_PER_CU
#define MPK_ADAMW_BLOCKS_PER_CU 4
#endif
#ifndef MPK_NORM_BLOCKS_PER_CU
#define MPK_NORM_BLOCKS_PER_CU 0
#endif
#ifndef MPK_ACC_BLOCKS_PER_CU
#define MPK_ACC_BLOCKS_PER_CU 4
#endif
#ifndef MPK_ACC_FIRST_BLOCKS_PER_CU
#define MPK_ACC_FIRST_BLOCKS_PER_CU 0   // the first accumulation (2 B read, 4 B written) lost
#endif                                  // 20-30% with a cap of 3-6 on every list

// Descriptor tables and device-resident weights read through the constant
// address space (scalar loads); 0: plain loads.  Timed in alternation, scalar
// reads made the first accumulation 5-8% and the later ones (weights read on
// the device) 8-9% faster on every list; AdamW's descriptor reads stay plain
// (0-3% faster there).
#ifndef MPK_SCALAR_TABLES
#define MPK_SCALAR_TABLES 1
#endif
#ifndef MPK_ADAMW_SCALAR_TABLES
#define MPK_ADAMW_SCALAR_TABLES 0
#endif

constexpr int kLdsPerCu = 160 * 1024;                // LDS of one gfx950 CU
// Dynamic LDS bytes per block that let at most n blocks share a CU (n = 0: none).
constexpr unsigned lds_for_blocks_per_cu(int n)
{
    return n > 0 ? static_cast<unsigned>(kLdsPerCu / n) & ~1023u : 0u;
}

constexpr int kBlock = 256;                          // 4 wavefronts of 64 lanes
constexpr int kWave = 64;
constexpr int kXcds = 8;                             // XCDs per MI355X
constexpr int kNormStage2 = 256;                     // second-stage sums of the norm
constexpr int kNormDirect = 8192;                    // at most this many partials: no second stage
constexpr int kMaxCountsK = 64;                      // micro-batches of a pass that reads counts
#ifndef MPK_NORM_CHUNKS
#define MPK_NORM_CHUNKS 1          // consecutive chunks per norm block (several streams)
#endif
#ifndef MPK_NORM_CHUNKS16
#define MPK_NORM_CHUNKS16 16       // consecutive chunks per norm block, one 16-bit stream
#endif
constexpr int kNormChunks = MPK_NORM_CHUNKS;
constexpr int kNormChunks16 = MPK_NORM_CHUNKS16;
constexpr int kGroup = 4;                            // elements per 16-byte fp32 vector
constexpr int kGroupsPerLane = MPK_GROUPS_PER_LANE;
constexpr int kWaveSlab = kWave * kGroup * kGroupsPerLane;   // 512 elements per wave pass
constexpr int kBlockSlab = kBlock * kGroup * kGroupsPerLane; // 2048 elements per block pass

struct TensorDesc {
    float* acc;
    float* master;
    float* m;
    float* v;
    uint16_t* w16;
    int64_t numel;
    float wd_mult;
    int32_t reserved;
};

struct Chunk {
    int32_t tensor;
    int32_t len;      // 1 .. chunk_elems
    int64_t start;    // element offset inside the tensor, a multiple of kBlockSlab
};

struct DevState {
    mp_stats s;             // public part (mp_state_read copies this prefix)
    float inv_scale;        // 1/S (exact: S is a power of two)
    float update_scale;     // fl(inv_scale * clip_coef), set by the norm pass
    float growth, backoff, min_scale, max_scale;
    int32_t interval;
    int32_t enabled;
};

struct PlanView {
    const TensorDesc* tensors;
    const Chunk* chunks;
    int64_t n_chunks;
};

struct AdamArgs {
    float lr, beta1, beta2, eps, weight_decay;
    int32_t clock_advanced;   // 1: the norm's finish already advanced the clock (Tail)
};

// The end of a whole update enqueued by one call: the norm's finishing block
// also advances the optimizer clock and takes the scaler's decision.
struct Tail {
    int32_t on;
    float beta1, beta2;
};

// A micro-batch weight n_i/N: a value passed with the launch or, when ptr is
// set, one read from device memory by every block -- so that target counts
// counted on the device need no host round trip, and a captured graph reads
// each replay's weight.
struct Weight {
    float value;
    const float* ptr;
};

// The 16-bit gradients one pass folds in, in micro-batch order: up to
// kMaxGroup gradsets (device tables uint16_t*[n_tensors]) with their weights,
// after the accumulator when `acc` is set.  Every term is added with the
// roundings of one mp_accumulate call, so a group gives the bits of the same
// micro-batches accumulated one by one.
constexpr int kMaxGroup = 4;

struct Grads {
    const uint16_t* const* set[kMaxGroup];
    Weight w[kMaxGroup];
    int32_t n;        // 0 .. kMaxGroup gradsets
    int32_t acc;      // 1: the accumulator is the first term
    // The first accumulation with its weights computed from the k token counts
    // (device int64[k], k <= kMaxCountsK) instead of w[]; block 0 writes all k
    // weights to weights_out (device float[k]).  NULL counts: the weights are w[].
    const int64_t* counts;
    float* weights_out;
    int32_t k;
};

// FP8 (E4M3) outputs of one tensor for the fused AdamW pass: numel codes and
// numel/16 block scales, or both NULL (the tensor is not cast).
struct Fp8Out {
    uint8_t* codes;
    float* scales;
};

// accumulate: acc = the group's terms (first: without the accumulator), n >= 1
hipError_t launch_accumulate(const PlanView& p, int grid, const Grads& g, int first, int dtype,
                             hipStream_t s);
// First-stage blocks (= partial sums) of the norm pass over group g on a plan of
// `grid` blocks; the pass needs that many doubles plus kNormStage2 of scratch.
int norm_blocks(int grid, const Grads& g);
hipError_t launch_norm(const PlanView& p, int grid, const Grads& g, int dtype, double* partials,
                       float max_norm, DevState* st, const Tail& tail, hipStream_t s);
hipError_t launch_norm_partial(const PlanView& p, int grid, const Grads& g, int dtype,
                               double* partials, const DevState* st, double* out, hipStream_t s);
hipError_t launch_norm_apply(const double* sumsq, float max_norm, DevState* st, hipStream_t s);
// with_scaler: the scaler's decision runs in the same tiny launch as the clock
hipError_t launch_adamw(const PlanView& p, int grid, const Grads& g, int dtype, const AdamArgs& a,
                        const Fp8Out* fp8, DevState* st, bool with_scaler, hipStream_t s);
hipError_t launch_scaler(DevState* st, hipStream_t s);
hipError_t launch_token_weights(const int64_t* counts, int k, float* weights, hipStream_t s);
hipError_t launch_cast_to_16(const float* src, uint16_t* dst, int64_t n, int dtype, hipStream_t s);
hipError_t launch_fp8_blocks(const float* src, uint8_t* codes, float* scales, int64_t n, int block,
                             hipStream_t s);
hipError_t launch_widen_16(const uint16_t* src, float* dst, int64_t n, int dtype, hipStream_t s);

}  // namespace mpk
