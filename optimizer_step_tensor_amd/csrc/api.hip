// C-ABI layer of the mixed-precision update step: argument validation, plan and
// chunk-table construction, device state management and kernel launches.
// Every entry point is declared and documented in include/mpstep.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

using mpk::Chunk;
using mpk::DevState;
using mpk::Fp8Out;
using mpk::TensorDesc;

// The micro-batches one pass folds in after the accumulator, in order: the
// host view of mpk::Grads.  no_acc: the group starts the update (no
// accumulator term).
struct Group {
    const mp_gradset* sets[mpk::kMaxGroup];
    mpk::Weight w[mpk::kMaxGroup];
    int32_t n;
    int32_t no_acc;
    // weights from token counts (mp_accumulate_first_counts), else NULL
    const int64_t* counts;
    float* weights_out;
    int32_t k;
};

struct mp_plan {
    int device;
    int32_t n_tensors;
    int32_t dtype;
    bool has_acc;
    int64_t total;
    int64_t n_chunks;
    int32_t chunk_elems;
    int grid;                 // blocks of the accumulate and AdamW passes
    int norm_grid;            // blocks of the norm pass (= first-stage partial sums)
    TensorDesc* d_tensors;
    Chunk* d_chunks;
    double* d_partials;       // norm_grid first-stage + kNormStage2 second-stage sums
    // call-order bookkeeping: mp_adamw_step must follow mp_unscale_check_norm (or
    // mp_norm_partial + mp_norm_finish)
    bool partial_pending;
    bool norm_pending;
    const mp_state* norm_state;
    Group norm_group;         // the micro-batches the pending norm folded in
    uint64_t norm_gen[mpk::kMaxGroup];   // their gradsets' generations at that time
    std::vector<int64_t> numel;  // per tensor, for validating FP8 output sets
};

constexpr int kGradsetSlots = 4;   // pinned staging slots of mp_gradset_update

struct mp_gradset {
    const mp_plan* plan;
    uint16_t** d_ptrs;
    // mp_gradset_update stages each new table in one of these pinned host
    // slots, round robin; a slot is rewritten only after the copy that last
    // read it has run (its event)
    uint16_t** h_slots[kGradsetSlots];
    hipEvent_t copied[kGradsetSlots];
    int next_slot;
    // bumped by every mp_gradset_update: a norm measured before it folded in
    // other buffers, so the AdamW step that would fold in these is refused
    uint64_t generation;
};

struct mp_fp8set {
    const mp_plan* plan;
    Fp8Out* d_out;            // one entry per tensor of the plan
};

struct mp_state {
    int device;
    DevState* d;
    // an overflow/norm decision was measured into this state and the scaler has
    // not consumed it yet (mp_scaler_update must follow a measurement)
    bool decision_pending;
};

// Norm scratch of mp_update_step_noalloc, for callers that cannot allocate:
// first-stage partial sums, then the second-stage sums.  Each device holds its
// own copy for the life of the process; host code uses the per-device address
// from hipGetSymbolAddress, never this name.
static __device__ __align__(256) double scratch[MP_NOALLOC_MAX_NORM_BLOCKS + mpk::kNormStage2];

namespace {

thread_local std::string g_error;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
double* g_scratch[kMaxDevices];              // device address of `scratch`, per device
hipError_t g_scratch_error[kMaxDevices];     // the lookup's result, once made

// Look up this device's copy of `scratch` once (the device must be current).
// Called when a plan is created, so that the hot call itself never loads code
// or touches the runtime's module tables.
void setup_scratch(int device)
{
    if (device < 0 || device >= kMaxDevices) return;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[device] != nullptr) return;
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_error[device] = e;
    if (e == hipSuccess) g_scratch[device] = static_cast<double*>(ptr);
}

double* scratch_of(int device, hipError_t* err)
{
    *err = hipErrorInvalidDevice;
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    *err = g_scratch[device] != nullptr ? hipSuccess : g_scratch_error[device];
    return g_scratch[device];
}

mp_status fail(mp_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

mp_status ok()
{
    g_error.clear();
    return MP_OK;
}

mp_status hip_fail(hipError_t e, const char* what)
{
    return fail(MP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Entry points that build host tables run their body through this, so that a
// failed host allocation becomes MP_ERR_NOMEM instead of an exception crossing
// the C ABI.
template <class Body>
mp_status guarded(Body&& body)
{
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(MP_ERR_NOMEM, "host allocation failed");
    }
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool is_pow2(float x)
{
    if (!(x > 0.0f) || !std::isfinite(x)) return false;
    int e;
    return std::frexp(x, &e) == 0.5f;
}

bool valid_dtype(int d)
{
    return d == MP_BF16 || d == MP_FP16;
}


int device_cus(int device)
{
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
}

// Chunk size: a power-of-two multiple of one block pass, small enough that the
// table has several chunks per block on small models, large enough that the
// table stays small (16 B per chunk) on large ones.
int32_t pick_chunk_elems(int64_t total, int grid_cap)
{
    int64_t target = total / (int64_t(MPK_CHUNKS_PER_SLOT) * grid_cap);
    int64_t ch = mpk::kBlockSlab;
    while (ch < target && ch < MPK_MAX_CHUNK) ch <<= 1;
    return static_cast<int32_t>(ch);
}

int32_t chunk_elems_of(int32_t n_tensors, const int64_t* numel, int cus)
{
    int64_t total = 0;
    for (int32_t i = 0; i < n_tensors; ++i) total += numel[i];
    return pick_chunk_elems(total, cus * 8);
}

// Whether a list needs more chunks than a launch grid holds, whatever the
// chunk size (it is at most MPK_MAX_CHUNK): checked before any table is built.
bool too_many_chunks(int32_t n_tensors, const int64_t* numel)
{
    int64_t n = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        n += (numel[i] + MPK_MAX_CHUNK - 1) / MPK_MAX_CHUNK;
        if (n > INT32_MAX) return true;
    }
    return false;
}

// The number of chunks build_chunks makes, without making them.
int64_t count_chunks(int32_t n_tensors, const int64_t* numel, int cus)
{
    const int64_t ch = chunk_elems_of(n_tensors, numel, cus);
    int64_t n = 0;
    for (int32_t i = 0; i < n_tensors; ++i) n += (numel[i] + ch - 1) / ch;
    return n;
}

// The chunk table of a tensor list: every tensor cut into ranges of at most
// chunk_elems elements (the last one ragged), tensor by tensor, in order.
int32_t build_chunks(int32_t n_tensors, const int64_t* numel, int cus, std::vector<Chunk>& chunks)
{
    const int32_t ch = chunk_elems_of(n_tensors, numel, cus);
    chunks.clear();
    for (int32_t i = 0; i < n_tensors; ++i)
        for (int64_t s = 0; s < numel[i]; s += ch)
            chunks.push_back(Chunk{i, static_cast<int32_t>(std::min<int64_t>(ch, numel[i] - s)), s});
    return ch;
}

template <class T>
hipError_t upload(T** dst, const std::vector<T>& src)
{
    *dst = nullptr;
    if (src.empty()) return hipSuccess;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), src.size() * sizeof(T));
    if (e != hipSuccess) return e;
    e = hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(*dst);
        *dst = nullptr;
    }
    return e;
}

mpk::PlanView view(const mp_plan* p)
{
    return mpk::PlanView{p->d_tensors, p->d_chunks, p->n_chunks};
}

mp_status check_hparams(const mp_adamw_hparams* hp)
{
    if (hp == nullptr) return fail(MP_ERR_INVALID, "hparams is NULL");
    if (!std::isfinite(hp->lr) || hp->lr < 0.0f) return fail(MP_ERR_INVALID, "lr must be finite and >= 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f)) return fail(MP_ERR_INVALID, "beta1 must be in [0, 1)");
    if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) return fail(MP_ERR_INVALID, "beta2 must be in [0, 1)");
    if (!std::isfinite(hp->eps) || !(hp->eps > 0.0f)) return fail(MP_ERR_INVALID, "eps must be finite and > 0");
    if (!std::isfinite(hp->weight_decay) || hp->weight_decay < 0.0f)
        return fail(MP_ERR_INVALID, "weight_decay must be finite and >= 0");
    return MP_OK;
}


// Plans and states are bound to the device current at their creation; a hot
// call made with another device current would launch on the wrong GPU.
mp_status check_device(int device, const char* what)
{
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != device)
        return fail(MP_ERR_INVALID, "%s was created on device %d but device %d is current", what,
                    device, cur);
    return MP_OK;
}

mp_status check_devices(const mp_plan* plan, const mp_state* state)
{
    mp_status st = plan ? check_device(plan->device, "the plan") : MP_OK;
    if (st == MP_OK && state) st = check_device(state->device, "the state");
    return st;
}

mp_status check_weight(mpk::Weight w, const char* name)
{
    if (w.ptr != nullptr) {
        if ((reinterpret_cast<uintptr_t>(w.ptr) & 3u) != 0)
            return fail(MP_ERR_ALIGN, "%s must be a 4-byte aligned device pointer", name);
        return MP_OK;          // the value is the device's: a bad one makes the step overflow
    }
    if (!std::isfinite(w.value) || !(w.value > 0.0f))
        return fail(MP_ERR_INVALID, "%s must be finite and > 0", name);
    return MP_OK;
}

mp_status check_group(const mp_plan* plan, const Group& g)
{
    if (g.n < 0 || g.n > mpk::kMaxGroup)
        return fail(MP_ERR_INVALID, "a group holds 1 to %d gradsets", mpk::kMaxGroup);
    for (int i = 0; i < g.n; ++i) {
        if (g.sets[i] == nullptr) return fail(MP_ERR_INVALID, "gradset %d of the group is NULL", i);
        if (g.sets[i]->plan != plan) return fail(MP_ERR_INVALID, "gradset belongs to another plan");
        if (g.counts != nullptr) continue;   // weights computed on the device from the counts
        mp_status st = check_weight(g.w[i], "a micro-batch weight");
        if (st != MP_OK) return st;
    }
    if (g.n == 0 && g.no_acc)
        return fail(MP_ERR_INVALID, "last_is_first needs a gradset");
    if (!g.no_acc && !plan->has_acc)
        return fail(MP_ERR_INVALID, "the plan has no accumulators: pass the only micro-batch "
                                    "as `last` with last_is_first = 1");
    return MP_OK;
}

bool same_weight(mpk::Weight a, mpk::Weight b)
{
    return a.ptr == b.ptr && (a.ptr != nullptr || a.value == b.value);
}

bool same_group(const Group& a, const Group& b)
{
    if (a.n != b.n || a.no_acc != b.no_acc) return false;
    for (int i = 0; i < a.n; ++i)
        if (a.sets[i] != b.sets[i] || !same_weight(a.w[i], b.w[i])) return false;
    return true;
}

// The group a pending norm measured, with its gradsets' generations.
void remember_norm_group(mp_plan* plan, const Group& g)
{
    plan->norm_group = g;
    for (int i = 0; i < g.n; ++i) plan->norm_gen[i] = g.sets[i]->generation;
}

// g is the group the pending norm measured and none of its gradsets has been
// pointed at other buffers since.
bool norm_measured(const mp_plan* plan, const Group& g)
{
    if (!same_group(plan->norm_group, g)) return false;
    for (int i = 0; i < g.n; ++i)
        if (g.sets[i]->generation != plan->norm_gen[i]) return false;
    return true;
}

mpk::Grads device_group(const Group& g)
{
    mpk::Grads d{};
    for (int i = 0; i < g.n; ++i) {
        d.set[i] = g.sets[i]->d_ptrs;
        d.w[i] = g.w[i];
    }
    d.n = g.n;
    d.acc = g.no_acc ? 0 : 1;
    d.counts = g.counts;
    d.weights_out = g.weights_out;
    d.k = g.k;
    return d;
}

mpk::Weight host_weight(float w)
{
    return mpk::Weight{w, nullptr};
}

mpk::Weight device_weight(const float* w)
{
    return mpk::Weight{0.0f, w};
}

// The single-`last` form of the hot calls as a group of 0 or 1.
Group single(const mp_gradset* last, mpk::Weight w_last, int32_t last_is_first)
{
    Group g{};
    g.n = last != nullptr ? 1 : 0;
    g.sets[0] = last;
    g.w[0] = w_last;
    g.no_acc = last_is_first ? 1 : 0;
    return g;
}

// A caller's array of n gradsets and n weights (host floats, or a device array
// of n floats when on_device).
mp_status make_group(const mp_gradset* const* sets, const float* weights, int32_t n,
                     int32_t on_device, int32_t no_acc, Group* out)
{
    if (n < 1 || n > mpk::kMaxGroup)
        return fail(MP_ERR_INVALID, "a group holds 1 to %d gradsets", mpk::kMaxGroup);
    if (sets == nullptr || weights == nullptr)
        return fail(MP_ERR_INVALID, "sets and weights are required");
    Group g{};
    g.n = n;
    g.no_acc = no_acc ? 1 : 0;
    for (int i = 0; i < n; ++i) {
        g.sets[i] = sets[i];
        g.w[i] = on_device ? device_weight(weights + i) : host_weight(weights[i]);
    }
    *out = g;
    return MP_OK;
}

}  // namespace

extern "C" {

const char* mp_status_string(mp_status status)
{
    switch (status) {
    case MP_OK: return "MP_OK";
    case MP_ERR_INVALID: return "MP_ERR_INVALID";
    case MP_ERR_ALIGN: return "MP_ERR_ALIGN";
    case MP_ERR_NOMEM: return "MP_ERR_NOMEM";
    case MP_ERR_HIP: return "MP_ERR_HIP";
    case MP_ERR_ORDER: return "MP_ERR_ORDER";
    default: break;
    }
    return "MP_ERR_UNKNOWN";
}

const char* mp_last_error(void)
{
    return g_error.c_str();
}

int32_t mp_abi_version(void)
{
    return MPSTEP_ABI_VERSION;
}

mp_status mp_token_weights(int32_t k, const int64_t* counts, float* weights_out)
{
    if (k < 1 || counts == nullptr || weights_out == nullptr)
        return fail(MP_ERR_INVALID, "need k >= 1 counts and an output array");
    const int64_t limit = int64_t(1) << 53;
    int64_t total = 0;
    for (int32_t i = 0; i < k; ++i) {
        if (counts[i] <= 0) return fail(MP_ERR_INVALID, "micro-batch %d has no targets", i);
        if (counts[i] > limit - total)
            return fail(MP_ERR_INVALID, "total target count exceeds 2^53");
        total += counts[i];
    }
    for (int32_t i = 0; i < k; ++i)
        weights_out[i] = static_cast<float>(static_cast<double>(counts[i]) / static_cast<double>(total));
    return ok();
}

size_t mp_state_bytes_per_param(mp_dtype16 dtype, int32_t with_accumulator)
{
    (void)dtype;  // both 16-bit formats take 2 bytes
    const size_t model16 = 2, grad16 = 2, master = 4, m = 4, v = 4;
    return model16 + grad16 + master + m + v + (with_accumulator ? 4 : 0);
}

mp_status mp_plan_create(int32_t n_tensors, const int64_t* numel, mp_dtype16 dtype,
                         void* const* acc, void* const* master, void* const* m, void* const* v,
                         void* const* w16, const float* wd_mult, mp_plan** out)
{
    return guarded([&]() -> mp_status {
        if (out == nullptr) return fail(MP_ERR_INVALID, "out is NULL");
        *out = nullptr;
        if (n_tensors < 1) return fail(MP_ERR_INVALID, "n_tensors must be >= 1");
        if (!valid_dtype(dtype)) return fail(MP_ERR_INVALID, "unknown dtype %d", (int)dtype);
        if (numel == nullptr || master == nullptr || m == nullptr || v == nullptr || w16 == nullptr)
            return fail(MP_ERR_INVALID, "numel, master, m, v and w16 arrays are required");
        std::vector<TensorDesc> tensors(n_tensors);
        std::vector<Chunk> chunks;
        int64_t total = 0;
        for (int32_t i = 0; i < n_tensors; ++i) {
            if (numel[i] < 1 || numel[i] > (int64_t(1) << 40))
                return fail(MP_ERR_INVALID, "tensor %d: numel %lld out of range", i, (long long)numel[i]);
            void* ptrs[5] = {acc ? acc[i] : nullptr, master[i], m[i], v[i], w16[i]};
            for (int k = 0; k < 5; ++k) {
                if (k == 0 && acc == nullptr) continue;
                if (ptrs[k] == nullptr) return fail(MP_ERR_INVALID, "tensor %d: NULL buffer", i);
                if (!aligned16(ptrs[k])) return fail(MP_ERR_ALIGN, "tensor %d: buffer not 16-byte aligned", i);
            }
            const float mult = wd_mult ? wd_mult[i] : 1.0f;
            if (!std::isfinite(mult) || mult < 0.0f)
                return fail(MP_ERR_INVALID, "tensor %d: wd_mult must be finite and >= 0", i);
            tensors[i] = TensorDesc{static_cast<float*>(ptrs[0]), static_cast<float*>(ptrs[1]),
                                    static_cast<float*>(ptrs[2]), static_cast<float*>(ptrs[3]),
                                    static_cast<uint16_t*>(ptrs[4]), numel[i], mult, 0};
            total += numel[i];
            if (total > (int64_t(1) << 48))
                return fail(MP_ERR_INVALID, "the plan holds more than 2^48 elements");
        }
        if (too_many_chunks(n_tensors, numel))
            return fail(MP_ERR_INVALID, "the plan needs more than 2^31 - 1 chunks");
        int device = 0;
        hipError_t e = hipGetDevice(&device);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        setup_scratch(device);
        const int cus = device_cus(device);
        const int64_t grid_cap = MPK_ELEM_BLOCKS_PER_CU > 0 ? int64_t(cus) * MPK_ELEM_BLOCKS_PER_CU
                                                             : int64_t(1) << 30;
        // the norm pass launches one block per chunk (or per group of chunks):
        // refuse a chunk count beyond a launch grid before building the table
        if (count_chunks(n_tensors, numel, cus) > INT32_MAX)
            return fail(MP_ERR_INVALID, "the plan needs more than 2^31 - 1 chunks");
        const int32_t ch = build_chunks(n_tensors, numel, cus, chunks);
        mp_plan* p = new (std::nothrow) mp_plan();
        if (p == nullptr) return fail(MP_ERR_NOMEM, "host allocation failed");
        p->device = device;
        p->n_tensors = n_tensors;
        p->dtype = dtype;
        p->has_acc = acc != nullptr;
        p->total = total;
        p->n_chunks = static_cast<int64_t>(chunks.size());
        p->chunk_elems = ch;
        p->grid = static_cast<int>(std::min<int64_t>(p->n_chunks, grid_cap));
        // the accumulate and AdamW blocks stride over the chunks when the grid is
        // capped; the norm's blocks each take a fixed chunk (or 16), never capped
        p->norm_grid = static_cast<int>(p->n_chunks);
        p->numel.assign(numel, numel + n_tensors);
        // every partial sum is written by its block before any kernel reads it
        const size_t partial_bytes = (static_cast<size_t>(p->norm_grid) + mpk::kNormStage2) * sizeof(double);
        if ((e = upload(&p->d_tensors, tensors)) != hipSuccess ||
            (e = upload(&p->d_chunks, chunks)) != hipSuccess ||
            (e = hipMalloc(reinterpret_cast<void**>(&p->d_partials), partial_bytes)) != hipSuccess) {
            mp_plan_destroy(p);
            return e == hipErrorOutOfMemory ? fail(MP_ERR_NOMEM, "device allocation failed")
                                            : hip_fail(e, "plan upload");
        }
        *out = p;
        return ok();
    });
}

mp_status mp_plan_destroy(mp_plan* plan)
{
    if (plan == nullptr) return ok();
    (void)hipFree(plan->d_tensors);
    (void)hipFree(plan->d_chunks);
    (void)hipFree(plan->d_partials);
    delete plan;
    return ok();
}

mp_status mp_plan_info(const mp_plan* plan, int32_t* n_tensors, int64_t* total_params,
                       int64_t* n_chunks, int32_t* chunk_elems)
{
    if (plan == nullptr) return fail(MP_ERR_INVALID, "plan is NULL");
    if (n_tensors) *n_tensors = plan->n_tensors;
    if (total_params) *total_params = plan->total;
    if (n_chunks) *n_chunks = plan->n_chunks;
    if (chunk_elems) *chunk_elems = plan->chunk_elems;
    return ok();
}

mp_status mp_chunk_layout(int32_t n_tensors, const int64_t* numel, int32_t n_cus,
                          int32_t* chunk_elems, int64_t* n_chunks, int32_t* tensor_out,
                          int64_t* start_out, int32_t* len_out, int64_t capacity)
{
    return guarded([&]() -> mp_status {
        if (n_tensors < 1 || numel == nullptr || n_cus < 1)
            return fail(MP_ERR_INVALID, "need n_tensors >= 1, numel and n_cus >= 1");
        for (int32_t i = 0; i < n_tensors; ++i)
            if (numel[i] < 1 || numel[i] > (int64_t(1) << 40))
                return fail(MP_ERR_INVALID, "tensor %d: numel out of range", i);
        if (too_many_chunks(n_tensors, numel) || count_chunks(n_tensors, numel, n_cus) > INT32_MAX)
            return fail(MP_ERR_INVALID, "the list needs more than 2^31 - 1 chunks");
        std::vector<Chunk> chunks;
        const int32_t ch = build_chunks(n_tensors, numel, n_cus, chunks);
        if (chunk_elems) *chunk_elems = ch;
        if (n_chunks) *n_chunks = static_cast<int64_t>(chunks.size());
        const int64_t n = std::min<int64_t>(capacity, static_cast<int64_t>(chunks.size()));
        for (int64_t c = 0; c < n; ++c) {
            if (tensor_out) tensor_out[c] = chunks[c].tensor;
            if (start_out) start_out[c] = chunks[c].start;
            if (len_out) len_out[c] = chunks[c].len;
        }
        return ok();
    });
}

namespace {

mp_status check_grad_ptrs(const mp_plan* plan, void* const* g16, std::vector<uint16_t*>& ptrs)
{
    ptrs.resize(plan->n_tensors);
    for (int32_t i = 0; i < plan->n_tensors; ++i) {
        if (g16[i] == nullptr) return fail(MP_ERR_INVALID, "gradient %d is NULL", i);
        if (!aligned16(g16[i])) return fail(MP_ERR_ALIGN, "gradient %d not 16-byte aligned", i);
        ptrs[i] = static_cast<uint16_t*>(g16[i]);
    }
    return MP_OK;
}

void free_gradset(mp_gradset* g)
{
    for (int i = 0; i < kGradsetSlots; ++i) {
        if (g->copied[i] != nullptr) {
            (void)hipEventSynchronize(g->copied[i]);   // no pending copy reads the slot
            (void)hipEventDestroy(g->copied[i]);
        }
        if (g->h_slots[i] != nullptr) (void)hipHostFree(g->h_slots[i]);
    }
    (void)hipFree(g->d_ptrs);
    delete g;
}

}  // namespace

mp_status mp_gradset_create(const mp_plan* plan, void* const* g16, mp_gradset** out)
{
    return guarded([&]() -> mp_status {
        if (out == nullptr) return fail(MP_ERR_INVALID, "out is NULL");
        *out = nullptr;
        if (plan == nullptr || g16 == nullptr) return fail(MP_ERR_INVALID, "plan and g16 are required");
        std::vector<uint16_t*> ptrs;
        mp_status st = check_grad_ptrs(plan, g16, ptrs);
        if (st != MP_OK) return st;
        mp_gradset* g = new (std::nothrow) mp_gradset();
        if (g == nullptr) return fail(MP_ERR_NOMEM, "host allocation failed");
        g->plan = plan;
        hipError_t e = upload(&g->d_ptrs, ptrs);
        const size_t slot_bytes = ptrs.size() * sizeof(uint16_t*);
        for (int i = 0; i < kGradsetSlots && e == hipSuccess; ++i) {
            e = hipHostMalloc(reinterpret_cast<void**>(&g->h_slots[i]), slot_bytes, hipHostMallocDefault);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&g->copied[i], hipEventDisableTiming);
        }
        if (e != hipSuccess) {
            free_gradset(g);
            return e == hipErrorOutOfMemory ? fail(MP_ERR_NOMEM, "allocation failed")
                                            : hip_fail(e, "gradset upload");
        }
        *out = g;
        return ok();
    });
}

mp_status mp_gradset_update(mp_gradset* set, void* const* g16, mp_stream stream)
{
    return guarded([&]() -> mp_status {
        if (set == nullptr || g16 == nullptr) return fail(MP_ERR_INVALID, "gradset and g16 are required");
        std::vector<uint16_t*> ptrs;
        mp_status st = check_grad_ptrs(set->plan, g16, ptrs);
        if (st == MP_OK) st = check_device(set->plan->device, "the gradset's plan");
        if (st != MP_OK) return st;
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &cap);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone)
            return fail(MP_ERR_INVALID, "mp_gradset_update cannot be captured in a graph: a replay "
                                        "would copy whatever the staging slot holds then");
        const int slot = set->next_slot;
        e = hipEventSynchronize(set->copied[slot]);     // the copy that last read this slot has run
        if (e != hipSuccess) return hip_fail(e, "gradset slot wait");
        std::memcpy(set->h_slots[slot], ptrs.data(), ptrs.size() * sizeof(uint16_t*));
        e = hipMemcpyAsync(set->d_ptrs, set->h_slots[slot], ptrs.size() * sizeof(uint16_t*),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipEventRecord(set->copied[slot], s);
        if (e != hipSuccess) return hip_fail(e, "gradset update");
        set->next_slot = (slot + 1) % kGradsetSlots;
        set->generation += 1;
        return ok();
    });
}

mp_status mp_gradset_destroy(mp_gradset* set)
{
    if (set == nullptr) return ok();
    free_gradset(set);
    return ok();
}

mp_status mp_fp8set_create(const mp_plan* plan, void* const* codes, void* const* scales,
                           mp_fp8set** out)
{
    return guarded([&]() -> mp_status {
        if (out == nullptr) return fail(MP_ERR_INVALID, "out is NULL");
        *out = nullptr;
        if (plan == nullptr || codes == nullptr || scales == nullptr)
            return fail(MP_ERR_INVALID, "plan, codes and scales are required");
        std::vector<Fp8Out> outs(plan->n_tensors);
        int32_t n_cast = 0;
        for (int32_t i = 0; i < plan->n_tensors; ++i) {
            if (codes[i] == nullptr && scales[i] == nullptr) {
                outs[i] = Fp8Out{nullptr, nullptr};
                continue;
            }
            if (codes[i] == nullptr || scales[i] == nullptr)
                return fail(MP_ERR_INVALID, "tensor %d: codes and scales must both be set or both NULL", i);
            if (plan->numel[i] % 16 != 0)
                return fail(MP_ERR_INVALID, "tensor %d: numel %lld is not a multiple of 16", i,
                            (long long)plan->numel[i]);
            if (!aligned16(codes[i]) || (reinterpret_cast<uintptr_t>(scales[i]) & 3u) != 0)
                return fail(MP_ERR_ALIGN, "tensor %d: codes must be 16-byte aligned, scales 4-byte aligned", i);
            outs[i] = Fp8Out{static_cast<uint8_t*>(codes[i]), static_cast<float*>(scales[i])};
            ++n_cast;
        }
        if (n_cast == 0) return fail(MP_ERR_INVALID, "no tensor has FP8 outputs");
        mp_status st = check_device(plan->device, "the plan");
        if (st != MP_OK) return st;
        mp_fp8set* f = new (std::nothrow) mp_fp8set();
        if (f == nullptr) return fail(MP_ERR_NOMEM, "host allocation failed");
        f->plan = plan;
        hipError_t e = upload(&f->d_out, outs);
        if (e != hipSuccess) {
            delete f;
            return e == hipErrorOutOfMemory ? fail(MP_ERR_NOMEM, "device allocation failed")
                                            : hip_fail(e, "fp8 set upload");
        }
        *out = f;
        return ok();
    });
}

mp_status mp_fp8set_destroy(mp_fp8set* set)
{
    if (set == nullptr) return ok();
    (void)hipFree(set->d_out);
    delete set;
    return ok();
}

mp_status mp_state_create(const mp_scaler_cfg* cfg, mp_state** out)
{
    if (out == nullptr) return fail(MP_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (cfg == nullptr) return fail(MP_ERR_INVALID, "cfg is NULL");
    if (!is_pow2(cfg->init_scale) || !is_pow2(cfg->growth) || !is_pow2(cfg->backoff) ||
        !is_pow2(cfg->min_scale) || !is_pow2(cfg->max_scale))
        return fail(MP_ERR_INVALID, "scales, growth and backoff must be positive powers of two");
    if (cfg->growth < 1.0f || cfg->backoff > 1.0f)
        return fail(MP_ERR_INVALID, "need growth >= 1 and backoff <= 1");
    if (!(cfg->min_scale <= cfg->init_scale && cfg->init_scale <= cfg->max_scale))
        return fail(MP_ERR_INVALID, "need min_scale <= init_scale <= max_scale");
    if (cfg->interval < 1) return fail(MP_ERR_INVALID, "interval must be >= 1");
    DevState h;
    std::memset(&h, 0, sizeof h);
    h.s.scale = cfg->init_scale;
    h.s.beta1_pow = 1.0;
    h.s.beta2_pow = 1.0;
    h.s.clip_coef = 1.0f;
    h.inv_scale = 1.0f / cfg->init_scale;
    h.update_scale = h.inv_scale;
    h.growth = cfg->growth;
    h.backoff = cfg->backoff;
    h.min_scale = cfg->min_scale;
    h.max_scale = cfg->max_scale;
    h.interval = cfg->interval;
    h.enabled = cfg->enabled ? 1 : 0;
    mp_state* s = new (std::nothrow) mp_state();
    if (s == nullptr) return fail(MP_ERR_NOMEM, "host allocation failed");
    hipError_t e = hipGetDevice(&s->device);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&s->d), sizeof(DevState));
    if (e == hipSuccess) e = hipMemcpy(s->d, &h, sizeof h, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(s->d);
        delete s;
        return hip_fail(e, "state allocation");
    }
    *out = s;
    return ok();
}

mp_status mp_state_destroy(mp_state* state)
{
    if (state == nullptr) return ok();
    (void)hipFree(state->d);
    delete state;
    return ok();
}

mp_status mp_state_read(const mp_state* state, mp_stats* out, mp_stream stream)
{
    if (state == nullptr || out == nullptr) return fail(MP_ERR_INVALID, "state and out are required");
    hipError_t e = hipMemcpyAsync(out, &state->d->s, sizeof(mp_stats), hipMemcpyDeviceToHost,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    return ok();
}

namespace {

const char kBlobMagic[8] = {'M', 'P', 'S', 'T', 'A', 'T', 'E', '1'};
constexpr uint32_t kBlobHeader = 16;

mp_status check_scaler_fields(const DevState& d)
{
    mp_scaler_cfg c{d.s.scale, d.growth, d.backoff, d.min_scale, d.max_scale, d.interval, d.enabled};
    if (!is_pow2(c.init_scale) || !is_pow2(c.growth) || !is_pow2(c.backoff) ||
        !is_pow2(c.min_scale) || !is_pow2(c.max_scale) || c.growth < 1.0f || c.backoff > 1.0f ||
        !(c.min_scale <= c.init_scale && c.init_scale <= c.max_scale) || c.interval < 1)
        return fail(MP_ERR_INVALID, "state blob: scaler fields out of range");
    if (d.s.good_steps < 0 || d.s.good_steps >= d.interval || d.s.step < 0 || d.s.skipped_total < 0)
        return fail(MP_ERR_INVALID, "state blob: counters out of range");
    if (!(d.s.beta1_pow > 0.0 && d.s.beta1_pow <= 1.0 && d.s.beta2_pow > 0.0 && d.s.beta2_pow <= 1.0))
        return fail(MP_ERR_INVALID, "state blob: beta powers out of range");
    return MP_OK;
}

}  // namespace

mp_status mp_state_export(const mp_state* state, void* blob, size_t blob_bytes, mp_stream stream)
{
    if (state == nullptr || blob == nullptr) return fail(MP_ERR_INVALID, "state and blob are required");
    if (blob_bytes < MP_STATE_BLOB_BYTES) return fail(MP_ERR_INVALID, "blob needs MP_STATE_BLOB_BYTES bytes");
    static_assert(kBlobHeader + sizeof(DevState) <= MP_STATE_BLOB_BYTES, "blob too small");
    unsigned char* b = static_cast<unsigned char*>(blob);
    std::memset(b, 0, MP_STATE_BLOB_BYTES);
    std::memcpy(b, kBlobMagic, 8);
    const uint32_t version = MPSTEP_ABI_VERSION, payload = sizeof(DevState);
    std::memcpy(b + 8, &version, 4);
    std::memcpy(b + 12, &payload, 4);
    hipError_t e = hipMemcpyAsync(b + kBlobHeader, state->d, sizeof(DevState), hipMemcpyDeviceToHost,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    return ok();
}

mp_status mp_state_import(mp_state* state, const void* blob, size_t blob_bytes, mp_stream stream)
{
    if (state == nullptr || blob == nullptr) return fail(MP_ERR_INVALID, "state and blob are required");
    if (blob_bytes < MP_STATE_BLOB_BYTES) return fail(MP_ERR_INVALID, "blob needs MP_STATE_BLOB_BYTES bytes");
    const unsigned char* b = static_cast<const unsigned char*>(blob);
    uint32_t version = 0, payload = 0;
    std::memcpy(&version, b + 8, 4);
    std::memcpy(&payload, b + 12, 4);
    if (std::memcmp(b, kBlobMagic, 8) != 0 || version != MPSTEP_ABI_VERSION || payload != sizeof(DevState))
        return fail(MP_ERR_INVALID, "not a state blob of this library version");
    DevState d;
    std::memcpy(&d, b + kBlobHeader, sizeof d);
    mp_status st = check_scaler_fields(d);
    if (st != MP_OK) return st;
    d.inv_scale = 1.0f / d.s.scale;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(state->d, &d, sizeof d, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);   // `d` lives on this stack frame
    if (e != hipSuccess) return hip_fail(e, "state import");
    state->decision_pending = false;                    // the blob is a state between steps
    return ok();
}

mp_status mp_state_scale_ptr(const mp_state* state, const float** dev_scale)
{
    if (state == nullptr || dev_scale == nullptr) return fail(MP_ERR_INVALID, "state and out are required");
    *dev_scale = &state->d->s.scale;
    return ok();
}

namespace {

mp_status accumulate(mp_plan* plan, const Group& g, int32_t first, mp_stream stream)
{
    if (plan == nullptr) return fail(MP_ERR_INVALID, "plan is required");
    if (g.n < 1) return fail(MP_ERR_INVALID, "a gradset is required");
    if (!plan->has_acc) return fail(MP_ERR_INVALID, "the plan has no accumulators");
    Group gg = g;
    gg.no_acc = 1;            // the accumulator is the destination, not a term
    mp_status st = check_group(plan, gg);
    if (st == MP_OK) st = check_devices(plan, nullptr);
    if (st != MP_OK) return st;
    hipError_t e = mpk::launch_accumulate(view(plan), plan->grid, device_group(gg), first != 0,
                                          plan->dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "accumulate launch");
    // the buffers changed: a norm measured before this no longer describes them
    plan->partial_pending = false;
    plan->norm_pending = false;
    return ok();
}

// partials: norm_blocks + kNormStage2 doubles of device scratch (NULL: the plan's).
// tail.on: the whole update is enqueued by one call (update_step), so the norm's
// finish also advances the clock and takes the scaler's decision.
mp_status unscale_check_norm(mp_plan* plan, mp_state* state, const Group& g, float max_norm,
                             mp_stream stream, double* partials = nullptr,
                             mpk::Tail tail = mpk::Tail{})
{
    if (plan == nullptr || state == nullptr) return fail(MP_ERR_INVALID, "plan and state are required");
    mp_status st = check_group(plan, g);
    if (st != MP_OK) return st;
    if (std::isnan(max_norm) || std::isinf(max_norm)) return fail(MP_ERR_INVALID, "max_norm must be finite");
    st = check_devices(plan, state);
    if (st != MP_OK) return st;
    hipError_t e = mpk::launch_norm(view(plan), plan->norm_grid, device_group(g), plan->dtype,
                                    partials != nullptr ? partials : plan->d_partials, max_norm,
                                    state->d, tail, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "norm launch");
    state->decision_pending = true;
    plan->partial_pending = false;
    plan->norm_pending = true;
    plan->norm_state = state;
    remember_norm_group(plan, g);
    return ok();
}

// with_scaler: the scaler's decision follows in the same tiny launch as the
// clock; clock_advanced: both already ran in the norm's finish (update_step).
mp_status adamw_step(mp_plan* plan, mp_state* state, const Group& g, const mp_adamw_hparams* hp,
                     const Fp8Out* fp8, mp_stream stream, bool with_scaler = false,
                     bool clock_advanced = false)
{
    if (plan == nullptr || state == nullptr) return fail(MP_ERR_INVALID, "plan and state are required");
    mp_status st = check_hparams(hp);
    if (st != MP_OK) return st;
    st = check_group(plan, g);
    if (st != MP_OK) return st;
    if (!plan->norm_pending || plan->norm_state != state || !norm_measured(plan, g))
        return fail(MP_ERR_ORDER, "the AdamW step must follow mp_unscale_check_norm on the same "
                                  "plan and state, with the same last micro-batch arguments and "
                                  "no mp_gradset_update of them in between");
    st = check_devices(plan, state);
    if (st != MP_OK) return st;
    mpk::AdamArgs a{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay,
                    clock_advanced ? 1 : 0};
    hipError_t e = mpk::launch_adamw(view(plan), plan->grid, device_group(g), plan->dtype, a, fp8,
                                     state->d, with_scaler, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "adamw launch");
    plan->norm_pending = false;
    if (with_scaler) state->decision_pending = false;   // the decision ran in the same launch
    return ok();
}

mp_status update_step(mp_plan* plan, mp_state* state, const Group& g, float max_norm,
                      const mp_adamw_hparams* hp, mp_stream stream, bool noalloc = false)
{
    // every structural check first, so that an error enqueues nothing
    if (plan == nullptr || state == nullptr) return fail(MP_ERR_INVALID, "plan and state are required");
    mp_status st = check_hparams(hp);
    if (st == MP_OK) st = check_group(plan, g);
    if (st == MP_OK && (std::isnan(max_norm) || std::isinf(max_norm)))
        st = fail(MP_ERR_INVALID, "max_norm must be finite");
    if (st == MP_OK) st = check_devices(plan, state);
    if (st != MP_OK) return st;
    double* partials = nullptr;
    if (noalloc) {
        const int blocks = mpk::norm_blocks(plan->norm_grid, device_group(g));
        if (blocks > MP_NOALLOC_MAX_NORM_BLOCKS)
            return fail(MP_ERR_INVALID, "the norm pass of this plan takes %d blocks; "
                        "mp_update_step_noalloc holds the partial sums of at most %d",
                        blocks, MP_NOALLOC_MAX_NORM_BLOCKS);
        hipError_t e = hipSuccess;
        partials = scratch_of(plan->device, &e);
        if (partials == nullptr) return hip_fail(e, "scratch of mp_update_step_noalloc");
    }
    // the finish of the norm takes the clock and the scaler's decision (the tail):
    // nothing else can run between the two passes of this call
    st = unscale_check_norm(plan, state, g, max_norm, stream, partials,
                            mpk::Tail{1, hp->beta1, hp->beta2});
    if (st == MP_OK) st = adamw_step(plan, state, g, hp, nullptr, stream, true, true);
    return st;
}

}  // namespace

mp_status mp_accumulate(mp_plan* plan, const mp_gradset* g16, float weight, int32_t first,
                        mp_stream stream)
{
    if (g16 == nullptr) return fail(MP_ERR_INVALID, "plan and gradset are required");
    return accumulate(plan, single(g16, host_weight(weight), 1), first, stream);
}

mp_status mp_accumulate_group(mp_plan* plan, const mp_gradset* const* sets, const float* weights,
                              int32_t n, int32_t weights_on_device, int32_t first,
                              mp_stream stream)
{
    Group g;
    mp_status st = make_group(sets, weights, n, weights_on_device, 1, &g);
    if (st != MP_OK) return st;
    return accumulate(plan, g, first, stream);
}

mp_status mp_accumulate_first_counts(mp_plan* plan, const mp_gradset* const* sets, int32_t n,
                                     int32_t k, const int64_t* counts, float* weights_out,
                                     mp_stream stream)
{
    if (sets == nullptr || counts == nullptr || weights_out == nullptr)
        return fail(MP_ERR_INVALID, "sets, counts and weights_out are required");
    if (n < 1 || n > mpk::kMaxGroup || k < n || k > mpk::kMaxCountsK)
        return fail(MP_ERR_INVALID, "need 1 <= n <= %d and n <= k <= %d", mpk::kMaxGroup,
                    mpk::kMaxCountsK);
    if ((reinterpret_cast<uintptr_t>(counts) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(weights_out) & 3u) != 0)
        return fail(MP_ERR_ALIGN, "counts must be 8-byte aligned, weights 4-byte aligned");
    Group g{};
    g.n = n;
    g.no_acc = 1;
    for (int i = 0; i < n; ++i) g.sets[i] = sets[i];
    g.counts = counts;
    g.weights_out = weights_out;
    g.k = k;
    return accumulate(plan, g, 1, stream);
}

mp_status mp_token_weights_dev(int32_t k, const int64_t* counts, float* weights_out,
                               mp_stream stream)
{
    if (k < 1 || counts == nullptr || weights_out == nullptr)
        return fail(MP_ERR_INVALID, "need k >= 1, device counts and a device output array");
    if ((reinterpret_cast<uintptr_t>(counts) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(weights_out) & 3u) != 0)
        return fail(MP_ERR_ALIGN, "counts must be 8-byte aligned, weights 4-byte aligned");
    hipError_t e = mpk::launch_token_weights(counts, k, weights_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "token weights launch");
    return ok();
}

mp_status mp_unscale_check_norm(mp_plan* plan, mp_state* state, const mp_gradset* last,
                                float w_last, int32_t last_is_first, float max_norm,
                                mp_stream stream)
{
    return unscale_check_norm(plan, state, single(last, host_weight(w_last), last_is_first),
                              max_norm, stream);
}

namespace {

mp_status norm_partial(mp_plan* plan, mp_state* state, const Group& g, double* partial_out,
                       mp_stream stream)
{
    if (plan == nullptr || state == nullptr) return fail(MP_ERR_INVALID, "plan and state are required");
    if (partial_out == nullptr || (reinterpret_cast<uintptr_t>(partial_out) & 7u) != 0)
        return fail(MP_ERR_INVALID, "partial_out must be an 8-byte aligned device pointer");
    mp_status st = check_group(plan, g);
    if (st == MP_OK) st = check_devices(plan, state);
    if (st != MP_OK) return st;
    hipError_t e = mpk::launch_norm_partial(view(plan), plan->norm_grid, device_group(g),
                                            plan->dtype, plan->d_partials, state->d, partial_out,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "norm partial launch");
    plan->partial_pending = true;
    plan->norm_pending = false;
    plan->norm_state = state;
    remember_norm_group(plan, g);
    return ok();
}

}  // namespace

mp_status mp_norm_partial(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                          int32_t last_is_first, double* partial_out, mp_stream stream)
{
    return norm_partial(plan, state, single(last, host_weight(w_last), last_is_first),
                        partial_out, stream);
}

mp_status mp_norm_partial_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                                const float* weights, int32_t n, int32_t weights_on_device,
                                int32_t last_is_first, double* partial_out, mp_stream stream)
{
    Group g;
    mp_status st = make_group(sets, weights, n, weights_on_device, last_is_first, &g);
    if (st != MP_OK) return st;
    return norm_partial(plan, state, g, partial_out, stream);
}

mp_status mp_norm_finish(mp_plan* plan, mp_state* state, const double* sumsq, float max_norm,
                         mp_stream stream)
{
    if (plan == nullptr || state == nullptr || sumsq == nullptr)
        return fail(MP_ERR_INVALID, "plan, state and sumsq are required");
    if ((reinterpret_cast<uintptr_t>(sumsq) & 7u) != 0)
        return fail(MP_ERR_INVALID, "sumsq must be 8-byte aligned");
    if (std::isnan(max_norm) || std::isinf(max_norm)) return fail(MP_ERR_INVALID, "max_norm must be finite");
    if (!plan->partial_pending || plan->norm_state != state)
        return fail(MP_ERR_ORDER, "mp_norm_finish must follow mp_norm_partial on the same plan "
                                  "and state");
    mp_status st = check_devices(plan, state);
    if (st != MP_OK) return st;
    hipError_t e = mpk::launch_norm_apply(sumsq, max_norm, state->d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "norm finish launch");
    state->decision_pending = true;
    plan->partial_pending = false;
    plan->norm_pending = true;
    return ok();
}

mp_status mp_adamw_step(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                        int32_t last_is_first, const mp_adamw_hparams* hp, mp_stream stream)
{
    return adamw_step(plan, state, single(last, host_weight(w_last), last_is_first), hp, nullptr,
                      stream);
}

mp_status mp_adamw_step_fp8(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                            int32_t last_is_first, const mp_adamw_hparams* hp,
                            const mp_fp8set* fp8, mp_stream stream)
{
    if (fp8 == nullptr) return fail(MP_ERR_INVALID, "fp8 set is NULL");
    if (fp8->plan != plan) return fail(MP_ERR_INVALID, "fp8 set belongs to another plan");
    return adamw_step(plan, state, single(last, host_weight(w_last), last_is_first), hp,
                      fp8->d_out, stream);
}

mp_status mp_update_step(mp_plan* plan, mp_state* state, const mp_gradset* last, float w_last,
                         int32_t last_is_first, float max_norm, const mp_adamw_hparams* hp,
                         mp_stream stream)
{
    return update_step(plan, state, single(last, host_weight(w_last), last_is_first), max_norm,
                       hp, stream);
}

mp_status mp_update_step_noalloc(mp_plan* plan, mp_state* state, const mp_gradset* last,
                                 float w_last, int32_t last_is_first, float max_norm,
                                 const mp_adamw_hparams* hp, mp_stream stream)
{
    return update_step(plan, state, single(last, host_weight(w_last), last_is_first), max_norm,
                       hp, stream, true);
}

mp_status mp_unscale_check_norm_group(mp_plan* plan, mp_state* state,
                                      const mp_gradset* const* sets, const float* weights,
                                      int32_t n, int32_t weights_on_device, int32_t last_is_first,
                                      float max_norm, mp_stream stream)
{
    Group g;
    mp_status st = make_group(sets, weights, n, weights_on_device, last_is_first, &g);
    if (st != MP_OK) return st;
    return unscale_check_norm(plan, state, g, max_norm, stream);
}

mp_status mp_adamw_step_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                              const float* weights, int32_t n, int32_t weights_on_device,
                              int32_t last_is_first, const mp_adamw_hparams* hp, mp_stream stream)
{
    Group g;
    mp_status st = make_group(sets, weights, n, weights_on_device, last_is_first, &g);
    if (st != MP_OK) return st;
    return adamw_step(plan, state, g, hp, nullptr, stream);
}

mp_status mp_update_step_group(mp_plan* plan, mp_state* state, const mp_gradset* const* sets,
                               const float* weights, int32_t n, int32_t weights_on_device,
                               int32_t last_is_first, float max_norm, const mp_adamw_hparams* hp,
                               mp_stream stream)
{
    Group g;
    mp_status st = make_group(sets, weights, n, weights_on_device, last_is_first, &g);
    if (st != MP_OK) return st;
    return update_step(plan, state, g, max_norm, hp, stream);
}

mp_status mp_scaler_update(mp_state* state, mp_stream stream)
{
    if (state == nullptr) return fail(MP_ERR_INVALID, "state is NULL");
    if (!state->decision_pending)
        return fail(MP_ERR_ORDER, "mp_scaler_update must follow mp_unscale_check_norm (or "
                                  "mp_norm_finish) on this state, once per measured step");
    mp_status st = check_devices(nullptr, state);
    if (st != MP_OK) return st;
    hipError_t e = mpk::launch_scaler(state->d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "scaler launch");
    state->decision_pending = false;
    return ok();
}

mp_status mp_cast_to_16(const float* src, uint16_t* dst, int64_t n, mp_dtype16 dtype,
                        mp_stream stream)
{
    if (n < 0 || !valid_dtype(dtype)) return fail(MP_ERR_INVALID, "n must be >= 0, dtype known");
    if (n > 0 && (src == nullptr || dst == nullptr)) return fail(MP_ERR_INVALID, "NULL buffer");
    if (!aligned16(src) || !aligned16(dst)) return fail(MP_ERR_ALIGN, "buffers must be 16-byte aligned");
    hipError_t e = mpk::launch_cast_to_16(src, dst, n, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cast launch");
    return ok();
}

mp_status mp_widen_16(const uint16_t* src, float* dst, int64_t n, mp_dtype16 dtype,
                      mp_stream stream)
{
    if (n < 0 || !valid_dtype(dtype)) return fail(MP_ERR_INVALID, "n must be >= 0, dtype known");
    if (n > 0 && (src == nullptr || dst == nullptr)) return fail(MP_ERR_INVALID, "NULL buffer");
    if (!aligned16(src) || !aligned16(dst)) return fail(MP_ERR_ALIGN, "buffers must be 16-byte aligned");
    hipError_t e = mpk::launch_widen_16(src, dst, n, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "widen launch");
    return ok();
}

mp_status mp_cast_fp8_blocks(const float* src, uint8_t* codes, float* scales, int64_t n,
                             int32_t block, mp_stream stream)
{
    if (block < 16 || block > 1024 || block % 16 != 0)
        return fail(MP_ERR_INVALID, "block must be a multiple of 16 in [16, 1024]");
    if (n < 0 || n % block != 0) return fail(MP_ERR_INVALID, "n must be a multiple of block");
    if (n > 0 && (src == nullptr || codes == nullptr || scales == nullptr))
        return fail(MP_ERR_INVALID, "NULL buffer");
    if (!aligned16(src) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return fail(MP_ERR_ALIGN, "src and codes must be 16-byte aligned, scales 4-byte aligned");
    hipError_t e = mpk::launch_fp8_blocks(src, codes, scales, n, block,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fp8 launch");
    return ok();
}

}  // extern "C"
