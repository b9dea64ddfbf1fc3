// Two logical updates through the C ABI of include/mpstep.h, with plain HIP
// allocations and no framework.  Step 1: two micro-batches (the first
// accumulated, the last folded in), then unscale/norm, AdamW and the scaler in
// one call.  Step 2: token weights computed on the device from device counts,
// and both micro-batches folded into the norm and AdamW passes as one resident
// group.  The inputs are chosen so that the results have closed forms, which
// the program checks; it prints one line and exits 0 on success.
//
// Gradients are 2^-10 everywhere in both micro-batches, so with token counts
// 3 and 1 the weighted sum 0.75 * 2^-10 + 0.25 * 2^-10 is exactly 2^-10, the
// sum of squares over P elements is exactly P * 2^-20, and the first AdamW
// step from m = v = 0 moves every weight by lr * g / (|g| + eps) ("Your
// weights fit on one device...", the Adam update; bias corrections make the
// first step's moment ratio exactly g / |g| up to rounding).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mpstep.h"

#define HIP_OK(call)                                                                 \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            std::fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));          \
            return 2;                                                                \
        }                                                                            \
    } while (0)

#define MP_OK_(call)                                                                 \
    do {                                                                             \
        mp_status s_ = (call);                                                       \
        if (s_ != MP_OK) {                                                           \
            std::fprintf(stderr, "%s: %s: %s\n", #call, mp_status_string(s_),        \
                         mp_last_error());                                           \
            return 2;                                                                \
        }                                                                            \
    } while (0)

int main()
{
    const int32_t n = 3;
    const int64_t numel[n] = {1000, 4096, 7};
    const int64_t total = numel[0] + numel[1] + numel[2];
    const float master0 = 0.5f;
    const uint16_t grad_bits = 0x3A80;            // bf16 2^-10

    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    // caller-owned device buffers, one allocation per tensor and kind
    std::vector<void*> acc(n), master(n), m(n), v(n), w16(n), g1(n), g2(n);
    for (int i = 0; i < n; ++i) {
        const size_t f = numel[i] * sizeof(float), h = numel[i] * sizeof(uint16_t);
        HIP_OK(hipMalloc(&acc[i], f));
        HIP_OK(hipMalloc(&master[i], f));
        HIP_OK(hipMalloc(&m[i], f));
        HIP_OK(hipMalloc(&v[i], f));
        HIP_OK(hipMalloc(&w16[i], h));
        HIP_OK(hipMalloc(&g1[i], h));
        HIP_OK(hipMalloc(&g2[i], h));
        std::vector<float> w(numel[i], master0);
        std::vector<uint16_t> g(numel[i], grad_bits);
        HIP_OK(hipMemcpy(master[i], w.data(), f, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(m[i], 0, f));
        HIP_OK(hipMemset(v[i], 0, f));
        HIP_OK(hipMemcpy(g1[i], g.data(), h, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(g2[i], g.data(), h, hipMemcpyHostToDevice));
    }

    mp_plan* plan = nullptr;
    MP_OK_(mp_plan_create(n, numel, MP_BF16, acc.data(), master.data(), m.data(), v.data(),
                          w16.data(), nullptr, &plan));
    mp_gradset* set1 = nullptr;
    mp_gradset* set2 = nullptr;
    MP_OK_(mp_gradset_create(plan, g1.data(), &set1));
    MP_OK_(mp_gradset_create(plan, g2.data(), &set2));
    const mp_scaler_cfg cfg = {1.0f, 2.0f, 0.5f, 1.0f, 1.0f, 1, 0};   // bf16: no dynamic scale
    mp_state* state = nullptr;
    MP_OK_(mp_state_create(&cfg, &state));

    const int64_t counts[2] = {3, 1};
    float weights[2];
    MP_OK_(mp_token_weights(2, counts, weights));
    const mp_adamw_hparams hp = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.0f};

    MP_OK_(mp_accumulate(plan, set1, weights[0], 1, stream));
    MP_OK_(mp_update_step(plan, state, set2, weights[1], 0, 0.0f, &hp, stream));

    mp_stats stats;
    MP_OK_(mp_state_read(state, &stats, stream));
    HIP_OK(hipStreamSynchronize(stream));

    const double g = std::ldexp(1.0, -10);
    const double want_sumsq = static_cast<double>(total) * g * g;
    const double want_w = master0 - 1e-3 * (g / (g + 1e-8));
    int bad = 0;
    if (stats.found_inf != 0 || stats.step != 1 || stats.scale != 1.0f) ++bad;
    if (stats.sumsq != want_sumsq) ++bad;
    double worst = 0.0;
    for (int i = 0; i < n; ++i) {
        std::vector<float> w(numel[i]);
        std::vector<uint16_t> h(numel[i]);
        HIP_OK(hipMemcpy(w.data(), master[i], numel[i] * sizeof(float), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(h.data(), w16[i], numel[i] * sizeof(uint16_t), hipMemcpyDeviceToHost));
        for (int64_t j = 0; j < numel[i]; ++j) {
            const double err = std::fabs(static_cast<double>(w[j]) - want_w);
            worst = err > worst ? err : worst;
            uint32_t wide = static_cast<uint32_t>(h[j]) << 16;
            float back;
            std::memcpy(&back, &wide, sizeof back);
            // the 16-bit weight is the master rounded to bf16: within half a bf16 step
            if (std::fabs(back - w[j]) > std::ldexp(1.0, -10)) ++bad;
        }
    }
    if (worst > 4 * std::ldexp(1.0, -25)) ++bad;        // a few fp32 ulps of 0.5

    // Step 2, all on the device: target counts in device memory, token weights computed there,
    // and both micro-batches, still resident, folded straight into the norm and AdamW passes
    // (no accumulator pass).  The weights 1/4 and 3/4 of equal gradients sum to g exactly, so
    // the sum of squares repeats, and with m, v bias-corrected the second step moves each
    // weight by lr * g / (g + eps) again.
    const int64_t counts2[2] = {1, 3};
    int64_t* d_counts = nullptr;
    float* d_weights = nullptr;
    HIP_OK(hipMalloc(&d_counts, sizeof counts2));
    HIP_OK(hipMalloc(&d_weights, 2 * sizeof(float)));
    HIP_OK(hipMemcpy(d_counts, counts2, sizeof counts2, hipMemcpyHostToDevice));
    const mp_gradset* both[2] = {set1, set2};
    MP_OK_(mp_token_weights_dev(2, d_counts, d_weights, stream));
    MP_OK_(mp_update_step_group(plan, state, both, d_weights, 2, 1, 1, 0.0f, &hp, stream));
    mp_stats stats2;
    MP_OK_(mp_state_read(state, &stats2, stream));
    HIP_OK(hipStreamSynchronize(stream));
    if (stats2.found_inf != 0 || stats2.step != 2 || stats2.sumsq != want_sumsq) ++bad;
    const double want_w2 = master0 - 2e-3 * (g / (g + 1e-8));
    double worst2 = 0.0;
    for (int i = 0; i < n; ++i) {
        std::vector<float> w(numel[i]);
        HIP_OK(hipMemcpy(w.data(), master[i], numel[i] * sizeof(float), hipMemcpyDeviceToHost));
        for (int64_t j = 0; j < numel[i]; ++j) {
            const double err = std::fabs(static_cast<double>(w[j]) - want_w2);
            worst2 = err > worst2 ? err : worst2;
        }
    }
    if (worst2 > 8 * std::ldexp(1.0, -25)) ++bad;

    // Step 3, one micro-batch at a time with the counts still on the device: the first
    // accumulation computes the token weights itself and leaves both in d_weights, where the
    // folded last micro-batch reads its own (1/4 and 3/4 again: the same sum of squares and
    // another lr * g / (g + eps) per weight).
    HIP_OK(hipMemset(d_weights, 0, 2 * sizeof(float)));
    MP_OK_(mp_accumulate_first_counts(plan, both, 1, 2, d_counts, d_weights, stream));
    MP_OK_(mp_update_step_group(plan, state, both + 1, d_weights + 1, 1, 1, 0, 0.0f, &hp,
                                stream));
    mp_stats stats3;
    MP_OK_(mp_state_read(state, &stats3, stream));
    float w3[2];
    HIP_OK(hipMemcpyAsync(w3, d_weights, sizeof w3, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    if (stats3.found_inf != 0 || stats3.step != 3 || stats3.sumsq != want_sumsq) ++bad;
    if (w3[0] != 0.25f || w3[1] != 0.75f) ++bad;
    const double want_w3 = master0 - 3e-3 * (g / (g + 1e-8));
    double worst3 = 0.0;
    for (int i = 0; i < n; ++i) {
        std::vector<float> w(numel[i]);
        HIP_OK(hipMemcpy(w.data(), master[i], numel[i] * sizeof(float), hipMemcpyDeviceToHost));
        for (int64_t j = 0; j < numel[i]; ++j) {
            const double err = std::fabs(static_cast<double>(w[j]) - want_w3);
            worst3 = err > worst3 ? err : worst3;
        }
    }
    if (worst3 > 12 * std::ldexp(1.0, -25)) ++bad;
    (void)hipFree(d_counts);
    (void)hipFree(d_weights);

    mp_gradset_destroy(set1);
    mp_gradset_destroy(set2);
    mp_state_destroy(state);
    mp_plan_destroy(plan);
    for (int i = 0; i < n; ++i) {
        for (void* p : {acc[i], master[i], m[i], v[i], w16[i], g1[i], g2[i]}) (void)hipFree(p);
    }
    (void)hipStreamDestroy(stream);

    std::printf("c_api_step: %s  params %lld  sumsq %.17g (want %.17g)  norm %.9g  "
                "max |w - closed form| %.3g after step 1, %.3g after step 2, %.3g after step 3\n",
                bad ? "MISMATCH" : "ok", static_cast<long long>(total), stats.sumsq, want_sumsq,
                static_cast<double>(stats.grad_norm), worst, worst2, worst3);
    return bad ? 1 : 0;
}
