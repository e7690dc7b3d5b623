// The C ABI on its own: a host program that drives libzero_mi355x through
// include/zero_mi355x.h with hipMalloc'ed buffers (no Python, no torch) and
// checks every step against the CPU oracle (oracle/zero_oracle.c, linked
// as test infrastructure), bit for bit.
//
// Case: a ragged 9-tensor model, data-parallel degree 3, rank 1, align 8,
// fp16 gradients and parameters, dynamic loss scale from 1024 with a window
// of 2, AdamW, 8 steps, +inf injected into step 3's gradients.  Then the
// same with Adam-L2 and bf16, and with gradients kept in fp32 (fp16
// parameters, dynamic scale).  Inputs come from the seeded generator
// (synth/synth_host.c); the fp32 -> half rounding of the inputs uses the
// compiler's _Float16 / __bf16 conversions (IEEE round to nearest even).
//
// The fp16 and fp32-gradient cases run a second time with the gated update
// through zero_adam_step_noalloc (the flag read from the caller's device
// int), and the update scalars that zero_adam_scalars forms on the device
// are compared with the host's for t = 1..4096.  Then the ZeRO-Offload
// pipeline through its calls alone (offload_case).
//
// Prints "c-abi ok" and exits 0 on success; prints the first mismatch and
// exits 1 otherwise.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "zero_mi355x.h"

extern "C" {
// oracle/zero_oracle.c
int oracle_plan(const int64_t* numels, int64_t n, int64_t R, int64_t r, int64_t A, int64_t B,
                int64_t* scal, int64_t* seg_tensor, int64_t* seg_tensor_off, int64_t* seg_shard_off,
                int64_t* seg_numel, int64_t* tensor_bucket);
void oracle_flatten(const uint16_t* const* grads, const int64_t* seg_tensor,
                    const int64_t* seg_tensor_off, const int64_t* seg_shard_off,
                    const int64_t* seg_numel, int64_t nseg, int64_t S, int64_t real, uint16_t* flat);
void oracle_flatten_f32(const uint32_t* const* grads, const int64_t* seg_tensor,
                        const int64_t* seg_tensor_off, const int64_t* seg_shard_off,
                        const int64_t* seg_numel, int64_t nseg, int64_t S, int64_t real,
                        uint32_t* flat);
int oracle_adam_step(int64_t n, int64_t t, double scale, const void* flat, int gdt,
                     float* master, float* m, float* v, double lr, double b1, double b2,
                     double eps, double wd, int adamw);
void oracle_write_param(const float* master, int64_t real, int64_t begin, int64_t base,
                        uint16_t* param, int pdt);
void oracle_update_scale(double* scale, int32_t* good, int overflow, int dynamic,
                         double min_scale, double backoff, double growth, int32_t window);
// synth/synth_host.c
uint64_t synth_key(uint64_t seed, uint32_t stream, uint32_t iter);
void synth_fill_f32(float* out, int64_t n, uint64_t key, int64_t index0, float sigma, float scale,
                    uint32_t outlier_thresh, float outlier_mult);
}

namespace {

#define HIP_OK(x)                                                                \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                            \
        }                                                                        \
    } while (0)

#define ZERO_OK_OR_FAIL(x)                                                       \
    do {                                                                         \
        int rc_ = (x);                                                           \
        if (rc_ < 0) {                                                           \
            std::printf("%s failed: %d (%s)\n", #x, rc_, zero_last_error());      \
            return 1;                                                            \
        }                                                                        \
    } while (0)

uint16_t to_half(float x, int dt) {
    uint16_t h;
    if (dt == ZERO_F16) {
        _Float16 y = static_cast<_Float16>(x);
        std::memcpy(&h, &y, 2);
    } else {
        __bf16 y = static_cast<__bf16>(x);
        std::memcpy(&h, &y, 2);
    }
    return h;
}

// The bits of one gradient element of dtype dt (fp32: the value as it is).
uint32_t grad_word(float x, int dt) {
    if (dt == ZERO_F32) {
        uint32_t u;
        std::memcpy(&u, &x, 4);
        return u;
    }
    return to_half(x, dt);
}

// noalloc = 1: the step goes through zero_adam_step_noalloc instead of
// zero_adam_step.
int run_case(int gdt, int pdt, int adamw, int noalloc) {
    const size_t esize = gdt == ZERO_F32 ? 4 : 2;
    const std::vector<int64_t> numels = {3000, 1, 7, 100003, 65, 2048, 511, 30000, 13};
    const int R = 3, r = 1, A = 8, steps = 8, inject_step = 3;
    const int64_t B = 20000;
    const int n = static_cast<int>(numels.size());
    int64_t P = 0;
    std::vector<int64_t> off(n + 1, 0);
    for (int i = 0; i < n; ++i) off[i + 1] = off[i] + numels[i];
    P = off[n];

    // plans: library and oracle
    zero_plan_t* plan = nullptr;
    ZERO_OK_OR_FAIL(zero_partition_plan(numels.data(), n, R, r, A, B, &plan));
    zero_plan_info_t info;
    ZERO_OK_OR_FAIL(zero_plan_info(plan, &info));
    int64_t scal[10];
    std::vector<int64_t> st(n), sto(n), sso(n), sn(n), tb(n);
    if (oracle_plan(numels.data(), n, R, r, A, B, scal, st.data(), sto.data(), sso.data(),
                    sn.data(), tb.data()) != 0) {
        std::printf("oracle_plan failed\n");
        return 1;
    }
    const int64_t S = scal[2], begin = scal[3], real = scal[4], nseg = scal[5];
    if (info.shard_numel != S || info.shard_begin != begin || info.real_numel != real ||
        info.n_segments != nseg) {
        std::printf("plan mismatch\n");
        return 1;
    }

    // device buffers
    std::vector<void*> d_grads(n, nullptr);
    for (int i = 0; i < n; ++i) HIP_OK(hipMalloc(&d_grads[i], esize * numels[i]));
    void *d_flat, *d_param;
    float *d_master, *d_m, *d_v;
    int32_t* d_flag = nullptr;
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_flag), sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_flat, esize * S));
    HIP_OK(hipMalloc(&d_param, 2 * P));
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_master), 4 * S));
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_m), 4 * S));
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_v), 4 * S));

    // initial state: master ~ N(0, 0.02) on the real part, moments zero,
    // parameters filled with a pattern no finite master casts to
    std::vector<float> o_master(S, 0.0f), o_m(S, 0.0f), o_v(S, 0.0f);
    synth_fill_f32(o_master.data(), real, synth_key(0, 2, 0), begin, 0.02f, 1.0f, 0, 1.0f);
    std::vector<uint16_t> o_param(P, 0xFFFF);
    HIP_OK(hipMemcpy(d_master, o_master.data(), 4 * S, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_m, 0, 4 * S));
    HIP_OK(hipMemset(d_v, 0, 4 * S));
    HIP_OK(hipMemcpy(d_param, o_param.data(), 2 * P, hipMemcpyHostToDevice));

    zero_adam_hparams_t hp = {1e-3, 0.9, 0.999, 1e-8, 0.05, adamw, 0};
    const int dynamic = gdt != ZERO_BF16;
    zero_scaler_t scaler = {dynamic ? 1024.0 : 1.0, 1.0, 0.5, 2.0, 2, 0, dynamic, 0};
    double o_scale = scaler.scale;
    int32_t o_good = 0;
    int64_t t = 0, o_t = 0;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    std::vector<std::vector<uint32_t>> grads(n);      // element bits (fp16/bf16 in the low half)
    std::vector<std::vector<unsigned char>> gbytes(n);  // the same, packed at esize bytes each
    std::vector<const void*> gptr(n);
    std::vector<unsigned char> o_flat(esize * S), g_flat(esize * S);
    std::vector<uint16_t> g_param(P);
    std::vector<float> g_master(S), g_m(S), g_v(S), vals;
    for (int it = 1; it <= steps; ++it) {
        // this step's gradients, scaled by the current loss scale
        for (int i = 0; i < n; ++i) {
            vals.assign(numels[i], 0.0f);
            synth_fill_f32(vals.data(), numels[i], synth_key(0, 1, it), off[i], 1e-2f,
                           static_cast<float>(o_scale), 0, 1.0f);
            grads[i].resize(numels[i]);
            for (int64_t k = 0; k < numels[i]; ++k) grads[i][k] = grad_word(vals[k], gdt);
        }
        if (it == inject_step) {  // +inf in the middle of the shard's first segment
            grads[st[0]][sto[0] + sn[0] / 2] =
                gdt == ZERO_F32 ? 0x7F800000u : gdt == ZERO_F16 ? 0x7C00u : 0x7F80u;
        }
        for (int i = 0; i < n; ++i) {
            gbytes[i].resize(esize * numels[i]);
            for (int64_t k = 0; k < numels[i]; ++k) {
                if (esize == 4) {
                    std::memcpy(&gbytes[i][4 * k], &grads[i][k], 4);
                } else {
                    const uint16_t h = static_cast<uint16_t>(grads[i][k]);
                    std::memcpy(&gbytes[i][2 * k], &h, 2);
                }
            }
            gptr[i] = gbytes[i].data();
            HIP_OK(hipMemcpy(d_grads[i], gbytes[i].data(), esize * numels[i],
                             hipMemcpyHostToDevice));
        }
        // library: flatten all buckets, gated step, scaler
        std::vector<const void*> dg(d_grads.begin(), d_grads.end());
        ZERO_OK_OR_FAIL(zero_flatten_grads(plan, -1, dg.data(), gdt, d_flat, s));
        const double scale_used = scaler.scale;
        int flag = 0;
        if (noalloc) {
            ZERO_OK_OR_FAIL(zero_adam_step_noalloc(plan, &hp, t + 1, scale_used, d_flat, gdt,
                                                   d_master, d_m, d_v, d_param, 0, P, pdt,
                                                   d_flag, s));
            int32_t h_flag = -1;
            HIP_OK(hipStreamSynchronize(s));
            HIP_OK(hipMemcpy(&h_flag, d_flag, sizeof(h_flag), hipMemcpyDeviceToHost));
            flag = h_flag;
        } else {
            flag = zero_adam_step(plan, &hp, t + 1, scale_used, d_flat, gdt, d_master, d_m, d_v,
                                  d_param, 0, P, pdt, s);
        }
        ZERO_OK_OR_FAIL(flag);
        ZERO_OK_OR_FAIL(zero_update_loss_scale(&scaler, flag));
        if (!flag) ++t;
        // oracle
        if (esize == 4) {
            oracle_flatten_f32(reinterpret_cast<const uint32_t* const*>(gptr.data()), st.data(),
                               sto.data(), sso.data(), sn.data(), nseg, S, real,
                               reinterpret_cast<uint32_t*>(o_flat.data()));
        } else {
            oracle_flatten(reinterpret_cast<const uint16_t* const*>(gptr.data()), st.data(),
                           sto.data(), sso.data(), sn.data(), nseg, S, real,
                           reinterpret_cast<uint16_t*>(o_flat.data()));
        }
        const int o_flag = oracle_adam_step(S, o_t + 1, o_scale, o_flat.data(), gdt,
                                            o_master.data(), o_m.data(), o_v.data(), hp.lr,
                                            hp.beta1, hp.beta2, hp.eps, hp.weight_decay, adamw);
        if (!o_flag) {
            ++o_t;
            oracle_write_param(o_master.data(), real, begin, 0, o_param.data(), pdt);
        }
        oracle_update_scale(&o_scale, &o_good, o_flag, dynamic, 1.0, 0.5, 2.0, 2);
        // compare
        if (flag != o_flag || t != o_t || scaler.scale != o_scale || scaler.good_steps != o_good) {
            std::printf("step %d: flag %d/%d t %lld/%lld scale %g/%g\n", it, flag, o_flag,
                        static_cast<long long>(t), static_cast<long long>(o_t), scaler.scale,
                        o_scale);
            return 1;
        }
        HIP_OK(hipMemcpy(g_flat.data(), d_flat, esize * S, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_master.data(), d_master, 4 * S, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_m.data(), d_m, 4 * S, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_v.data(), d_v, 4 * S, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_param.data(), d_param, 2 * P, hipMemcpyDeviceToHost));
        if (std::memcmp(g_flat.data(), o_flat.data(), esize * S) != 0 ||
            std::memcmp(g_master.data(), o_master.data(), 4 * S) != 0 ||
            std::memcmp(g_m.data(), o_m.data(), 4 * S) != 0 ||
            std::memcmp(g_v.data(), o_v.data(), 4 * S) != 0 ||
            std::memcmp(g_param.data(), o_param.data(), 2 * P) != 0) {
            std::printf("step %d: state differs from the oracle\n", it);
            return 1;
        }
    }
    // window 2, overflow at step 3: x2 after step 2, /2 at step 3, x2 after
    // steps 5 and 7 -> 4096
    if (dynamic && o_scale != 4096.0) {
        std::printf("unexpected scale trajectory: %g\n", o_scale);
        return 1;
    }
    for (void* p : d_grads) HIP_OK(hipFree(p));
    HIP_OK(hipFree(d_flag));
    HIP_OK(hipFree(d_flat));
    HIP_OK(hipFree(d_param));
    HIP_OK(hipFree(d_master));
    HIP_OK(hipFree(d_m));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipStreamDestroy(s));
    zero_plan_destroy(plan);
    std::printf("case gdt=%d pdt=%d adamw=%d%s: %d steps, %lld applied, scale %g\n", gdt, pdt,
                adamw, noalloc ? " (allocation-free step)" : "", steps,
                static_cast<long long>(t), scaler.scale);
    return 0;
}

// ZeRO-Offload through the C ABI: host-resident master / moments, the
// pipeline at lag 1 (one-step delayed update) or lag 0, an overflow at step
// 3.  Each iteration a stand-in forward copies the device parameters after
// zero_offload_wait_params; they must be the oracle's after iteration
// it - 1 - lag.  After the drain the host state and the device parameters
// must equal the oracle's, and the timeline must hold every piece's copies
// and host update in the pipeline's order.
int offload_case(int gdt, int pdt, int lag) {
    const size_t esize = gdt == ZERO_F32 ? 4 : 2;
    const std::vector<int64_t> numels = {3000, 1, 7, 100003, 65, 2048, 511, 30000, 13};
    const int R = 3, r = 1, A = 8, steps = 7, inject_step = 3;
    const int64_t B = 20000;
    const int n = static_cast<int>(numels.size());
    std::vector<int64_t> off(n + 1, 0);
    for (int i = 0; i < n; ++i) off[i + 1] = off[i] + numels[i];
    const int64_t P = off[n];
    zero_plan_t* plan = nullptr;
    ZERO_OK_OR_FAIL(zero_partition_plan(numels.data(), n, R, r, A, B, &plan));
    int64_t scal[10];
    std::vector<int64_t> st(n), sto(n), sso(n), sn(n), tb(n);
    if (oracle_plan(numels.data(), n, R, r, A, B, scal, st.data(), sto.data(), sso.data(),
                    sn.data(), tb.data()) != 0) {
        std::printf("oracle_plan failed\n");
        return 1;
    }
    const int64_t S = scal[2], begin = scal[3], real = scal[4], nseg = scal[5];

    std::vector<void*> d_grads(n, nullptr);
    for (int i = 0; i < n; ++i) HIP_OK(hipMalloc(&d_grads[i], esize * numels[i]));
    void *d_flat, *d_param;
    HIP_OK(hipMalloc(&d_flat, esize * S));
    HIP_OK(hipMalloc(&d_param, 2 * P));
    std::vector<float> o_master(S, 0.0f), o_m(S, 0.0f), o_v(S, 0.0f);
    synth_fill_f32(o_master.data(), real, synth_key(0, 2, 0), begin, 0.02f, 1.0f, 0, 1.0f);
    std::vector<float> h_master(o_master), h_m(S, 0.0f), h_v(S, 0.0f);  // the pipeline's state
    std::vector<uint16_t> o_param(P, 0xFFFF);
    HIP_OK(hipMemcpy(d_param, o_param.data(), 2 * P, hipMemcpyHostToDevice));
    std::vector<std::vector<uint16_t>> hist = {o_param};  // oracle parameters after iteration k

    const zero_adam_hparams_t hp = {1e-3, 0.9, 0.999, 1e-8, 0.05, 1, 0};
    const int dynamic = gdt != ZERO_BF16;
    zero_scaler_t scaler = {dynamic ? 1024.0 : 1.0, 1.0, 0.5, 2.0, 2, 0, dynamic, 0};
    double o_scale = scaler.scale;
    int32_t o_good = 0;
    int64_t o_t = 0;
    int skipped = 0;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    ZERO_OK_OR_FAIL(zero_state_upload(plan, 0, &scaler, s));
    zero_offload_t* offl = nullptr;
    ZERO_OK_OR_FAIL(zero_offload_create(plan, &hp, gdt, pdt, h_master.data(), h_m.data(),
                                        h_v.data(), 3, &offl));
    ZERO_OK_OR_FAIL(zero_offload_timeline_start(offl, 4096));

    std::vector<std::vector<unsigned char>> gbytes(n);
    std::vector<const void*> gptr(n);
    std::vector<unsigned char> o_flat(esize * S);
    std::vector<uint16_t> seen(P);
    std::vector<float> vals;
    for (int it = 1; it <= steps; ++it) {
        ZERO_OK_OR_FAIL(zero_offload_wait_params(offl, lag, s));
        HIP_OK(hipMemcpyAsync(seen.data(), d_param, 2 * P, hipMemcpyDeviceToHost, s));
        HIP_OK(hipStreamSynchronize(s));
        const std::vector<uint16_t>& want = hist[it - 1 - lag > 0 ? it - 1 - lag : 0];
        if (std::memcmp(seen.data(), want.data(), 2 * P) != 0) {
            std::printf("offload lag %d it %d: the forward saw other parameters\n", lag, it);
            return 1;
        }
        double dev_scale = 0;
        zero_scaler_t dsc;
        ZERO_OK_OR_FAIL(zero_state_download(plan, nullptr, &dsc, nullptr, nullptr, s));
        dev_scale = dsc.scale;
        if (dev_scale != o_scale) {
            std::printf("offload lag %d it %d: device scale %g, oracle %g\n", lag, it, dev_scale,
                        o_scale);
            return 1;
        }
        for (int i = 0; i < n; ++i) {
            vals.assign(numels[i], 0.0f);
            synth_fill_f32(vals.data(), numels[i], synth_key(0, 1, it), off[i], 1e-2f,
                           static_cast<float>(o_scale), 0, 1.0f);
            gbytes[i].resize(esize * numels[i]);
            for (int64_t k = 0; k < numels[i]; ++k) {
                uint32_t w = grad_word(vals[k], gdt);
                if (it == inject_step && i == st[0] && k == sto[0] + sn[0] / 2) {
                    w = gdt == ZERO_F32 ? 0x7F800000u : gdt == ZERO_F16 ? 0x7C00u : 0x7F80u;
                }
                std::memcpy(&gbytes[i][esize * k], &w, esize);  // little endian: low half first
            }
            gptr[i] = gbytes[i].data();
            HIP_OK(hipMemcpyAsync(d_grads[i], gbytes[i].data(), esize * numels[i],
                                  hipMemcpyHostToDevice, s));
        }
        std::vector<const void*> dg(d_grads.begin(), d_grads.end());
        ZERO_OK_OR_FAIL(zero_flatten_grads(plan, -1, dg.data(), gdt, d_flat, s));
        ZERO_OK_OR_FAIL(zero_offload_submit(offl, d_flat, d_param, 0, P, s));
        HIP_OK(hipStreamSynchronize(s));  // the host gradient copies are read below
        // oracle
        if (esize == 4) {
            oracle_flatten_f32(reinterpret_cast<const uint32_t* const*>(gptr.data()), st.data(),
                               sto.data(), sso.data(), sn.data(), nseg, S, real,
                               reinterpret_cast<uint32_t*>(o_flat.data()));
        } else {
            oracle_flatten(reinterpret_cast<const uint16_t* const*>(gptr.data()), st.data(),
                           sto.data(), sso.data(), sn.data(), nseg, S, real,
                           reinterpret_cast<uint16_t*>(o_flat.data()));
        }
        const int o_flag = oracle_adam_step(S, o_t + 1, o_scale, o_flat.data(), gdt,
                                            o_master.data(), o_m.data(), o_v.data(), hp.lr,
                                            hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1);
        if (!o_flag) {
            ++o_t;
            oracle_write_param(o_master.data(), real, begin, 0, o_param.data(), pdt);
        } else {
            ++skipped;
        }
        oracle_update_scale(&o_scale, &o_good, o_flag, dynamic, 1.0, 0.5, 2.0, 2);
        hist.push_back(o_param);
    }
    ZERO_OK_OR_FAIL(zero_offload_drain(offl, s));
    zero_offload_stats_t stats;
    ZERO_OK_OR_FAIL(zero_offload_stats(offl, &stats));
    if (stats.applied != o_t || stats.skipped != skipped || stats.processed != steps) {
        std::printf("offload lag %d: stats applied %lld skipped %lld\n", lag,
                    static_cast<long long>(stats.applied), static_cast<long long>(stats.skipped));
        return 1;
    }
    if (std::memcmp(h_master.data(), o_master.data(), 4 * S) != 0 ||
        std::memcmp(h_m.data(), o_m.data(), 4 * S) != 0 ||
        std::memcmp(h_v.data(), o_v.data(), 4 * S) != 0) {
        std::printf("offload lag %d: host state differs from the oracle\n", lag);
        return 1;
    }
    HIP_OK(hipMemcpy(seen.data(), d_param, 2 * P, hipMemcpyDeviceToHost));
    if (std::memcmp(seen.data(), o_param.data(), 2 * P) != 0) {
        std::printf("offload lag %d: final parameters differ\n", lag);
        return 1;
    }
    // the timeline: per step, every gradient piece; per applied step, each
    // piece's update after its gradient copy and its parameter copy after it
    const int64_t n_iv = zero_offload_timeline(offl, nullptr, 0);
    ZERO_OK_OR_FAIL(static_cast<int>(n_iv < 0 ? n_iv : 0));
    std::vector<zero_offload_interval_t> iv(n_iv > 0 ? n_iv : 1);
    const int64_t got = zero_offload_timeline(offl, iv.data(), n_iv);
    if (got != n_iv || n_iv < 3 * (steps - skipped)) {
        std::printf("offload lag %d: %lld timeline intervals\n", lag, static_cast<long long>(n_iv));
        return 1;
    }
    for (int64_t a = 0; a < n_iv; ++a) {
        if (iv[a].end_ms < iv[a].start_ms - 0.05) {
            std::printf("offload lag %d: an interval ends before it starts\n", lag);
            return 1;
        }
        for (int64_t b = 0; b < n_iv; ++b) {
            if (iv[b].step != iv[a].step || iv[b].piece != iv[a].piece) continue;
            if (iv[a].kind == 1 && iv[b].kind == 0 && iv[a].start_ms < iv[b].end_ms - 0.05) {
                std::printf("offload lag %d: an update started before its gradient arrived\n", lag);
                return 1;
            }
            if (iv[a].kind == 2 && iv[b].kind == 1 && iv[a].start_ms < iv[b].end_ms - 0.05) {
                std::printf("offload lag %d: parameters went back before their update\n", lag);
                return 1;
            }
        }
    }
    zero_offload_destroy(offl);
    for (void* p : d_grads) HIP_OK(hipFree(p));
    HIP_OK(hipFree(d_flat));
    HIP_OK(hipFree(d_param));
    HIP_OK(hipStreamDestroy(s));
    zero_plan_destroy(plan);
    std::printf("offload gdt=%d pdt=%d lag %d: %d steps, %lld applied, %lld timeline intervals\n",
                gdt, pdt, lag, steps, static_cast<long long>(o_t), static_cast<long long>(n_iv));
    return 0;
}

// zero_adam_scalars: the device's scalars equal the host's, bit for bit.
int scalars_case() {
    const int64_t n = 4096;
    const zero_adam_hparams_t hp = {3e-4, 0.95, 0.98, 1e-6, 0.1, 1, 0};
    std::vector<float> host(10 * n), dev(10 * n);
    ZERO_OK_OR_FAIL(zero_adam_scalars(&hp, 1, n, 65536.0, host.data(), 0, nullptr));
    float* d_out = nullptr;
    HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_out), sizeof(float) * 10 * n));
    ZERO_OK_OR_FAIL(zero_adam_scalars(&hp, 1, n, 65536.0, d_out, 1, nullptr));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(dev.data(), d_out, sizeof(float) * 10 * n, hipMemcpyDeviceToHost));
    HIP_OK(hipFree(d_out));
    if (std::memcmp(host.data(), dev.data(), sizeof(float) * 10 * n) != 0) {
        std::printf("device and host update scalars differ\n");
        return 1;
    }
    std::printf("update scalars: device = host for t = 1..%lld\n", static_cast<long long>(n));
    return 0;
}

}  // namespace

int main() {
    if (run_case(ZERO_F16, ZERO_F16, 1, 0) != 0) return 1;
    if (run_case(ZERO_BF16, ZERO_BF16, 0, 0) != 0) return 1;
    if (run_case(ZERO_F32, ZERO_F16, 1, 0) != 0) return 1;
    if (run_case(ZERO_F16, ZERO_F16, 1, 1) != 0) return 1;
    if (run_case(ZERO_F32, ZERO_F16, 1, 1) != 0) return 1;
    if (scalars_case() != 0) return 1;
    if (offload_case(ZERO_F16, ZERO_F16, 1) != 0) return 1;
    if (offload_case(ZERO_BF16, ZERO_BF16, 0) != 0) return 1;
    if (offload_case(ZERO_F32, ZERO_F16, 1) != 0) return 1;
    std::printf("c-abi ok\n");
    return 0;
}
