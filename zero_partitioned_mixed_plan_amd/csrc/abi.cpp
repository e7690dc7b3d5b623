// C-ABI entry points of libzero_mi355x: argument checks, host scalars,
// device state of a plan, and kernel launches on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include <unistd.h>

#include "internal.h"

namespace zmi {

namespace {
// The calling thread's last error message, in a fixed buffer: setting it
// never allocates (the allocation-free step reports errors through it too).
thread_local char g_last_error[512];
}

void set_error(const char* msg) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
}

void set_error(const std::string& msg) { set_error(msg.c_str()); }

int fail(int code, const char* msg) {
    set_error(msg);
    return code;
}

int fail(int code, const std::string& msg) { return fail(code, msg.c_str()); }

int hip_fail(hipError_t e, const char* what) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", what, hipGetErrorName(e),
                  hipGetErrorString(e));
    return ZERO_EHIP;
}

int check_hparams(const zero_adam_hparams_t* hp) {
    if (!(hp->lr >= 0 && std::isfinite(hp->lr)) || !(hp->beta1 >= 0 && hp->beta1 < 1) ||
        !(hp->beta2 >= 0 && hp->beta2 < 1) || !(hp->eps > 0 && std::isfinite(hp->eps)) ||
        !(hp->weight_decay >= 0 && std::isfinite(hp->weight_decay))) {
        return fail(ZERO_EINVAL, "hyperparameters out of range (lr >= 0, 0 <= betas < 1, eps > 0, "
                                 "weight_decay >= 0)");
    }
    return ZERO_OK;
}

// Whether every real gradient of flat_grad went through the flatten (and so
// through its overflow test) since the last step; if not, the step scans.
bool flatten_covered(const zero_plan* p, const void* flat_grad, int32_t grad_dtype) {
    bool covered = p->flattened_into == flat_grad && p->flattened_dtype == grad_dtype;
    if (covered && !p->flatten_all_done) {
        for (int32_t b = 0; b < p->n_buckets && covered; ++b) {
            if (p->bucket_seg_last[b] > p->bucket_seg_first[b] && !p->bucket_flattened[b]) {
                covered = false;
            }
        }
    }
    return covered;
}

// The overflow decision for a step on flat_grad.  When the flattens since
// the last step covered flat_grad, their fused test already raised the flag.
// Otherwise the flag is cleared (it may hold what a flatten into another
// buffer found) and the real elements [0, real) are scanned; the padding
// [real, S) only feeds padding state, which never reaches a parameter.
int gate_flag(zero_plan* p, const void* flat_grad, int32_t grad_dtype, hipStream_t s,
              bool* scanned) {
    *scanned = false;
    if (flatten_covered(p, flat_grad, grad_dtype)) return ZERO_OK;
    hipError_t e = launch_flag_clear(p->dev.d_flag, s);
    if (e != hipSuccess) return hip_fail(e, "flag clear");
    e = launch_scan(flat_grad, p->real, p->dev.d_flag, grad_dtype, s);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    *scanned = true;
    return ZERO_OK;
}

void reset_flatten_bookkeeping(zero_plan* p) {
    std::fill(p->bucket_flattened.begin(), p->bucket_flattened.end(), 0);
    p->flatten_all_done = false;
    p->flattened_into = nullptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool valid_dtype(int32_t d) { return d == ZERO_F16 || d == ZERO_BF16; }

bool valid_grad_dtype(int32_t d) { return valid_dtype(d) || d == ZERO_F32; }

int bad_grad_dtype() {
    return fail(ZERO_EINVAL, "grad_dtype must be ZERO_F16, ZERO_BF16 or ZERO_F32");
}

// Parameter destination of shard element 0, after checking that the
// caller's window [base, base + numel) covers the shard's real elements.
int param_target(const zero_plan* p, void* param, int64_t base, int64_t numel, int32_t dtype,
                 uint16_t** out) {
    *out = nullptr;
    if (param == nullptr) return ZERO_OK;
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "param_dtype must be ZERO_F16 or ZERO_BF16");
    if ((reinterpret_cast<uintptr_t>(param) & 1u) != 0) {
        return fail(ZERO_EALIGN, "param must be 2-byte aligned");
    }
    if (p->real <= 0) return ZERO_OK;  // a shard of padding writes no parameter
    if (base < 0 || numel < 0 || p->begin < base || p->begin + p->real - base > numel) {
        return fail(ZERO_EINVAL, "param window [param_base, param_base + param_numel) must "
                                 "contain the shard's flat range [shard_begin, shard_begin + "
                                 "real)");
    }
    *out = static_cast<uint16_t*>(param) + (p->begin - base);
    return ZERO_OK;
}

// Checks shared by the synchronous and asynchronous steps.
int check_step_buffers(const zero_plan* p, const void* flat_grad, int32_t grad_dtype,
                       const float* master, const float* exp_avg, const float* exp_avg_sq) {
    if (!valid_grad_dtype(grad_dtype)) return bad_grad_dtype();
    if (p->S > 0 && (flat_grad == nullptr || master == nullptr || exp_avg == nullptr ||
                     exp_avg_sq == nullptr)) {
        return fail(ZERO_ENULL, "flat_grad, master, exp_avg and exp_avg_sq must be non-NULL");
    }
    if (!aligned16(flat_grad)) return fail(ZERO_EALIGN, "flat_grad must be 16-byte aligned");
    if (!aligned4(master) || !aligned4(exp_avg) || !aligned4(exp_avg_sq)) {
        return fail(ZERO_EALIGN, "master, exp_avg and exp_avg_sq must be 4-byte aligned");
    }
    return ZERO_OK;
}

namespace {

// Binds the plan to the current device on first use and creates its device
// block.  The overflow flag is cleared by a one-thread kernel on the first
// call that brings a stream (stream-ordered before that call's own work; no
// memset and nothing on the null stream, so even a captured first call is
// fine); the rest of the block is written before it is read.
int ensure_device(zero_plan* p, hipStream_t s, bool have_stream = true) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DeviceState& d = p->dev;
    if (d.ready) {
        if (dev != d.device) {
            return fail(ZERO_ESTATE, "plan is bound to device " + std::to_string(d.device) +
                                         " but device " + std::to_string(dev) + " is current");
        }
        if (have_stream && !d.flag_cleared) {
            e = launch_flag_clear(d.d_flag, s);
            if (e != hipSuccess) return hip_fail(e, "flag clear");
            d.flag_cleared = true;
        }
        return ZERO_OK;
    }
    // on any failure below, release what was created so a later call starts over
    auto undo = [&d](hipError_t err, const char* what) {
        for (int i = 0; i < kTimers; ++i) {
            if (d.ev_start[i]) (void)hipEventDestroy(d.ev_start[i]);
            if (d.ev_stop[i]) (void)hipEventDestroy(d.ev_stop[i]);
            d.ev_start[i] = d.ev_stop[i] = nullptr;
        }
        if (d.h_flag) (void)hipHostFree(d.h_flag);
        if (d.d_flag) (void)hipFree(d.d_flag);
        d.h_flag = nullptr;
        d.d_flag = nullptr;
        return hip_fail(err, what);
    };
    e = hipMalloc(reinterpret_cast<void**>(&d.d_flag), kBlockBytes);
    if (e != hipSuccess) {
        d.d_flag = nullptr;
        return undo(e, "hipMalloc(device block)");
    }
    e = hipHostMalloc(reinterpret_cast<void**>(&d.h_flag), kBlockBytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        d.h_flag = nullptr;
        return undo(e, "hipHostMalloc(device block mirror)");
    }
    std::memset(d.h_flag, 0, kBlockBytes);
    for (int i = 0; i < kTimers; ++i) {
        e = hipEventCreate(&d.ev_start[i]);
        if (e == hipSuccess) e = hipEventCreate(&d.ev_stop[i]);
        if (e != hipSuccess) return undo(e, "hipEventCreate");
    }
    if (have_stream) {
        e = launch_flag_clear(d.d_flag, s);
        if (e != hipSuccess) return undo(e, "flag clear");
        d.flag_cleared = true;
    }
    d.device = dev;
    d.ready = true;
    return ZERO_OK;
}

// Event timing is skipped while the stream is being captured into a graph.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

int timer_start(zero_plan* p, Timer t, hipStream_t s) {
    if (!p->dev.timing || capturing(s)) return ZERO_OK;
    hipError_t e = hipEventRecord(p->dev.ev_start[t], s);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "hipEventRecord");
}

int timer_stop(zero_plan* p, Timer t, hipStream_t s) {
    if (!p->dev.timing || capturing(s)) return ZERO_OK;
    hipError_t e = hipEventRecord(p->dev.ev_stop[t], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    p->dev.timed[t] = true;
    return ZERO_OK;
}

// gate_flag with the scan, when it runs, timed like the other kernels.
int timed_gate(zero_plan* p, const void* flat_grad, int32_t grad_dtype, hipStream_t s) {
    if (flatten_covered(p, flat_grad, grad_dtype)) return ZERO_OK;
    int rc = timer_start(p, kTimerScan, s);
    if (rc != ZERO_OK) return rc;
    bool scanned = false;
    if ((rc = gate_flag(p, flat_grad, grad_dtype, s, &scanned)) != ZERO_OK) return rc;
    return timer_stop(p, kTimerScan, s);
}

DeviceStep* device_step(zero_plan* p) {
    return reinterpret_cast<DeviceStep*>(reinterpret_cast<char*>(p->dev.d_flag) + kStateOffset);
}

AdamScalars* device_scalars(zero_plan* p) {
    return reinterpret_cast<AdamScalars*>(reinterpret_cast<char*>(p->dev.d_flag) +
                                          kScalarsOffset);
}

int check_scaler(const zero_scaler_t* sc) {
    if (!(std::isfinite(sc->scale) && sc->scale > 0) ||
        !(std::isfinite(sc->min_scale) && sc->min_scale > 0) ||
        !(sc->backoff > 0 && sc->backoff <= 1) || !(std::isfinite(sc->growth) && sc->growth >= 1) ||
        sc->window < 1 || sc->good_steps < 0) {
        return fail(ZERO_EINVAL, "scaler fields out of range");
    }
    return ZERO_OK;
}

// Host threads kept for zero_cpu_adam_step across calls (starting threads
// per call costs about a millisecond on a 16-thread share).  One caller at a
// time uses it; a concurrent caller starts threads of its own instead.
// The pool is never destroyed at exit, and a process made by fork() does not
// use the one it inherited: that copy's threads were not copied, so joining
// or waiting for them would never end.  A child that inherits the mutex
// locked only ever starts threads of its own.
std::mutex g_host_pool_mu;
HostPool* g_host_pool = nullptr;
pid_t g_host_pool_pid = 0;

// The overflow test (overflow < 0) and the update, on the kept threads when
// they are free.  Returns 1 when the step is skipped.
int run_host_step(const CpuAdamArgs& a, int32_t overflow, int n_threads) {
    std::unique_lock<std::mutex> lk(g_host_pool_mu, std::try_to_lock);
    HostPool* pool = nullptr;
    if (lk.owns_lock()) {
        if (g_host_pool != nullptr && g_host_pool_pid != getpid()) g_host_pool = nullptr;
        if (g_host_pool != nullptr && g_host_pool->size() != n_threads) {
            delete g_host_pool;
            g_host_pool = nullptr;
        }
        if (g_host_pool == nullptr) {
            try {
                g_host_pool = new HostPool(n_threads);
                g_host_pool_pid = getpid();
            } catch (const std::exception&) {
                // its threads could not all be started: this call starts
                // what it can itself (parallel_ranges), and a later call
                // tries to build the pool again
            }
        }
        pool = g_host_pool;
    }
    // like the device gate, the test covers the real elements only
    const bool skip =
        overflow < 0 ? cpu_nonfinite(a.g, a.real, a.gdt, n_threads, pool) : overflow != 0;
    if (skip) return 1;
    cpu_adam(a, n_threads, pool);
    return 0;
}

}  // namespace
}  // namespace zmi

using namespace zmi;

extern "C" {

int zero_partition_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size,
                        int32_t rank, int64_t align_elems, int64_t bucket_elems,
                        zero_plan_t** out) {
    if (out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    *out = nullptr;
    zero_plan* p = new (std::nothrow) zero_plan();
    if (p == nullptr) return fail(ZERO_ENOMEM, "plan allocation failed");
    int rc;
    try {
        rc = build_plan(numels, n_tensors, world_size, rank, align_elems, bucket_elems, p);
    } catch (const std::bad_alloc&) {
        rc = fail(ZERO_ENOMEM, "plan tables allocation failed");
    }
    if (rc != ZERO_OK) {
        delete p;
        return rc;
    }
    *out = p;
    return ZERO_OK;
}

int zero_plan_info(const zero_plan_t* p, zero_plan_info_t* out) {
    if (p == nullptr || out == nullptr) return fail(ZERO_ENULL, "plan or out is NULL");
    std::memset(out, 0, sizeof(*out));
    out->total_numel = p->P;
    out->padded_numel = p->P_pad;
    out->shard_numel = p->S;
    out->shard_begin = p->begin;
    out->real_numel = p->real;
    out->align_elems = p->align;
    out->bucket_elems = p->bucket_elems;
    // per-rank model-state bytes: half params 2 B, half grads 2 B, fp32
    // master + momentum + variance 12 B per element held
    out->bytes_stage1 = 2 * p->P + 2 * p->P + 12 * p->S;
    out->bytes_stage2 = 2 * p->P + 2 * p->S + 12 * p->S;
    out->bytes_stage3 = 2 * p->S + 2 * p->S + 12 * p->S;
    out->world_size = p->R;
    out->rank = p->r;
    out->n_tensors = static_cast<int32_t>(p->numels.size());
    out->n_segments = static_cast<int32_t>(p->segs.size());
    out->n_buckets = p->n_buckets;
    return ZERO_OK;
}

int64_t zero_plan_segments(const zero_plan_t* p, zero_segment_t* out, int64_t cap) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (cap < 0) return fail(ZERO_EINVAL, "cap must be >= 0");
    if (cap > 0 && out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    const int64_t n = static_cast<int64_t>(p->segs.size());
    for (int64_t s = 0; s < n && s < cap; ++s) {
        const Segment& g = p->segs[s];
        out[s] = zero_segment_t{g.tensor, g.tensor_off, g.shard_off, g.numel, g.bucket, 0};
    }
    return n;
}

int zero_plan_tensor_buckets(const zero_plan_t* p, int32_t* out, int64_t cap) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (cap < 0) return fail(ZERO_EINVAL, "cap must be >= 0");
    if (cap > 0 && out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    const int64_t n = static_cast<int64_t>(p->tensor_bucket.size());
    for (int64_t i = 0; i < n && i < cap; ++i) out[i] = p->tensor_bucket[i];
    return ZERO_OK;
}

void zero_plan_destroy(zero_plan_t* p) {
    if (p == nullptr) return;
    DeviceState& d = p->dev;
    if (d.ready) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != d.device) (void)hipSetDevice(d.device);
        for (int i = 0; i < kTimers; ++i) {
            if (d.ev_start[i]) (void)hipEventDestroy(d.ev_start[i]);
            if (d.ev_stop[i]) (void)hipEventDestroy(d.ev_stop[i]);
        }
        if (d.d_flag) (void)hipFree(d.d_flag);
        if (d.h_flag) (void)hipHostFree(d.h_flag);
        if (cur != d.device && cur >= 0) (void)hipSetDevice(cur);
    }
    delete p;
}

int zero_flatten_grads(zero_plan_t* p, int32_t bucket, const void* const* grads,
                       int32_t grad_dtype, void* flat_grad, void* stream) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (!valid_grad_dtype(grad_dtype)) return bad_grad_dtype();
    if (bucket < -1 || bucket >= p->n_buckets) {
        return fail(ZERO_EINVAL, "bucket must be -1 or in [0, n_buckets)");
    }
    if (p->S > 0 && flat_grad == nullptr) return fail(ZERO_ENULL, "flat_grad is NULL");
    if (!aligned16(flat_grad)) return fail(ZERO_EALIGN, "flat_grad must be 16-byte aligned");
    int64_t s_first = 0, s_last = static_cast<int64_t>(p->segs.size());
    if (bucket >= 0) {
        s_first = p->bucket_seg_first[bucket];
        s_last = p->bucket_seg_last[bucket];
    }
    if (s_last > s_first && grads == nullptr) return fail(ZERO_ENULL, "grads is NULL");
    // pieces of this call: the bucket's segments, then the padding tail
    const uintptr_t esize = static_cast<uintptr_t>(grad_bytes(grad_dtype));
    std::vector<FlatPiece> pieces;
    try {
        pieces.reserve(static_cast<size_t>(s_last - s_first) + 1);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "flatten piece table allocation failed");
    }
    for (int64_t s = s_first; s < s_last; ++s) {
        const Segment& g = p->segs[s];
        const void* src = grads[g.tensor];
        if (src == nullptr) {
            return fail(ZERO_ENULL, "grads[" + std::to_string(g.tensor) +
                                        "] is NULL but the tensor has elements in this shard");
        }
        if ((reinterpret_cast<uintptr_t>(src) & (esize - 1u)) != 0) {
            return fail(ZERO_EALIGN, "grads[" + std::to_string(g.tensor) + "] is not " +
                                         std::to_string(esize) + "-byte aligned");
        }
        // byte address of the source of flat element 0 (mod 2^64)
        const uintptr_t base = reinterpret_cast<uintptr_t>(src) +
                               esize * static_cast<uintptr_t>(g.tensor_off) -
                               esize * static_cast<uintptr_t>(g.shard_off);
        pieces.push_back(FlatPiece{g.shard_off, g.shard_off + g.numel, base});
    }
    if (p->S > p->real) pieces.push_back(FlatPiece{p->real, p->S, 0});
    int rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a flatten into another buffer (or dtype) than the one the pending
    // flag belongs to starts the flag over: a step gates on what was found
    // in the buffer it consumes
    if (p->flattened_into != flat_grad || p->flattened_dtype != grad_dtype) {
        if (p->flattened_into != nullptr) {
            hipError_t e = launch_flag_clear(p->dev.d_flag, s);
            if (e != hipSuccess) return hip_fail(e, "flag clear");
        }
        // the bookkeeping follows the new buffer before anything is launched
        // into it, so a launch that fails below leaves it uncovered (a step
        // on it scans), never the previous buffer covered by a cleared flag
        std::fill(p->bucket_flattened.begin(), p->bucket_flattened.end(), 0);
        p->flatten_all_done = false;
        p->flattened_into = flat_grad;
        p->flattened_dtype = grad_dtype;
    }
    if ((rc = timer_start(p, kTimerFlatten, s)) != ZERO_OK) return rc;
    // launches of up to kMaxPiecesPerLaunch contiguous pieces each
    size_t i = 0;
    while (i < pieces.size()) {
        size_t j = i + 1;
        while (j < pieces.size() && j - i < static_cast<size_t>(kMaxPiecesPerLaunch) &&
               pieces[j].begin == pieces[j - 1].end) {
            ++j;
        }
        hipError_t e = launch_flatten(pieces.data() + i, static_cast<int>(j - i), flat_grad,
                                      p->dev.d_flag, grad_dtype, s);
        if (e != hipSuccess) return hip_fail(e, "flatten launch");
        i = j;
    }
    if ((rc = timer_stop(p, kTimerFlatten, s)) != ZERO_OK) return rc;
    // bookkeeping for the gate: which buckets reached this flat buffer
    if (bucket < 0) {
        p->flatten_all_done = true;
    } else {
        p->bucket_flattened[bucket] = 1;
    }
    return ZERO_OK;
}

int zero_flatten_invalidate(zero_plan_t* p) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    reset_flatten_bookkeeping(p);
    return ZERO_OK;
}

int zero_adam_step(zero_plan_t* p, const zero_adam_hparams_t* hp, int64_t step, double loss_scale,
                   const void* flat_grad, int32_t grad_dtype, float* master, float* exp_avg,
                   float* exp_avg_sq, void* param, int64_t param_base, int64_t param_numel,
                   int32_t param_dtype, void* stream) {
    if (p == nullptr || hp == nullptr) return fail(ZERO_ENULL, "plan or hparams is NULL");
    if (!valid_grad_dtype(grad_dtype)) return bad_grad_dtype();
    if (step < 1) return fail(ZERO_EINVAL, "step must be >= 1");
    if (!(std::isfinite(loss_scale) && loss_scale > 0)) {
        return fail(ZERO_EINVAL, "loss_scale must be finite and > 0");
    }
    int rc = check_hparams(hp);
    if (rc != ZERO_OK) return rc;
    rc = check_step_buffers(p, flat_grad, grad_dtype, master, exp_avg, exp_avg_sq);
    if (rc != ZERO_OK) return rc;
    uint16_t* param0 = nullptr;
    rc = param_target(p, param, param_base, param_numel, param_dtype, &param0);
    if (rc != ZERO_OK) return rc;
    rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // host scalars: double, each rounded once to fp32
    const AdamScalars sc = make_scalars(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay,
                                        hp->adamw, static_cast<double>(step), loss_scale);

    // the gate needs every real gradient of this flat buffer tested
    if ((rc = timed_gate(p, flat_grad, grad_dtype, s)) != ZERO_OK) return rc;
    if ((rc = timer_start(p, kTimerAdam, s)) != ZERO_OK) return rc;
    hipError_t e = launch_adam(flat_grad, master, exp_avg,
                               exp_avg_sq, param0, p->S, p->real, p->dev.d_flag, sc, nullptr,
                               grad_dtype, param_dtype, hp->adamw != 0, s);
    if (e != hipSuccess) return hip_fail(e, "adam launch");
    if ((rc = timer_stop(p, kTimerAdam, s)) != ZERO_OK) return rc;
    e = hipMemcpyAsync(p->dev.h_flag, p->dev.d_flag, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "flag readback");
    e = launch_flag_clear(p->dev.d_flag, s);
    if (e != hipSuccess) return hip_fail(e, "flag clear");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    reset_flatten_bookkeeping(p);
    return *p->dev.h_flag != 0 ? 1 : 0;
}

int zero_state_upload(zero_plan_t* p, int64_t applied_steps, const zero_scaler_t* scaler,
                      void* stream) {
    if (p == nullptr || scaler == nullptr) return fail(ZERO_ENULL, "plan or scaler is NULL");
    if (applied_steps < 0) return fail(ZERO_EINVAL, "applied_steps must be >= 0");
    int rc = check_scaler(scaler);
    if (rc != ZERO_OK) return rc;
    rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // stage in the pinned mirror; the stream is drained before returning, so
    // the mirror is free again afterwards
    DeviceStep d{};
    d.t = applied_steps;
    d.skipped = 0;
    d.scale = scaler->scale;
    d.min_scale = scaler->min_scale;
    d.backoff = scaler->backoff;
    d.growth = scaler->growth;
    d.window = scaler->window;
    d.good_steps = scaler->good_steps;
    d.dynamic = scaler->dynamic != 0;
    d.last_flag = 0;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    char* mirror = reinterpret_cast<char*>(p->dev.h_flag);
    std::memcpy(mirror + kStateOffset, &d, sizeof(d));
    e = hipMemcpyAsync(device_step(p), mirror + kStateOffset, sizeof(d), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "state upload");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    p->dev.state_ready = true;
    return ZERO_OK;
}

int zero_state_download(zero_plan_t* p, int64_t* applied_steps, zero_scaler_t* scaler,
                        int32_t* last_flag, int64_t* skipped_steps, void* stream) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (!p->dev.ready || !p->dev.state_ready) {
        return fail(ZERO_ESTATE, "no device state: call zero_state_upload first");
    }
    int rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* mirror = reinterpret_cast<char*>(p->dev.h_flag);
    hipError_t e = hipMemcpyAsync(mirror + kStateOffset, device_step(p), sizeof(DeviceStep),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "state download");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    DeviceStep d;
    std::memcpy(&d, mirror + kStateOffset, sizeof(d));
    if (applied_steps) *applied_steps = d.t;
    if (skipped_steps) *skipped_steps = d.skipped;
    if (last_flag) *last_flag = d.last_flag;
    if (scaler) {
        scaler->scale = d.scale;
        scaler->min_scale = d.min_scale;
        scaler->backoff = d.backoff;
        scaler->growth = d.growth;
        scaler->window = d.window;
        scaler->good_steps = d.good_steps;
        scaler->dynamic = d.dynamic;
    }
    return ZERO_OK;
}

int zero_state_device_scale(zero_plan_t* p, const double** out) {
    if (p == nullptr || out == nullptr) return fail(ZERO_ENULL, "plan or out is NULL");
    if (!p->dev.ready || !p->dev.state_ready) {
        return fail(ZERO_ESTATE, "no device state: call zero_state_upload first");
    }
    *out = &device_step(p)->scale;
    return ZERO_OK;
}

int zero_adam_step_async(zero_plan_t* p, const zero_adam_hparams_t* hp, const void* flat_grad,
                         int32_t grad_dtype, float* master, float* exp_avg, float* exp_avg_sq,
                         void* param, int64_t param_base, int64_t param_numel,
                         int32_t param_dtype, void* stream) {
    if (p == nullptr || hp == nullptr) return fail(ZERO_ENULL, "plan or hparams is NULL");
    int rc = check_hparams(hp);
    if (rc != ZERO_OK) return rc;
    rc = check_step_buffers(p, flat_grad, grad_dtype, master, exp_avg, exp_avg_sq);
    if (rc != ZERO_OK) return rc;
    uint16_t* param0 = nullptr;
    rc = param_target(p, param, param_base, param_numel, param_dtype, &param0);
    if (rc != ZERO_OK) return rc;
    // allocation happens at zero_state_upload, never here: this call may be
    // captured into a graph
    if (!p->dev.ready || !p->dev.state_ready) {
        return fail(ZERO_ESTATE, "no device state: call zero_state_upload first");
    }
    rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = timed_gate(p, flat_grad, grad_dtype, s)) != ZERO_OK) return rc;
    hipError_t e = launch_step_prologue(p->dev.d_flag, device_step(p), device_scalars(p), *hp, s);
    if (e != hipSuccess) return hip_fail(e, "step prologue launch");
    if ((rc = timer_start(p, kTimerAdam, s)) != ZERO_OK) return rc;
    const AdamScalars unused{};
    e = launch_adam(flat_grad, master, exp_avg, exp_avg_sq, param0,
                    p->S, p->real, p->dev.d_flag, unused, device_scalars(p), grad_dtype,
                    param_dtype, hp->adamw != 0, s);
    if (e != hipSuccess) return hip_fail(e, "adam launch");
    if ((rc = timer_stop(p, kTimerAdam, s)) != ZERO_OK) return rc;
    e = launch_step_epilogue(p->dev.d_flag, device_step(p), s);
    if (e != hipSuccess) return hip_fail(e, "step epilogue launch");
    reset_flatten_bookkeeping(p);
    return ZERO_OK;
}

int zero_update_loss_scale(zero_scaler_t* sc, int32_t overflow) {
    if (sc == nullptr) return fail(ZERO_ENULL, "scaler is NULL");
    int rc = check_scaler(sc);
    if (rc != ZERO_OK) return rc;
    if (overflow) {
        if (sc->dynamic) sc->scale = std::max(sc->scale * sc->backoff, sc->min_scale);
        sc->good_steps = 0;
        return ZERO_OK;
    }
    sc->good_steps += 1;
    if (sc->dynamic && sc->good_steps >= sc->window) {
        sc->scale *= sc->growth;
        sc->good_steps = 0;
    }
    return ZERO_OK;
}

int zero_write_param_shard(zero_plan_t* p, const float* master, void* param, int64_t param_base,
                           int64_t param_numel, int32_t param_dtype, void* stream) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (param == nullptr) return fail(ZERO_ENULL, "param is NULL");
    if (p->real > 0 && master == nullptr) return fail(ZERO_ENULL, "master is NULL");
    if (!aligned4(master)) return fail(ZERO_EALIGN, "master must be 4-byte aligned");
    uint16_t* param0 = nullptr;
    int rc = param_target(p, param, param_base, param_numel, param_dtype, &param0);
    if (rc != ZERO_OK) return rc;
    rc = ensure_device(p, static_cast<hipStream_t>(stream));
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = timer_start(p, kTimerWrite, s)) != ZERO_OK) return rc;
    hipError_t e = launch_write_param(master, param0, p->real, param_dtype, s);
    if (e != hipSuccess) return hip_fail(e, "write_param launch");
    return timer_stop(p, kTimerWrite, s);
}

int zero_cpu_adam_step(const zero_plan_t* p, const zero_adam_hparams_t* hp, int64_t step,
                       double loss_scale, const void* flat_grad, int32_t grad_dtype,
                       float* master, float* exp_avg, float* exp_avg_sq, void* param,
                       int64_t param_base, int64_t param_numel, int32_t param_dtype,
                       int32_t overflow, int32_t n_threads) {
    if (p == nullptr || hp == nullptr) return fail(ZERO_ENULL, "plan or hparams is NULL");
    if (!valid_grad_dtype(grad_dtype)) return bad_grad_dtype();
    if (step < 1) return fail(ZERO_EINVAL, "step must be >= 1");
    if (!(std::isfinite(loss_scale) && loss_scale > 0)) {
        return fail(ZERO_EINVAL, "loss_scale must be finite and > 0");
    }
    if (overflow < -1 || overflow > 1) return fail(ZERO_EINVAL, "overflow must be -1, 0 or 1");
    if (n_threads < 1 || n_threads > 1024) return fail(ZERO_EINVAL, "n_threads must be in [1, 1024]");
    int rc = check_hparams(hp);
    if (rc != ZERO_OK) return rc;
    if (p->S > 0 && (flat_grad == nullptr || master == nullptr || exp_avg == nullptr ||
                     exp_avg_sq == nullptr)) {
        return fail(ZERO_ENULL, "flat_grad, master, exp_avg and exp_avg_sq must be non-NULL");
    }
    if ((reinterpret_cast<uintptr_t>(flat_grad) & (grad_bytes(grad_dtype) - 1u)) != 0 ||
        !aligned4(master) || !aligned4(exp_avg) || !aligned4(exp_avg_sq)) {
        return fail(ZERO_EALIGN,
                    "flat_grad must be aligned to its element size and the fp32 arrays to 4 bytes");
    }
    uint16_t* param0 = nullptr;
    rc = param_target(p, param, param_base, param_numel, param_dtype, &param0);
    if (rc != ZERO_OK) return rc;
    CpuAdamArgs a;
    a.g = flat_grad;
    a.p = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.param = param0;
    a.n = p->S;
    a.real = p->real;
    a.sc = make_scalars(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->adamw,
                        static_cast<double>(step), loss_scale);
    a.gdt = grad_dtype;
    a.pdt = param_dtype;
    a.adamw = hp->adamw != 0;
    try {
        return run_host_step(a, overflow, n_threads);
    } catch (const std::exception& ex) {
        return fail(ZERO_ENOMEM, std::string("host update failed: ") + ex.what());
    }
}

int zero_adam_scalars(const zero_adam_hparams_t* hp, int64_t t_first, int64_t count,
                      double loss_scale, float* out, int32_t on_device, void* stream) {
    if (hp == nullptr) return fail(ZERO_ENULL, "hparams is NULL");
    int rc = check_hparams(hp);
    if (rc != ZERO_OK) return rc;
    if (t_first < 1 || count < 0 || count > (int64_t(1) << 40) - t_first) {
        return fail(ZERO_EINVAL, "need t_first >= 1 and 0 <= count < 2^40 - t_first");
    }
    if (!(std::isfinite(loss_scale) && loss_scale > 0)) {
        return fail(ZERO_EINVAL, "loss_scale must be finite and > 0");
    }
    if (on_device != 0 && on_device != 1) return fail(ZERO_EINVAL, "on_device must be 0 or 1");
    if (count == 0) return ZERO_OK;
    if (out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    if (!aligned4(out)) return fail(ZERO_EALIGN, "out must be 4-byte aligned");
    auto* dst = reinterpret_cast<AdamScalars*>(out);
    if (on_device) {
        hipError_t e = launch_adam_scalars(*hp, t_first, count, loss_scale, dst,
                                           static_cast<hipStream_t>(stream));
        return e == hipSuccess ? ZERO_OK : hip_fail(e, "scalars launch");
    }
    for (int64_t i = 0; i < count; ++i) {
        dst[i] = make_scalars(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->adamw,
                              static_cast<double>(t_first + i), loss_scale);
    }
    return ZERO_OK;
}

const char* zero_cpu_isa(void) { return cpu_isa_name(cpu_isa()); }

const char* zero_last_error(void) { return g_last_error; }

int zero_plan_set_timing(zero_plan_t* p, int32_t on) {
    if (p == nullptr) return fail(ZERO_ENULL, "plan is NULL");
    if (on) {
        int rc = ensure_device(p, nullptr, false);
        if (rc != ZERO_OK) return rc;
    }
    p->dev.timing = on != 0;
    for (int i = 0; i < kTimers; ++i) p->dev.timed[i] = false;
    return ZERO_OK;
}

int zero_plan_kernel_ms(zero_plan_t* p, int32_t which, float* ms) {
    if (p == nullptr || ms == nullptr) return fail(ZERO_ENULL, "plan or ms is NULL");
    if (which < 0 || which >= kTimers) return fail(ZERO_EINVAL, "which must be in [0, 4)");
    if (!p->dev.ready || !p->dev.timed[which]) {
        return fail(ZERO_ESTATE, "that kernel has not run with timing enabled");
    }
    hipError_t e = hipEventSynchronize(p->dev.ev_stop[which]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    e = hipEventElapsedTime(ms, p->dev.ev_start[which], p->dev.ev_stop[which]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    return ZERO_OK;
}

}  // extern "C"
