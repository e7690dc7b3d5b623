// ZeRO-Offload for one rank, with the one-step delayed parameter update.
//
// "ZeRO Optimization", inferensys glossary: the legal pre-training page,
// offload list (CPU-offload bullet: optimizer states in CPU DRAM, Adam on the
// CPU while the GPU runs forward and backward; DPU bullet: the CPU optimizer
// step of one iteration overlaps the next iteration's forward pass), and the
// genomic MLOps page, offload list (fp32 master weights and optimizer states
// in CPU RAM, half parameters and gradients on the GPU; DPU overlaps CPU and
// GPU computation).
//
// Per submitted step i (caller's stream, after zero_flatten_grads):
//   snapshot kernel   flag, t + 1 and the scale of step i -> device slot i%2;
//                     loss-scale policy applied to the device state; flag
//                     cleared (so the next backward already sees the new scale)
//   D2H               slot -> host, then the flat gradient shard -> pinned host
//                     buffer i%2 in chunks (up to kMaxChunks, an event after each)
// Worker thread, steps in order:
//   wait for the slot; skipped step: nothing else.  Otherwise, chunk by chunk
//   as each arrives, the host update (cpu_adam on the pipeline's thread pool,
//   same arithmetic as the device update) writes master / moments in host
//   memory and the half parameters into pinned buffer i%2.  The parameters
//   go back to the rank's offset on the library's transfer stream once the
//   caller has released the device parameters of step i (event recorded by
//   the next submit, by zero_offload_wait_params or by zero_offload_drain):
//   chunk by chunk while the update runs if the release is already there
//   (the serialised step, lag 0), otherwise all at once after the update --
//   the update never waits for the release.  So the copies of a step overlap
//   its own update instead of running before and after it.
// zero_offload_wait_params(lag) makes the caller's stream wait until the
// parameters of every submitted step but the last `lag` are on the device:
// lag = 1 is the one-step delayed update (the host work of step i runs while
// the GPU computes step i + 1), lag = 0 the plain, serialised step.
#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"

namespace zmi {
namespace {

struct Pending {
    int64_t idx = -1;
    uint16_t* param_dst = nullptr;  // device address of shard element 0's parameter
    bool free_recorded = false;     // ev_free[b] holds the release point
    bool processed = false;         // host part done, H2D enqueued (or step skipped)
    bool applied = false;
    bool timeline = false;          // the submit recorded timeline events for this step
};

constexpr int kMaxChunks = 16;                       // gradient / parameter copy pieces
constexpr int64_t kMinChunkElems = int64_t(1) << 25;  // per piece (64-128 MB of gradients)

}  // namespace
}  // namespace zmi

using namespace zmi;

using Clock0 = std::chrono::steady_clock::time_point;

struct zero_offload {
    zero_plan* plan = nullptr;
    zero_adam_hparams_t hp{};
    int gdt = 0, pdt = 0;
    float* master = nullptr;
    float* m = nullptr;
    float* v = nullptr;
    int n_threads = 1;
    int device = -1;
    HostPool* pool = nullptr;
    int n_chunks = 0;   // pieces of the shard for the copies and the update
    int64_t chunk = 0;  // elements per piece (a multiple of 64; the last may be short)
    // library-owned buffers
    void* hgrad[2] = {nullptr, nullptr};       // pinned, S gradients each
    uint16_t* hparam[2] = {nullptr, nullptr};  // pinned, max(real, 1) each
    OffloadSlot* hslot = nullptr;              // pinned, 2 slots
    OffloadSlot* dslot = nullptr;              // device, 2 slots
    hipStream_t xfer = nullptr;
    hipEvent_t ev_slot[2] = {}, ev_free[2] = {}, ev_h2d[2] = {};
    hipEvent_t ev_d2h[2][kMaxChunks] = {};
    bool h2d_recorded[2] = {false, false};  // written under mu; the worker also reads it unlocked
    // steps
    Pending rec[2];
    int64_t submitted = 0;
    int64_t processed = 0;
    // worker
    std::thread worker;
    std::mutex mu;
    std::condition_variable cv;
    bool stop = false;
    // stats (under mu)
    int64_t applied = 0, skipped = 0;
    int32_t last_flag = 0;
    double host_ms_last = 0, host_ms_total = 0;
    double wait_submit_ms = 0, wait_grad_ms = 0, wait_h2d_ms = 0, wait_release_ms = 0;
    double caller_wait_ms = 0;
    int err = ZERO_OK;
    std::string err_msg;
    // optional timeline (zero_offload_timeline_start): timing events around
    // every piece's copies, host times around its update, all on one host
    // clock; tl_* written by the submitting thread before a step is handed
    // over, or by the worker while it owns the step, read under mu
    bool tl_on = false;
    int64_t tl_cap = 0;
    Clock0 tl_t0{};                 // host time of the reference event
    hipEvent_t tl_ref = nullptr;    // reference event, completed at tl_t0
    hipEvent_t tl_d2h[2][kMaxChunks][2] = {};  // start / end of each gradient piece
    hipEvent_t tl_h2d[2][kMaxChunks][2] = {};  // start / end of each parameter piece
    bool tl_d2h_rec[2] = {false, false};       // step in buffer b recorded its gradient events
    int64_t tl_h2d_step[2] = {-1, -1};         // step whose parameter events buffer b holds
    bool tl_h2d_sent[2][kMaxChunks] = {};      // pieces of that step with recorded events
    std::vector<zero_offload_interval_t> tl;
};

namespace {

using Clock = std::chrono::steady_clock;

double ms_since(Clock::time_point t0) {
    return std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
}

void set_worker_error(zero_offload* o, int code, const std::string& msg) {
    std::lock_guard<std::mutex> g(o->mu);
    if (o->err == ZERO_OK) {
        o->err = code;
        o->err_msg = msg;
    }
    o->cv.notify_all();
}

int worker_hip(zero_offload* o, hipError_t e, const char* what) {
    if (e == hipSuccess) return ZERO_OK;
    set_worker_error(o, ZERO_EHIP,
                     std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
    return ZERO_EHIP;
}

// ---- timeline (caller holds mu for tl_push and tl_read_h2d)
double tl_host_ms(const zero_offload* o, Clock::time_point t) {
    return std::chrono::duration<double, std::milli>(t - o->tl_t0).count();
}

void tl_push(zero_offload* o, int64_t step, int piece, int kind, double t0, double t1) {
    if (static_cast<int64_t>(o->tl.size()) >= o->tl_cap) return;  // past the capacity: dropped
    zero_offload_interval_t r{};
    r.step = step;
    r.piece = piece;
    r.kind = kind;
    r.start_ms = t0;
    r.end_ms = t1;
    try {
        o->tl.push_back(r);
    } catch (const std::bad_alloc&) {
        // the worker thread must not throw: out of host memory, the
        // timeline keeps what it holds and records nothing more
        o->tl_cap = static_cast<int64_t>(o->tl.size());
    }
}

// Start and end of an event pair on the host clock; false if not complete.
bool tl_pair_ms(const zero_offload* o, hipEvent_t const (&ev)[2], double* t0, double* t1) {
    float a = 0.f, b = 0.f;
    if (hipEventElapsedTime(&a, o->tl_ref, ev[0]) != hipSuccess) return false;
    if (hipEventElapsedTime(&b, o->tl_ref, ev[1]) != hipSuccess) return false;
    *t0 = a;
    *t1 = b;
    return true;
}

// Moves the parameter-copy intervals buffer b holds into the timeline if
// its copies are complete (one stream: the last piece's end implies the
// others'); otherwise leaves them for a later call.
void tl_read_h2d(zero_offload* o, int b) {
    if (o->tl_h2d_step[b] < 0) return;
    int last = -1;
    for (int c = 0; c < o->n_chunks; ++c) {
        if (o->tl_h2d_sent[b][c]) last = c;
    }
    if (last >= 0) {
        if (hipEventQuery(o->tl_h2d[b][last][1]) != hipSuccess) return;
        for (int c = 0; c <= last; ++c) {
            double t0 = 0, t1 = 0;
            if (o->tl_h2d_sent[b][c] && tl_pair_ms(o, o->tl_h2d[b][c], &t0, &t1)) {
                tl_push(o, o->tl_h2d_step[b], c, 2, t0, t1);
            }
            o->tl_h2d_sent[b][c] = false;
        }
    }
    o->tl_h2d_step[b] = -1;
}

// Enqueues the parameter copies of chunks [*sent, upto) of step buffer b on
// the transfer stream, gated once on the caller's release of the device
// parameters.  block = false: does nothing until that release is recorded.
// Returns ZERO_OK, or ZERO_ESTATE when stopped while waiting, or the HIP error.
int send_params(zero_offload* o, int b, int upto, bool block, int* sent, bool* gated,
                double* wait_release) {
    const zero_plan* p = o->plan;
    if (o->pdt == 0 || p->real <= 0) {
        *sent = upto;
        return ZERO_OK;
    }
    uint16_t* dst = nullptr;
    bool tl = false;
    int64_t step = -1;
    {
        std::unique_lock<std::mutex> lk(o->mu);
        if (!o->rec[b].free_recorded) {
            if (!block) return ZERO_OK;
            const auto tw = Clock::now();
            o->cv.wait(lk, [&] { return o->stop || o->rec[b].free_recorded; });
            if (!o->rec[b].free_recorded) return ZERO_ESTATE;
            *wait_release += ms_since(tw);
        }
        dst = o->rec[b].param_dst;
        tl = o->rec[b].timeline;
        step = o->rec[b].idx;
    }
    if (dst == nullptr) {
        *sent = upto;
        return ZERO_OK;
    }
    if (!*gated) {
        if (worker_hip(o, hipStreamWaitEvent(o->xfer, o->ev_free[b], 0), "wait") != ZERO_OK) {
            return ZERO_EHIP;
        }
        *gated = true;
    }
    for (int c = *sent; c < upto; ++c) {
        const int64_t lo = c * o->chunk;
        const int64_t hi = std::min(p->real, lo + o->chunk);
        if (hi <= lo) continue;
        if (tl && worker_hip(o, hipEventRecord(o->tl_h2d[b][c][0], o->xfer), "hipEventRecord") !=
                      ZERO_OK) {
            return ZERO_EHIP;
        }
        if (worker_hip(o, hipMemcpyAsync(dst + lo, o->hparam[b] + lo,
                                         2 * static_cast<size_t>(hi - lo),
                                         hipMemcpyHostToDevice, o->xfer),
                       "parameter copy") != ZERO_OK) {
            return ZERO_EHIP;
        }
        if (tl) {
            if (worker_hip(o, hipEventRecord(o->tl_h2d[b][c][1], o->xfer), "hipEventRecord") !=
                ZERO_OK) {
                return ZERO_EHIP;
            }
            std::lock_guard<std::mutex> g(o->mu);
            o->tl_h2d_step[b] = step;
            o->tl_h2d_sent[b][c] = true;
        }
    }
    *sent = upto;
    return ZERO_OK;
}

void worker_main(zero_offload* o) {
    if (worker_hip(o, hipSetDevice(o->device), "hipSetDevice") != ZERO_OK) return;
    const zero_plan* p = o->plan;
    const size_t esize = static_cast<size_t>(grad_bytes(o->gdt));
    for (int64_t j = 0;; ++j) {
        const int b = static_cast<int>(j & 1);
        auto tw = Clock::now();
        {
            std::unique_lock<std::mutex> lk(o->mu);
            o->cv.wait(lk, [&] { return o->stop || o->submitted > j; });
            if (o->submitted <= j) return;  // stopped with nothing left
        }
        const double wait_submit = ms_since(tw);
        bool tl = false;
        {
            std::lock_guard<std::mutex> g(o->mu);
            tl = o->rec[b].timeline;
        }
        // gradient piece c of this step as an interval (its copies are done)
        const auto tl_d2h = [&](int c) {
            double t0 = 0, t1 = 0;
            if (tl && tl_pair_ms(o, o->tl_d2h[b][c], &t0, &t1)) {
                std::lock_guard<std::mutex> g(o->mu);
                tl_push(o, j, c, 0, t0, t1);
            }
        };
        tw = Clock::now();
        if (worker_hip(o, hipEventSynchronize(o->ev_slot[b]), "slot copy") != ZERO_OK) return;
        double wait_grad = ms_since(tw), wait_h2d = 0, wait_release = 0, host_ms = 0;
        const OffloadSlot slot = o->hslot[b];
        bool applied = false;
        bool gated = false;
        if (slot.flag == 0) {
            // the pinned parameter buffer b was last sent by step j - 2
            tw = Clock::now();
            if (o->h2d_recorded[b] &&
                worker_hip(o, hipEventSynchronize(o->ev_h2d[b]), "parameter copy") != ZERO_OK) {
                return;
            }
            wait_h2d = ms_since(tw);
            if (o->h2d_recorded[b]) {  // step j - 2's parameter copies are complete
                std::lock_guard<std::mutex> g(o->mu);
                tl_read_h2d(o, b);
            }
            CpuAdamArgs a;
            a.sc = make_scalars(o->hp.lr, o->hp.beta1, o->hp.beta2, o->hp.eps,
                                o->hp.weight_decay, o->hp.adamw, static_cast<double>(slot.t),
                                slot.scale);
            a.gdt = o->gdt;
            a.pdt = o->pdt;
            a.adamw = o->hp.adamw != 0;
            int sent = 0;
            for (int c = 0; c < o->n_chunks; ++c) {
                const int64_t lo = c * o->chunk;
                const int64_t hi = std::min(p->S, lo + o->chunk);
                tw = Clock::now();
                if (worker_hip(o, hipEventSynchronize(o->ev_d2h[b][c]), "gradient copy") !=
                    ZERO_OK) {
                    return;
                }
                wait_grad += ms_since(tw);
                tl_d2h(c);
                a.g = static_cast<const char*>(o->hgrad[b]) + esize * static_cast<size_t>(lo);
                a.p = o->master + lo;
                a.m = o->m + lo;
                a.v = o->v + lo;
                a.param = o->pdt ? o->hparam[b] + lo : nullptr;
                a.n = hi - lo;
                a.real = std::max<int64_t>(0, std::min(p->real, hi) - lo);
                const auto t0 = Clock::now();
                cpu_adam(a, o->n_threads, o->pool);
                const auto t1 = Clock::now();
                host_ms += std::chrono::duration<double, std::milli>(t1 - t0).count();
                if (tl) {
                    std::lock_guard<std::mutex> g(o->mu);
                    tl_push(o, j, c, 1, tl_host_ms(o, t0), tl_host_ms(o, t1));
                }
                // this chunk's parameters go back now if the caller has released
                if (send_params(o, b, c + 1, false, &sent, &gated, &wait_release) != ZERO_OK) {
                    return;
                }
            }
            applied = true;
            if (send_params(o, b, o->n_chunks, true, &sent, &gated, &wait_release) != ZERO_OK) {
                return;  // stopped, or a HIP error (recorded)
            }
            if (gated &&
                worker_hip(o, hipEventRecord(o->ev_h2d[b], o->xfer), "hipEventRecord") != ZERO_OK) {
                return;
            }
        } else if (o->n_chunks > 0) {
            // skipped: nothing reads the gradients, but buffer b is reused (or
            // freed) once this step counts as processed, so its copies must end
            tw = Clock::now();
            if (worker_hip(o, hipEventSynchronize(o->ev_d2h[b][o->n_chunks - 1]),
                           "gradient copy") != ZERO_OK) {
                return;
            }
            wait_grad += ms_since(tw);
            for (int c = 0; c < o->n_chunks; ++c) tl_d2h(c);
        }
        std::lock_guard<std::mutex> g(o->mu);
        if (gated) o->h2d_recorded[b] = true;
        if (applied) {
            o->host_ms_last = host_ms;
            o->host_ms_total += host_ms;
        }
        o->wait_submit_ms += wait_submit;
        o->wait_grad_ms += wait_grad;
        o->wait_h2d_ms += wait_h2d;
        o->wait_release_ms += wait_release;
        o->rec[b].processed = true;
        o->rec[b].applied = applied;
        o->processed = j + 1;
        o->last_flag = slot.flag;
        if (applied) o->applied += 1; else o->skipped += 1;
        o->cv.notify_all();
    }
}

int offload_error(zero_offload* o) {
    std::lock_guard<std::mutex> g(o->mu);
    if (o->err != ZERO_OK) return fail(o->err, "offload worker failed: " + o->err_msg);
    return ZERO_OK;
}

int check_device(zero_offload* o) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != o->device) return fail(ZERO_ESTATE, "offload object is bound to another device");
    return ZERO_OK;
}

// Records the release point of step j's device parameters on `s` unless
// the next submit already did.  Caller holds no lock.
int release_params(zero_offload* o, int64_t j, hipStream_t s) {
    const int b = static_cast<int>(j & 1);
    std::lock_guard<std::mutex> g(o->mu);
    if (o->rec[b].idx != j || o->rec[b].free_recorded) return ZERO_OK;
    hipError_t e = hipEventRecord(o->ev_free[b], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    o->rec[b].free_recorded = true;
    o->cv.notify_all();
    return ZERO_OK;
}

// Host wait until step j's host part is done (or an error / stop).
int wait_processed(zero_offload* o, int64_t j) {
    std::unique_lock<std::mutex> lk(o->mu);
    if (o->err == ZERO_OK && o->processed <= j) {
        const auto tw = Clock::now();
        o->cv.wait(lk, [&] { return o->err != ZERO_OK || o->processed > j; });
        o->caller_wait_ms += ms_since(tw);
    }
    if (o->err != ZERO_OK) return fail(o->err, "offload worker failed: " + o->err_msg);
    return ZERO_OK;
}

void release_all(zero_offload* o) {
    if (o->worker.joinable()) {
        {
            std::lock_guard<std::mutex> g(o->mu);
            o->stop = true;
        }
        o->cv.notify_all();
        o->worker.join();
    }
    if (o->xfer) (void)hipStreamSynchronize(o->xfer);
    delete o->pool;
    o->pool = nullptr;
    for (int b = 0; b < 2; ++b) {
        if (o->hgrad[b]) (void)hipHostFree(o->hgrad[b]);
        if (o->hparam[b]) (void)hipHostFree(o->hparam[b]);
        if (o->ev_slot[b]) (void)hipEventDestroy(o->ev_slot[b]);
        for (int c = 0; c < kMaxChunks; ++c) {
            if (o->ev_d2h[b][c]) (void)hipEventDestroy(o->ev_d2h[b][c]);
        }
        if (o->ev_free[b]) (void)hipEventDestroy(o->ev_free[b]);
        if (o->ev_h2d[b]) (void)hipEventDestroy(o->ev_h2d[b]);
    }
    if (o->tl_ref) (void)hipEventDestroy(o->tl_ref);
    for (int b = 0; b < 2; ++b) {
        for (int c = 0; c < kMaxChunks; ++c) {
            for (int k = 0; k < 2; ++k) {
                if (o->tl_d2h[b][c][k]) (void)hipEventDestroy(o->tl_d2h[b][c][k]);
                if (o->tl_h2d[b][c][k]) (void)hipEventDestroy(o->tl_h2d[b][c][k]);
            }
        }
    }
    if (o->hslot) (void)hipHostFree(o->hslot);
    if (o->dslot) (void)hipFree(o->dslot);
    if (o->xfer) (void)hipStreamDestroy(o->xfer);
}

}  // namespace

extern "C" {

int zero_offload_create(zero_plan_t* p, const zero_adam_hparams_t* hp, int32_t grad_dtype,
                        int32_t param_dtype, float* master, float* exp_avg, float* exp_avg_sq,
                        int32_t n_threads, zero_offload_t** out) {
    if (out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    *out = nullptr;
    if (p == nullptr || hp == nullptr) return fail(ZERO_ENULL, "plan or hparams is NULL");
    if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_BF16 && grad_dtype != ZERO_F32) {
        return fail(ZERO_EINVAL, "grad_dtype must be ZERO_F16, ZERO_BF16 or ZERO_F32");
    }
    if (param_dtype != 0 && param_dtype != ZERO_F16 && param_dtype != ZERO_BF16) {
        return fail(ZERO_EINVAL, "param_dtype must be 0, ZERO_F16 or ZERO_BF16");
    }
    if (n_threads < 1 || n_threads > 1024) return fail(ZERO_EINVAL, "n_threads must be in [1, 1024]");
    const int hrc = check_hparams(hp);
    if (hrc != ZERO_OK) return hrc;
    if (p->S > 0 && (master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr)) {
        return fail(ZERO_ENULL, "master, exp_avg and exp_avg_sq must be non-NULL");
    }
    if (!p->dev.ready || !p->dev.state_ready) {
        return fail(ZERO_ESTATE, "no device state: call zero_state_upload first");
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != p->dev.device) return fail(ZERO_ESTATE, "plan is bound to another device");
    zero_offload* o = new (std::nothrow) zero_offload();
    if (o == nullptr) return fail(ZERO_ENOMEM, "offload allocation failed");
    o->plan = p;
    o->hp = *hp;
    o->gdt = grad_dtype;
    o->pdt = param_dtype;
    o->master = master;
    o->m = exp_avg;
    o->v = exp_avg_sq;
    o->n_threads = n_threads;
    o->device = dev;
    // copy / update pieces: at least kMinChunkElems each (ZERO_OFFLOAD_MIN_CHUNK
    // overrides it, down to 64, so tests can cover many pieces on small
    // shards), at most kMaxChunks
    if (p->S > 0) {
        int64_t min_chunk = kMinChunkElems;
        if (const char* env = std::getenv("ZERO_OFFLOAD_MIN_CHUNK")) {
            const long long v = std::atoll(env);
            if (v >= 64) min_chunk = v;
        }
        const int64_t want = (p->S + min_chunk - 1) / min_chunk;
        const int64_t pieces = std::max<int64_t>(1, std::min<int64_t>(kMaxChunks, want));
        o->chunk = ((p->S + pieces - 1) / pieces + 63) / 64 * 64;
        o->n_chunks = static_cast<int>((p->S + o->chunk - 1) / o->chunk);
    }
    const size_t gbytes =
        static_cast<size_t>(grad_bytes(grad_dtype)) * static_cast<size_t>(p->S > 0 ? p->S : 1);
    const size_t pbytes = 2 * static_cast<size_t>(p->real > 0 ? p->real : 1);
    for (int b = 0; b < 2 && e == hipSuccess; ++b) {
        e = hipHostMalloc(reinterpret_cast<void**>(&o->hgrad[b]), gbytes, hipHostMallocDefault);
        if (e == hipSuccess) {
            e = hipHostMalloc(reinterpret_cast<void**>(&o->hparam[b]), pbytes, hipHostMallocDefault);
        }
        if (e == hipSuccess) e = hipEventCreateWithFlags(&o->ev_slot[b], hipEventDisableTiming);
        for (int c = 0; c < o->n_chunks && e == hipSuccess; ++c) {
            e = hipEventCreateWithFlags(&o->ev_d2h[b][c], hipEventDisableTiming);
        }
        if (e == hipSuccess) e = hipEventCreateWithFlags(&o->ev_free[b], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&o->ev_h2d[b], hipEventDisableTiming);
    }
    if (e == hipSuccess) {
        e = hipHostMalloc(reinterpret_cast<void**>(&o->hslot), 2 * sizeof(OffloadSlot),
                          hipHostMallocDefault);
    }
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&o->dslot), 2 * sizeof(OffloadSlot));
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&o->xfer, hipStreamNonBlocking);
    if (e != hipSuccess) {
        const int rc = hip_fail(e, "offload buffers");
        release_all(o);
        delete o;
        return rc == ZERO_EHIP && e == hipErrorOutOfMemory ? ZERO_ENOMEM : rc;
    }
    try {
        o->pool = new HostPool(n_threads);
        o->worker = std::thread(worker_main, o);
    } catch (const std::exception& ex) {
        release_all(o);
        delete o;
        return fail(ZERO_ENOMEM, std::string("worker thread: ") + ex.what());
    }
    *out = o;
    return ZERO_OK;
}

int zero_offload_submit(zero_offload_t* o, const void* flat_grad, void* param, int64_t param_base,
                        int64_t param_numel, void* stream) {
    if (o == nullptr) return fail(ZERO_ENULL, "offload is NULL");
    zero_plan* p = o->plan;
    if (p->S > 0 && flat_grad == nullptr) return fail(ZERO_ENULL, "flat_grad is NULL");
    if ((reinterpret_cast<uintptr_t>(flat_grad) & 15u) != 0) {
        return fail(ZERO_EALIGN, "flat_grad must be 16-byte aligned");
    }
    if (p->flattened_into == flat_grad && p->flattened_dtype != o->gdt) {
        return fail(ZERO_EINVAL, "flat_grad was flattened in another dtype than the offload's "
                                 "grad_dtype");
    }
    if (o->pdt != 0 && p->real > 0 && param == nullptr) {
        return fail(ZERO_ENULL, "param is NULL but the offload writes parameters");
    }
    uint16_t* param0 = nullptr;
    if (o->pdt != 0 && p->real > 0) {
        if ((reinterpret_cast<uintptr_t>(param) & 1u) != 0) {
            return fail(ZERO_EALIGN, "param must be 2-byte aligned");
        }
        if (param_base < 0 || param_numel < 0 || p->begin < param_base ||
            p->begin + p->real - param_base > param_numel) {
            return fail(ZERO_EINVAL, "param window must contain the shard's real range");
        }
        param0 = static_cast<uint16_t*>(param) + (p->begin - param_base);
    }
    int rc = check_device(o);
    if (rc != ZERO_OK) return rc;
    if ((rc = offload_error(o)) != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t i = o->submitted;
    const int b = static_cast<int>(i & 1);
    // everything enqueued so far on `s` (this step's forward and backward)
    // was computed with the parameters the previous step's update replaces
    if (i >= 1 && (rc = release_params(o, i - 1, s)) != ZERO_OK) return rc;
    // buffers b were last used by step i - 2
    if (i >= 2 && (rc = wait_processed(o, i - 2)) != ZERO_OK) return rc;
    DeviceStep* st = reinterpret_cast<DeviceStep*>(reinterpret_cast<char*>(p->dev.d_flag) +
                                                   kStateOffset);
    // the flag must cover every real gradient of this buffer, as in a device
    // step: scanned here unless the flattens since the last step covered it
    bool scanned = false;
    if ((rc = gate_flag(p, flat_grad, o->gdt, s, &scanned)) != ZERO_OK) return rc;
    hipError_t e = launch_offload_snapshot(p->dev.d_flag, st, o->dslot + b, s);
    if (e != hipSuccess) return hip_fail(e, "snapshot launch");
    e = hipMemcpyAsync(o->hslot + b, o->dslot + b, sizeof(OffloadSlot), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "slot copy");
    e = hipEventRecord(o->ev_slot[b], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    const size_t esize = static_cast<size_t>(grad_bytes(o->gdt));
    const bool tl = o->tl_on;
    for (int c = 0; c < o->n_chunks; ++c) {
        const int64_t lo = c * o->chunk;
        const int64_t hi = std::min(p->S, lo + o->chunk);
        if (tl && (e = hipEventRecord(o->tl_d2h[b][c][0], s)) != hipSuccess) {
            return hip_fail(e, "hipEventRecord");
        }
        e = hipMemcpyAsync(static_cast<char*>(o->hgrad[b]) + esize * static_cast<size_t>(lo),
                           static_cast<const char*>(flat_grad) + esize * static_cast<size_t>(lo),
                           esize * static_cast<size_t>(hi - lo), hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return hip_fail(e, "gradient copy");
        // the timeline's end event before ev_d2h: complete once the worker sees ev_d2h
        if (tl && (e = hipEventRecord(o->tl_d2h[b][c][1], s)) != hipSuccess) {
            return hip_fail(e, "hipEventRecord");
        }
        e = hipEventRecord(o->ev_d2h[b][c], s);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    {
        std::lock_guard<std::mutex> g(o->mu);
        Pending& r = o->rec[b];
        r = Pending{};
        r.idx = i;
        r.param_dst = param0;
        r.timeline = tl;
        o->submitted = i + 1;
    }
    o->cv.notify_all();
    // the flatten bookkeeping of this flat buffer is consumed
    reset_flatten_bookkeeping(p);
    return ZERO_OK;
}

int zero_offload_wait_params(zero_offload_t* o, int32_t lag, void* stream) {
    if (o == nullptr) return fail(ZERO_ENULL, "offload is NULL");
    // with one device parameter buffer, step j's copy may start once the
    // next step is submitted, so only the parameters of all steps but the
    // newest one (lag 1) or of all steps (lag 0) can be waited for safely
    if (lag != 0 && lag != 1) return fail(ZERO_EINVAL, "lag must be 0 or 1");
    int rc = check_device(o);
    if (rc != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t submitted;
    {
        std::lock_guard<std::mutex> g(o->mu);
        submitted = o->submitted;
    }
    const int64_t last = submitted - 1 - lag;  // newest step whose parameters are needed
    if (last < 0) return offload_error(o);
    // the older of the (at most two) pending steps first
    for (int64_t j = last > 0 ? last - 1 : 0; j <= last; ++j) {
        if ((rc = release_params(o, j, s)) != ZERO_OK) return rc;
        if ((rc = wait_processed(o, j)) != ZERO_OK) return rc;
    }
    // the newest H2D enqueued covers every older one (one transfer stream)
    for (int b = 0; b < 2; ++b) {
        bool wait;
        {
            std::lock_guard<std::mutex> g(o->mu);
            wait = o->h2d_recorded[b];
        }
        if (wait) {
            hipError_t e = hipStreamWaitEvent(s, o->ev_h2d[b], 0);
            if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        }
    }
    return offload_error(o);
}

int zero_offload_drain(zero_offload_t* o, void* stream) {
    if (o == nullptr) return fail(ZERO_ENULL, "offload is NULL");
    int rc = zero_offload_wait_params(o, 0, stream);
    if (rc != ZERO_OK) return rc;
    hipError_t e = hipStreamSynchronize(o->xfer);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return offload_error(o);
}

int zero_offload_stats(zero_offload_t* o, zero_offload_stats_t* out) {
    if (o == nullptr || out == nullptr) return fail(ZERO_ENULL, "offload or out is NULL");
    {
        std::lock_guard<std::mutex> g(o->mu);
        std::memset(out, 0, sizeof(*out));
        out->submitted = o->submitted;
        out->processed = o->processed;
        out->applied = o->applied;
        out->skipped = o->skipped;
        out->last_flag = o->last_flag;
        out->host_ms_last = o->host_ms_last;
        out->host_ms_total = o->host_ms_total;
        out->wait_submit_ms_total = o->wait_submit_ms;
        out->wait_grad_ms_total = o->wait_grad_ms;
        out->wait_h2d_ms_total = o->wait_h2d_ms;
        out->wait_release_ms_total = o->wait_release_ms;
        out->caller_wait_ms_total = o->caller_wait_ms;
    }
    return offload_error(o);
}

int zero_offload_timeline_start(zero_offload_t* o, int64_t capacity) {
    if (o == nullptr) return fail(ZERO_ENULL, "offload is NULL");
    if (capacity < 1 || capacity > (int64_t(1) << 24)) {
        return fail(ZERO_EINVAL, "capacity must be in [1, 2^24]");
    }
    int rc = check_device(o);
    if (rc != ZERO_OK) return rc;
    if ((rc = offload_error(o)) != ZERO_OK) return rc;
    {
        std::lock_guard<std::mutex> g(o->mu);
        if (o->processed != o->submitted) {
            return fail(ZERO_ESTATE, "steps in flight: drain the pipeline first");
        }
    }
    hipError_t e = hipSuccess;
    if (o->tl_ref == nullptr) {
        e = hipEventCreate(&o->tl_ref);
        for (int b = 0; b < 2 && e == hipSuccess; ++b) {
            for (int c = 0; c < o->n_chunks && e == hipSuccess; ++c) {
                for (int k = 0; k < 2 && e == hipSuccess; ++k) {
                    e = hipEventCreate(&o->tl_d2h[b][c][k]);
                    if (e == hipSuccess) e = hipEventCreate(&o->tl_h2d[b][c][k]);
                }
            }
        }
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    // The GPU clock tied to the host's: a reference event on the idle transfer
    // stream, polled by the host.  It completed after the last poll that
    // found it pending began (or after it was recorded) and before the first
    // poll that found it done returned; the midpoint of that window is its
    // host time.  A window over kRefWindowMs (the thread was descheduled, say)
    // is retried with a new reference event, up to kRefTries times.
    constexpr double kRefWindowMs = 0.02;
    constexpr int kRefTries = 64;
    if ((e = hipStreamSynchronize(o->xfer)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    Clock::time_point t0{};
    for (int attempt = 0; attempt < kRefTries; ++attempt) {
        auto lo = Clock::now();
        if ((e = hipEventRecord(o->tl_ref, o->xfer)) != hipSuccess) {
            return hip_fail(e, "hipEventRecord");
        }
        Clock::time_point hi{};
        for (;;) {
            const auto a = Clock::now();
            e = hipEventQuery(o->tl_ref);
            hi = Clock::now();
            if (e != hipErrorNotReady) break;
            lo = a;
        }
        if (e != hipSuccess) return hip_fail(e, "hipEventQuery");
        t0 = lo + (hi - lo) / 2;
        if (std::chrono::duration<double, std::milli>(hi - lo).count() <= kRefWindowMs) break;
    }
    std::lock_guard<std::mutex> g(o->mu);
    o->tl.clear();
    try {
        o->tl.reserve(static_cast<size_t>(std::min<int64_t>(capacity, int64_t(1) << 16)));
    } catch (const std::exception&) {
        return fail(ZERO_ENOMEM, "timeline allocation failed");
    }
    for (int b = 0; b < 2; ++b) {
        o->tl_h2d_step[b] = -1;
        for (int c = 0; c < kMaxChunks; ++c) o->tl_h2d_sent[b][c] = false;
    }
    o->tl_cap = capacity;
    o->tl_t0 = t0;
    o->tl_on = true;
    return ZERO_OK;
}

int64_t zero_offload_timeline(zero_offload_t* o, zero_offload_interval_t* out, int64_t cap) {
    if (o == nullptr) return fail(ZERO_ENULL, "offload is NULL");
    if (cap < 0) return fail(ZERO_EINVAL, "cap must be >= 0");
    if (cap > 0 && out == nullptr) return fail(ZERO_ENULL, "out is NULL");
    int rc = check_device(o);
    if (rc != ZERO_OK) return rc;
    std::lock_guard<std::mutex> g(o->mu);
    if (!o->tl_on) return fail(ZERO_ESTATE, "no timeline was started");
    // parameter copies not read yet: those already complete
    for (int b = 0; b < 2; ++b) tl_read_h2d(o, b);
    const int64_t n = std::min<int64_t>(cap, static_cast<int64_t>(o->tl.size()));
    if (n > 0) std::memcpy(out, o->tl.data(), static_cast<size_t>(n) * sizeof(*out));
    return static_cast<int64_t>(o->tl.size());
}

void zero_offload_destroy(zero_offload_t* o) {
    if (o == nullptr) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != o->device) (void)hipSetDevice(o->device);
    // let the worker finish what was submitted, then stop it; if a release
    // point cannot be recorded, stop it at once (it would wait for that
    // release forever)
    {
        std::unique_lock<std::mutex> lk(o->mu);
        for (int b = 0; b < 2; ++b) {
            if (o->rec[b].idx >= 0 && !o->rec[b].free_recorded) {
                if (hipEventRecord(o->ev_free[b], nullptr) == hipSuccess) {
                    o->rec[b].free_recorded = true;
                } else {
                    o->stop = true;
                }
            }
        }
        o->cv.notify_all();
        o->cv.wait(lk, [&] {
            return o->stop || o->err != ZERO_OK || o->processed >= o->submitted;
        });
    }
    release_all(o);
    if (cur != o->device && cur >= 0) (void)hipSetDevice(cur);
    delete o;
}

}  // extern "C"
