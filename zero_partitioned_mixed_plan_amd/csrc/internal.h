// Internal declarations shared by the host planner, the ABI layer and the
// HIP kernels of libzero_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "zero_mi355x.h"

namespace zmi {

// ---------------------------------------------------------------- errors
// The message goes to a fixed per-thread buffer (setting it never allocates).
void set_error(const char* msg);
void set_error(const std::string& msg);
int fail(int code, const char* msg);
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);
// ZERO_OK, or ZERO_EINVAL (with the message set) for hyperparameters out of
// range: lr >= 0, 0 <= betas < 1, eps > 0, weight_decay >= 0, all finite.
int check_hparams(const zero_adam_hparams_t* hp);

// ---------------------------------------------------------------- plan
struct Segment {
    int64_t tensor;
    int64_t tensor_off;
    int64_t shard_off;
    int64_t numel;
    int32_t bucket;
};

enum Timer { kTimerFlatten = 0, kTimerScan = 1, kTimerAdam = 2, kTimerWrite = 3, kTimers = 4 };

// Loss-scale and step-count state of the asynchronous step, kept in device
// memory so that a whole step needs no host round trip.
struct DeviceStep {
    int64_t t;        // applied (not skipped) steps so far
    int64_t skipped;  // skipped steps so far
    double scale;
    double min_scale;
    double backoff;
    double growth;
    int32_t window;
    int32_t good_steps;
    int32_t dynamic;
    int32_t last_flag;  // flag of the last asynchronous step (1 = skipped)
};

struct AdamScalars {
    float inv_scale, b1, omb1, b2, omb2, step, rsbc2, eps, decay, wd;
};
static_assert(sizeof(AdamScalars) == 10 * sizeof(float), "scalars are ten packed floats");

// What an offloaded step needs from the device: its overflow flag, its
// bias-correction step and the loss scale its gradients carry.
struct OffloadSlot {
    int32_t flag;
    int32_t _pad;
    int64_t t;
    double scale;
};

// The loss-scale policy of zero_update_loss_scale on the device state
// (also advances t or the skip count).
__host__ __device__ inline void apply_scale_policy(DeviceStep& d, int overflow) {
    if (overflow) {
        if (d.dynamic) {
            const double s = d.scale * d.backoff;
            d.scale = s < d.min_scale ? d.min_scale : s;
        }
        d.good_steps = 0;
        d.skipped += 1;
    } else {
        d.t += 1;
        d.good_steps += 1;
        if (d.dynamic && d.good_steps >= d.window) {
            d.scale *= d.growth;
            d.good_steps = 0;
        }
    }
    d.last_flag = overflow;
}

// The plan's device block (one 256-byte allocation): the overflow flag, the
// asynchronous step state and the update scalars formed on the device.
constexpr size_t kBlockBytes = 256;
constexpr size_t kStateOffset = 64;
constexpr size_t kScalarsOffset = 128;
static_assert(kStateOffset + sizeof(DeviceStep) <= kScalarsOffset, "device block layout");
static_assert(kScalarsOffset + sizeof(AdamScalars) <= kBlockBytes, "device block layout");

// The update's fp32 scalars for bias-correction step t and loss scale
// `scale`: formed in double, each rounded once to fp32.  The same function
// serves the host (synchronous step) and the device (asynchronous step).
__host__ __device__ inline AdamScalars make_scalars(double lr, double beta1, double beta2,
                                                    double eps, double weight_decay, int adamw,
                                                    double t, double scale) {
    AdamScalars sc;
    sc.inv_scale = static_cast<float>(1.0 / scale);
    sc.b1 = static_cast<float>(beta1);
    sc.omb1 = static_cast<float>(1.0 - beta1);
    sc.b2 = static_cast<float>(beta2);
    sc.omb2 = static_cast<float>(1.0 - beta2);
    sc.step = static_cast<float>(lr / (1.0 - pow(beta1, t)));
    sc.rsbc2 = static_cast<float>(1.0 / sqrt(1.0 - pow(beta2, t)));
    sc.eps = static_cast<float>(eps);
    sc.decay = adamw ? static_cast<float>(1.0 - lr * weight_decay) : 1.0f;
    sc.wd = static_cast<float>(weight_decay);
    return sc;
}

struct DeviceState {
    bool ready = false;
    bool flag_cleared = false;  // the flag's clear is enqueued (on the first call's stream)
    bool state_ready = false;   // zero_state_upload has run
    int device = -1;
    int* d_flag = nullptr;      // device block: overflow flag at offset 0
    int* h_flag = nullptr;      // pinned host mirror of the device block
    bool timing = false;
    hipEvent_t ev_start[kTimers] = {};
    hipEvent_t ev_stop[kTimers] = {};
    bool timed[kTimers] = {};
};

}  // namespace zmi

struct zero_plan {
    // sizes
    int64_t P = 0, P_pad = 0, S = 0, begin = 0, real = 0;
    int64_t align = 1, bucket_elems = 1;
    int32_t R = 1, r = 0;
    std::vector<int64_t> numels;
    std::vector<int32_t> tensor_bucket;
    int32_t n_buckets = 0;
    std::vector<zmi::Segment> segs;          // shard order
    // per-bucket segment ranges [first, last) in segs (buckets hold
    // contiguous tensor ranges, so their segments are contiguous too)
    std::vector<int64_t> bucket_seg_first, bucket_seg_last;
    // flatten bookkeeping for the gate of zero_adam_step
    std::vector<uint8_t> bucket_flattened;
    const void* flattened_into = nullptr;
    int32_t flattened_dtype = 0;
    bool flatten_all_done = false;
    zmi::DeviceState dev;
};

namespace zmi {

int build_plan(const int64_t* numels, int32_t n, int32_t R, int32_t r, int64_t A, int64_t B,
               zero_plan* p);

// The gate of a step (or an offloaded step) on flat_grad: whether the
// flattens since the last step covered every bucket of that buffer in that
// dtype; if not, gate_flag clears the flag and scans the real elements on
// `s` (*scanned = true).  reset_flatten_bookkeeping marks the flag consumed.
bool flatten_covered(const zero_plan* p, const void* flat_grad, int32_t grad_dtype);
int gate_flag(zero_plan* p, const void* flat_grad, int32_t grad_dtype, hipStream_t s,
              bool* scanned);
void reset_flatten_bookkeeping(zero_plan* p);

// Argument checks shared by the entry points (ZERO_OK, or the error code
// with the message set).
bool aligned16(const void* p);
bool aligned4(const void* p);
bool valid_dtype(int32_t d);
bool valid_grad_dtype(int32_t d);
int bad_grad_dtype();
// *out = the parameter destination of shard element 0 (nullptr when param
// is NULL or the shard holds only padding), after checking the window.
int param_target(const zero_plan* p, void* param, int64_t base, int64_t numel, int32_t dtype,
                 uint16_t** out);
int check_step_buffers(const zero_plan* p, const void* flat_grad, int32_t grad_dtype,
                       const float* master, const float* exp_avg, const float* exp_avg_sq);

// ---------------------------------------------------------------- kernels
// One contiguous piece of the flat destination and where its source is:
// element d of the flat shard (begin <= d < end) comes from
// src_base + esize*d bytes (esize 2 for half gradients, 4 for fp32 ones),
// or is zero when src_base == 0.
struct FlatPiece {
    int64_t begin;
    int64_t end;
    uintptr_t src_base;
};

constexpr int kMaxPiecesPerLaunch = 96;

hipError_t launch_flatten(const FlatPiece* pieces, int n, void* flat, int* flag, int grad_dtype,
                          hipStream_t s);
hipError_t launch_scan(const void* flat, int64_t n, int* flag, int grad_dtype, hipStream_t s);
// sc_dev == nullptr: the update uses the scalars passed by value in sc;
// otherwise it reads them from device memory at sc_dev.
hipError_t launch_adam(const void* g, float* master, float* m, float* v, uint16_t* param_at_0,
                       int64_t S, int64_t real, const int* flag, const AdamScalars& sc,
                       const AdamScalars* sc_dev, int grad_dtype, int param_dtype, bool adamw,
                       hipStream_t s);
hipError_t launch_write_param(const float* master, uint16_t* param_at_0, int64_t real,
                              int param_dtype, hipStream_t s);
hipError_t launch_flag_clear(int* flag, hipStream_t s);
// Asynchronous step: the prologue forms the scalars of step t + 1 from the
// device state (skipped when the flag is raised); the epilogue applies the
// loss-scale policy, advances t or the skip count, and clears the flag.
hipError_t launch_step_prologue(const int* flag, const DeviceStep* st, AdamScalars* out,
                                const zero_adam_hparams_t& hp, hipStream_t s);
hipError_t launch_step_epilogue(int* flag, DeviceStep* st, hipStream_t s);
// The scalars the prologue would form for steps t_first .. t_first + count
// - 1 at loss scale `scale`, into out[0 .. count) (device memory).
hipError_t launch_adam_scalars(const zero_adam_hparams_t& hp, int64_t t_first, int64_t count,
                               double scale, AdamScalars* out, hipStream_t s);
// Offloaded step: snapshot (flag, t + 1, scale) into *slot, apply the
// loss-scale policy to the device state, clear the flag.
hipError_t launch_offload_snapshot(int* flag, DeviceStep* st, OffloadSlot* slot, hipStream_t s);

// ---------------------------------------------------------------- host Adam
enum class CpuIsa { kScalar = 0, kAvx2 = 1, kAvx512 = 2 };

// One host update over shard elements [0, n): the arithmetic of the device
// update.  param points at shard element 0's destination (nullptr: no
// parameter write); elements k >= real are never written to it.
struct CpuAdamArgs {
    const void* g;  // n gradients of dtype gdt (2 or 4 bytes each)
    float* p;
    float* m;
    float* v;
    uint16_t* param;
    int64_t n;
    int64_t real;
    AdamScalars sc;
    int gdt;
    int pdt;
    bool adamw;
};

// A fixed set of host threads that runs one job at a time: run(fn) calls
// fn(i) for i in [0, size()) -- i = 0 on the calling thread -- and returns
// when all have finished.  One caller at a time.  Idle threads (and a
// waiting caller) spin for a short while before sleeping, so jobs that come
// back to back do not pay a wake-up each; an oversubscribed pool does not spin.
class HostPool {
public:
    explicit HostPool(int n_threads);
    ~HostPool();
    HostPool(const HostPool&) = delete;
    HostPool& operator=(const HostPool&) = delete;
    int size() const { return n_; }
    void run(const std::function<void(int)>& fn);

private:
    void worker(int idx);
    int n_;
    std::chrono::nanoseconds spin_;
    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable go_, done_;
    std::atomic<const std::function<void(int)>*> job_{nullptr};
    std::atomic<uint64_t> gen_{0};
    std::atomic<int> pending_{0};
    std::atomic<bool> stop_{false};
};

CpuIsa cpu_isa();
const char* cpu_isa_name(CpuIsa isa);
// pool == nullptr: n_threads threads are started for this call.
void cpu_adam(const CpuAdamArgs& a, int n_threads, HostPool* pool = nullptr);
bool cpu_nonfinite(const void* g, int64_t n, int gdt, int n_threads, HostPool* pool = nullptr);

// Bytes per gradient element.
inline int grad_bytes(int gdt) { return gdt == ZERO_F32 ? 4 : 2; }

}  // namespace zmi
