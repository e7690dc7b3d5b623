// Internal declarations shared by the host planner, the ABI layer and the
// HIP kernels of libzero_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "zero_mi355x.h"

namespace zmi {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

// ---------------------------------------------------------------- plan
struct Segment {
    int64_t tensor;
    int64_t tensor_off;
    int64_t shard_off;
    int64_t numel;
    int32_t bucket;
};

enum Timer { kTimerFlatten = 0, kTimerScan = 1, kTimerAdam = 2, kTimerWrite = 3, kTimers = 4 };

struct DeviceState {
    bool ready = false;
    int device = -1;
    int* d_flag = nullptr;      // device overflow flag (256 B allocation)
    int* h_flag = nullptr;      // pinned host mirror
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

// ---------------------------------------------------------------- kernels
// One contiguous piece of the flat destination and where its source is:
// element d of the flat shard (begin <= d < end) comes from
// src_base + 2*d bytes, or is zero when src_base == 0.
struct FlatPiece {
    int64_t begin;
    int64_t end;
    uintptr_t src_base;
};

constexpr int kMaxPiecesPerLaunch = 64;

struct AdamScalars {
    float inv_scale, b1, omb1, b2, omb2, step, rsbc2, eps, decay, wd;
};

hipError_t launch_flatten(const FlatPiece* pieces, int n, uint16_t* flat, int* flag,
                          int grad_dtype, hipStream_t s);
hipError_t launch_scan(const uint16_t* flat, int64_t n, int* flag, int grad_dtype, hipStream_t s);
hipError_t launch_adam(const uint16_t* g, float* master, float* m, float* v, uint16_t* param_at_0,
                       int64_t S, int64_t real, const int* flag, const AdamScalars& sc,
                       int grad_dtype, int param_dtype, bool adamw, hipStream_t s);
hipError_t launch_write_param(const float* master, uint16_t* param_at_0, int64_t real,
                              int param_dtype, hipStream_t s);
hipError_t launch_flag_clear(int* flag, hipStream_t s);

}  // namespace zmi
