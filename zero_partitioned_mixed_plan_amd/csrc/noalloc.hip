// zero_adam_step_noalloc: the gated update of zero_adam_step for callers
// that cannot allocate (code under HIP graph capture, serving loops that
// forbid allocation).  Its overflow accumulator lives in a file-scope device
// array instead of the plan's device block, so the call never creates
// anything: it launches kernels on the caller's stream and returns.
#include <mutex>

#include "internal.h"

namespace zmi {
namespace {

// Scratch of the allocation-free step, one copy per device for the life of
// the process: word 0 is the overflow accumulator of the call in flight.
// The call needs kNoAllocWords of it whatever the shard size.
constexpr int kScratchWords = 64;  // 256 bytes
constexpr int kNoAllocWords = 1;
static_assert(kNoAllocWords <= kScratchWords, "scratch too small for the step");
static __device__ __align__(256) int scratch[kScratchWords];

// Device address of `scratch` on each device (the host-side name is only a
// stand-in), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int* g_scratch[kMaxDevices] = {};

int scratch_address(int dev, int** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr) return fail(ZERO_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch[dev] = static_cast<int*>(ptr);
    }
    *out = g_scratch[dev];
    return ZERO_OK;
}

// One thread, after the update: the call's flag to the caller's output and,
// when the plan has a device block, that block's flag cleared (this step
// consumed whatever the flattens since the last step had found).
__global__ void noalloc_finish_kernel(const int* __restrict__ acc, int32_t* __restrict__ out,
                                      int* __restrict__ plan_flag) {
    const int32_t f = *acc != 0 ? 1 : 0;
    *out = f;
    if (plan_flag != nullptr) *plan_flag = 0;
}

}  // namespace
}  // namespace zmi

using namespace zmi;

extern "C" int zero_adam_step_noalloc(zero_plan_t* p, const zero_adam_hparams_t* hp, int64_t step,
                                      double loss_scale, const void* flat_grad,
                                      int32_t grad_dtype, float* master, float* exp_avg,
                                      float* exp_avg_sq, void* param, int64_t param_base,
                                      int64_t param_numel, int32_t param_dtype,
                                      int32_t* overflow_out, void* stream) {
    if (p == nullptr || hp == nullptr) return fail(ZERO_ENULL, "plan or hparams is NULL");
    if (overflow_out == nullptr) return fail(ZERO_ENULL, "overflow_out is NULL");
    if (!aligned4(overflow_out)) return fail(ZERO_EALIGN, "overflow_out must be 4-byte aligned");
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
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(ZERO_ESTATE, "device ordinal out of range");
    DeviceState& d = p->dev;
    if (d.ready && d.device != dev) {
        return fail(ZERO_ESTATE, "the plan is bound to another device than the current one");
    }
    int* acc = nullptr;
    if ((rc = scratch_address(dev, &acc)) != ZERO_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // scalars formed on the host in double, each rounded once to fp32
    const AdamScalars sc = make_scalars(hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay,
                                        hp->adamw, static_cast<double>(step), loss_scale);
    // the accumulator starts at zero (a fill kernel, not a memset), the scan
    // of the real gradients raises it, the update is gated on it
    if ((e = launch_flag_clear(acc, s)) != hipSuccess) return hip_fail(e, "scratch clear");
    if ((e = launch_scan(flat_grad, p->real, acc, grad_dtype, s)) != hipSuccess) {
        return hip_fail(e, "scan launch");
    }
    e = launch_adam(flat_grad, master, exp_avg, exp_avg_sq, param0, p->S, p->real, acc, sc,
                    nullptr, grad_dtype, param_dtype, hp->adamw != 0, s);
    if (e != hipSuccess) return hip_fail(e, "adam launch");
    int* plan_flag = d.ready ? d.d_flag : nullptr;
    hipLaunchKernelGGL(noalloc_finish_kernel, dim3(1), dim3(1), 0, s, acc, overflow_out,
                       plan_flag);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "finish launch");
    if (d.ready) d.flag_cleared = true;
    reset_flatten_bookkeeping(p);
    return ZERO_OK;
}
