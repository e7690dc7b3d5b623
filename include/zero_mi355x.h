/*
 * zero_mi355x.h -- C ABI of one data-parallel rank's share of ZeRO's
 * partitioned mixed-precision Adam step, on one AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on ZeRO, cited by page title and paragraph topic):
 *   [legal]   "ZeRO Optimization", inferensys glossary, domain-specific
 *             legal pre-training page
 *   [instr]   "ZeRO Optimization", inferensys glossary, instruction-tuning
 *             methodologies page
 *   [genomic] "ZeRO Optimization", inferensys glossary, genomic MLOps page
 *
 * The step of rank r of R, per call:
 *   zero_partition_plan     flat partition + bucket plan (host only)
 *   zero_flatten_grads      gradients -> the rank's flat gradient shard,
 *                           with the inf/NaN test fused into the copy
 *   zero_adam_step          unscale + Adam/AdamW + cast back to half, gated
 *                           on the overflow flag; returns the flag
 *   zero_update_loss_scale  dynamic loss-scale policy (host only)
 *   zero_write_param_shard  fp32 master shard -> half params at its offset
 *
 * and the same step without host round trips, for HIP graph capture:
 *   zero_state_upload       step count and loss scaler -> device state
 *   zero_adam_step_async    gated update + cast + loss-scale policy, all on
 *                           the device state; never waits
 *   zero_state_download     device state -> host (waits)
 *   zero_state_device_scale device address of the current loss scale
 *
 * Conventions
 *   Errors   every call returns an int: 0 (ZERO_OK) or a negative ZERO_E*
 *            code; zero_adam_step returns 0 (applied) or 1 (overflow,
 *            skipped).  A message for the last error of the calling thread
 *            is available from zero_last_error().
 *   Memory   the caller allocates and owns every device buffer and stream.
 *            The plan owns only its host tables, a 256-byte device block
 *            (overflow flag, asynchronous step state, update scalars) and
 *            its pinned host mirror, created on the first device call and
 *            released by zero_plan_destroy.  Buffers are not retained
 *            between calls.
 *   Streams  all device work is enqueued on the caller's stream (a
 *            hipStream_t passed as void*; NULL means the default stream).
 *            zero_adam_step waits for its own stream to read the flag back,
 *            and so do zero_state_upload and zero_state_download; nothing
 *            else waits.
 *   Devices  a plan binds to the device that is current at its first device
 *            call; later device calls must run with that device current.
 *   Threads  a plan is not thread safe; distinct plans are independent.
 *   Layout   element counts, offsets and indices are int64 elements, not
 *            bytes.  Tensors are concatenated in registration order into
 *            one flat index space [0, P).
 *   Dtypes   gradients and parameters are fp16 (ZERO_F16) or bf16
 *            (ZERO_BF16); master weights and both moments are fp32.
 *            Gradients may also be kept in fp32 (ZERO_F32, e.g. an
 *            accumulation buffer; the pages describe half gradients only):
 *            they are flattened, tested and read as they are, 4 bytes per
 *            element.  Parameters are always fp16 or bf16.
 */
#ifndef ZERO_MI355X_H
#define ZERO_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zero_plan zero_plan_t; /* opaque, library owned */

enum zero_dtype { ZERO_F16 = 1, ZERO_BF16 = 2, ZERO_F32 = 3 /* gradients only */ };

enum zero_status {
    ZERO_OK = 0,
    ZERO_EINVAL = -1, /* bad argument value */
    ZERO_EALIGN = -2, /* a buffer is not aligned as required */
    ZERO_ENULL = -3,  /* a required pointer is NULL */
    ZERO_EHIP = -4,   /* the HIP runtime reported an error */
    ZERO_ENOMEM = -5, /* host or device allocation failed */
    ZERO_ESTATE = -6  /* call not valid in the plan's state (e.g. wrong device) */
};

/* One tensor's part of the rank's shard: elements
 * [tensor_off, tensor_off + numel) of tensor `tensor` sit at
 * [shard_off, shard_off + numel) of the shard; `bucket` is the tensor's
 * bucket. */
typedef struct {
    int64_t tensor;
    int64_t tensor_off;
    int64_t shard_off;
    int64_t numel;
    int32_t bucket;
    int32_t _pad;
} zero_segment_t;

typedef struct {
    int64_t total_numel;  /* P: sum of tensor sizes */
    int64_t padded_numel; /* P_pad: P rounded up to a multiple of R * align */
    int64_t shard_numel;  /* S = P_pad / R: elements of every rank's shard */
    int64_t shard_begin;  /* r * S: flat index of the shard's first element */
    int64_t real_numel;   /* elements of the shard below P (the rest is padding) */
    int64_t align_elems;
    int64_t bucket_elems;
    int64_t bytes_stage1; /* 4 P + 12 S  (optimizer states partitioned)       */
    int64_t bytes_stage2; /* 2 P + 14 S  (+ gradients partitioned)            */
    int64_t bytes_stage3; /* 16 S        (+ parameters partitioned)           */
    int32_t world_size;
    int32_t rank;
    int32_t n_tensors;
    int32_t n_segments;
    int32_t n_buckets;
    int32_t _pad;
} zero_plan_info_t;

typedef struct {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int32_t adamw; /* 1: decoupled decay (AdamW); 0: L2 term added to the gradient */
    int32_t _pad;
} zero_adam_hparams_t;

typedef struct {
    double scale;     /* current loss scale (> 0) */
    double min_scale; /* floor for backoff (> 0) */
    double backoff;   /* factor on overflow, in (0, 1] (0.5: halve) */
    double growth;    /* factor after `window` clean steps, >= 1 (2: double) */
    int32_t window;   /* clean steps before growth, >= 1 */
    int32_t good_steps;
    int32_t dynamic;  /* 0: static scale (bf16 needs none) */
    int32_t _pad;
} zero_scaler_t;

/* Partition plan.  [instr] ZeRO-1 mechanism and memory reduction: each of
 * the R data-parallel ranks owns one partition and updates only it;
 * [genomic] memory breakdown: per-rank memory is the total divided by R.
 * [legal] bandwidth bullet / [genomic] overlap paragraph: small tensors are
 * fused into buckets.
 *   P_pad = ceil(P / (R*align)) * R*align, S = P_pad / R, rank r owns the
 *   contiguous flat range [r*S, (r+1)*S).  Buckets are formed from the last
 *   tensor to the first, whole tensors only, each closed once it holds at
 *   least bucket_elems elements; bucket 0 holds the last tensor.
 * numels: host array of n_tensors sizes (>= 0; zero-size tensors allowed).
 * world_size >= 1, 0 <= rank < world_size, align_elems >= 1 (64 keeps every
 * shard 256-byte aligned in fp32), bucket_elems >= 1.
 * Host only: needs no GPU.  *out receives a new plan (free with
 * zero_plan_destroy).  Errors: ZERO_ENULL, ZERO_EINVAL, ZERO_ENOMEM. */
int zero_partition_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size,
                        int32_t rank, int64_t align_elems, int64_t bucket_elems,
                        zero_plan_t** out);

/* Sizes and byte accounting of a plan (host only). */
int zero_plan_info(const zero_plan_t* plan, zero_plan_info_t* out);

/* Copies up to `cap` segments, in shard order, into `out` (host memory) and
 * returns the plan's segment count (>= 0) or a negative error. */
int64_t zero_plan_segments(const zero_plan_t* plan, zero_segment_t* out, int64_t cap);

/* Writes the bucket id of each of the first min(cap, n_tensors) tensors. */
int zero_plan_tensor_buckets(const zero_plan_t* plan, int32_t* out, int64_t cap);

/* Releases the plan, its device block and pinned mirror (NULL is a no-op). */
void zero_plan_destroy(zero_plan_t* plan);

/* Bucketed flatten of the gradients into the rank's flat shard.
 * [legal] ZeRO-2 bullet / [instr] ZeRO-2 mechanism: a rank keeps only the
 * gradients of its partition.  For every segment of `bucket` (0 <= bucket
 * < n_buckets) or of all buckets (bucket = -1):
 *   flat_grad[shard_off + k] = grads[tensor][tensor_off + k]   (bit copy)
 * and flat_grad[real, S) = 0 on every call.  While copying, any element
 * whose exponent field is all ones (+-inf or NaN) raises the plan's device
 * overflow flag ([legal] dynamic loss scaling bullet); the flag stays
 * raised until the next step on this plan consumes it.  The flag belongs to
 * one buffer: a flatten into another flat_grad (or in another dtype) than
 * the previous flattens since the last step clears it first.
 * grads: HOST array of n_tensors DEVICE pointers, each to tensor i's first
 * element, aligned to the element size (2 bytes; 4 for ZERO_F32); entries
 * of tensors without a segment in the requested bucket(s) may be NULL.
 * grad_dtype: ZERO_F16, ZERO_BF16 or ZERO_F32.  flat_grad: device, >= S
 * elements of grad_dtype, 16-byte aligned.  Async on `stream`.
 * Errors: ZERO_ENULL, ZERO_EINVAL (bucket, dtype), ZERO_EALIGN, ZERO_EHIP,
 * ZERO_ESTATE (wrong device). */
int zero_flatten_grads(zero_plan_t* plan, int32_t bucket, const void* const* grads,
                       int32_t grad_dtype, void* flat_grad, void* stream);

/* Declares that the flat gradient buffer was written after the flattens
 * since the last step (for example averaged in place): the next step (or
 * offloaded step) on this plan then clears the flag and scans the buffer's
 * real elements instead of trusting the flattens' fused test.  Host only;
 * no device work.  Errors: ZERO_ENULL. */
int zero_flatten_invalidate(zero_plan_t* plan);

/* One gated Adam/AdamW step on the shard, with the half cast fused in.
 * [genomic] memory breakdown / [instr] ZeRO-1 mechanism: fp32 master
 * weights, momentum and variance of the partition, updated by their owner;
 * [instr] mixed-precision bullets: the gradient is scaled down and upcast
 * to fp32 for the update, and the weights are cast to fp16/bf16.
 * If the flag is raised, nothing is written and 1 is returned.  The flag
 * is the fused test of the flattens into this flat_grad since the last step
 * when they covered every bucket of the shard; otherwise the flag is cleared
 * and a scan of flat_grad's real elements [0, real) decides it (the gate
 * reads the buffer as it is when the step runs: a write into flat_grad
 * after a covering flatten is not tested again unless the caller declares
 * it with zero_flatten_invalidate).  The padding gradients
 * flat_grad[real, S) are never tested: they update only the padding state,
 * which is never cast to a parameter.  Otherwise, per shard element k < S, in
 * fp32 with one rounding per operation (scalars formed on the host in
 * double and rounded once):
 *   g = fp32(flat_grad[k]) * fp32(1/loss_scale)  [adamw=0: g += wd * p]
 *   m = b1*m + (1-b1)*g ;  v = b2*v + (1-b2)*(g*g)
 *   d = sqrt(v) * fp32(1/sqrt(1-b2^t)) + eps ;  u = m / d
 *   p = p * fp32(1 - lr*wd [adamw] or 1) - fp32(lr/(1-b1^t)) * u
 * and, if param != NULL, for k < real:
 *   param[shard_begin + k - param_base] = round_to_nearest_even_half(p)
 * step: the bias-correction step t >= 1 (count applied steps only).
 * loss_scale: finite, > 0.  flat_grad: device, >= S elements of grad_dtype
 * (ZERO_F16, ZERO_BF16 or ZERO_F32), 16-byte aligned.  master/exp_avg/exp_avg_sq: device fp32 arrays of >= S
 * elements, 4-byte aligned (for full bandwidth: all five arrays at the same
 * offset within a 4 KB page, as separate hipMalloc / torch allocations give
 * them -- on MI355X an array starting 12 bytes past a 128-byte line ran the
 * update at 57% of peak instead of 81%, and arrays 256 or 768 bytes apart
 * within a page 3-5% slower).  param: device buffer holding flat
 * indices [param_base, param_base + param_numel), which must contain
 * [shard_begin, shard_begin + real); 2-byte aligned.
 * Returns 0 applied, 1 skipped, or a negative error (ZERO_ENULL,
 * ZERO_EINVAL, ZERO_EALIGN, ZERO_EHIP, ZERO_ESTATE).  Waits for `stream`. */
int zero_adam_step(zero_plan_t* plan, const zero_adam_hparams_t* hp, int64_t step,
                   double loss_scale, const void* flat_grad, int32_t grad_dtype, float* master,
                   float* exp_avg, float* exp_avg_sq, void* param, int64_t param_base,
                   int64_t param_numel, int32_t param_dtype, void* stream);

/* Dynamic loss scale, host only.  [legal] dynamic loss scaling bullet: the
 * scale adjusts itself; [instr] loss-scaling bullet: scaled up before
 * backward, down before the update; [legal] bfloat16 bullet: bf16 needs no
 * loss scaling (use dynamic = 0).
 *   overflow != 0: scale = max(scale * backoff, min_scale) (if dynamic),
 *                  good_steps = 0
 *   overflow == 0: good_steps += 1; if dynamic and good_steps >= window:
 *                  scale *= growth, good_steps = 0
 * Errors: ZERO_ENULL, ZERO_EINVAL (non-finite or non-positive fields). */
int zero_update_loss_scale(zero_scaler_t* scaler, int32_t overflow);

/* Standalone cast of the fp32 master shard to half parameters at the
 * rank's offset ([instr] mixed-precision bullet: weights are cast to
 * FP16/BF16): param[shard_begin + k - param_base] = rne_half(master[k]) for
 * k < real; padding is never written.  Arguments as in zero_adam_step.
 * Fastest (16-byte loads, 8-byte stores) when master is 16-byte aligned and
 * the shard's first parameter, param + (shard_begin - param_base), is 8-byte
 * aligned; any other 4-byte / 2-byte alignment gives the same bits about 7%
 * slower.  Async on `stream`. */
int zero_write_param_shard(zero_plan_t* plan, const float* master, void* param,
                           int64_t param_base, int64_t param_numel, int32_t param_dtype,
                           void* stream);

/* ------------------------------------------------------------------------
 * The step without host round trips.  The step count t and the loss scaler
 * live in the plan's device block, so that zero_flatten_grads followed by
 * zero_adam_step_async can be recorded once into a HIP graph (stream
 * capture) and replayed every step: nothing in them allocates, waits or
 * issues a memset.  The arithmetic is that of zero_adam_step and
 * zero_update_loss_scale; only the bias-correction scalars are formed on
 * the device (in double, rounded once to fp32, with the device's pow and
 * sqrt instead of the host C library's).
 * ---------------------------------------------------------------------- */

/* Loads the device state: applied_steps = steps applied so far (the next
 * applied step uses t = applied_steps + 1), the scaler's fields, and zero
 * skipped steps.  Creates the plan's device block if needed.  Waits for
 * `stream`.  Call it before capturing a graph that contains the plan.
 * Errors: ZERO_ENULL, ZERO_EINVAL (negative count, scaler fields out of
 * range), ZERO_EHIP, ZERO_ESTATE. */
int zero_state_upload(zero_plan_t* plan, int64_t applied_steps, const zero_scaler_t* scaler,
                      void* stream);

/* Reads the device state back after the work queued on `stream` (waits):
 * applied steps, the scaler (all fields), the flag of the last asynchronous
 * step (1 = skipped) and the number of skipped steps since the upload.  Any
 * output pointer may be NULL.  Errors: ZERO_ENULL, ZERO_ESTATE (no upload
 * yet), ZERO_EHIP. */
int zero_state_download(zero_plan_t* plan, int64_t* applied_steps, zero_scaler_t* scaler,
                        int32_t* last_flag, int64_t* skipped_steps, void* stream);

/* Device address of the current loss scale (a double in the plan's device
 * block), for scaling the loss on the device before backward ([instr]
 * loss-scaling bullet).  It changes only inside zero_adam_step_async.
 * Errors: ZERO_ENULL, ZERO_ESTATE (no upload yet). */
int zero_state_device_scale(zero_plan_t* plan, const double** out);

/* zero_adam_step with the step count and the loss scale taken from the
 * device state, followed on the device by the policy of
 * zero_update_loss_scale:
 *   flag clear: scalars of step t + 1 at the current scale, the update and
 *               cast exactly as zero_adam_step, then t += 1 and the
 *               clean-step count / growth rule;
 *   flag set:   nothing written, scale = max(scale * backoff, min_scale)
 *               when dynamic, clean-step count reset, skipped += 1;
 * then the flag is cleared.  The scan of flat_grad runs first under the
 * same rule as in zero_adam_step.  Arguments as in zero_adam_step.  Never
 * waits and never allocates; returns 0 once the work is enqueued.  Calls
 * on one plan must be ordered (one stream).  Errors: ZERO_ENULL,
 * ZERO_EINVAL, ZERO_EALIGN, ZERO_EHIP, ZERO_ESTATE (no zero_state_upload
 * yet, or wrong device). */
int zero_adam_step_async(zero_plan_t* plan, const zero_adam_hparams_t* hp, const void* flat_grad,
                         int32_t grad_dtype, float* master, float* exp_avg, float* exp_avg_sq,
                         void* param, int64_t param_base, int64_t param_numel,
                         int32_t param_dtype, void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate: code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc.
 * ---------------------------------------------------------------------- */

/* zero_adam_step with nothing allocated, created or waited for, by the call
 * or by the plan.  Its overflow accumulator is a 256-byte device array of
 * the library (one copy per device, held until the process ends); the call
 * uses 4 bytes of it whatever the shard size, so no shard is rejected for
 * its size.  Enqueued on `stream`: a kernel clears the accumulator, a scan
 * of flat_grad's real elements [0, real) raises it on any inf/NaN, the
 * update and cast of zero_adam_step run gated on it (same host scalars,
 * same order, same rounding), and a one-thread kernel writes 1 (skipped) or
 * 0 (applied) to *overflow_out.  It always scans: what zero_flatten_grads
 * found since the last step is consumed unused, as a step would consume it
 * (the plan's flag, if the plan has its device block, is cleared).
 * overflow_out: DEVICE memory, 4-byte aligned, valid once `stream` reaches
 * the end of the call.  Other arguments as in zero_adam_step.  Returns 0
 * once the work is enqueued.  All calls on one device share the array: two
 * calls that overlap in time on one device (other streams, other threads)
 * race.  Errors: ZERO_ENULL, ZERO_EINVAL, ZERO_EALIGN, ZERO_EHIP,
 * ZERO_ESTATE (the plan is bound to another device). */
int zero_adam_step_noalloc(zero_plan_t* plan, const zero_adam_hparams_t* hp, int64_t step,
                           double loss_scale, const void* flat_grad, int32_t grad_dtype,
                           float* master, float* exp_avg, float* exp_avg_sq, void* param,
                           int64_t param_base, int64_t param_numel, int32_t param_dtype,
                           int32_t* overflow_out, void* stream);

/* ------------------------------------------------------------------------
 * ZeRO-Offload: the rank's optimizer state in host memory, the update on
 * the host cores ([legal] offload list, CPU-offload bullet: optimizer states
 * in CPU DRAM, Adam on the CPU while the GPU runs forward and backward;
 * [genomic] offload list, CPU-offload bullet: fp32 master weights and
 * optimizer states in CPU RAM, half parameters and gradients on the GPU).
 * ---------------------------------------------------------------------- */

/* The update of zero_adam_step, run on the host over HOST buffers: same
 * scalars, same operation order, same rounding, so the result is bit for
 * bit that of the device update.  flat_grad: S gradients of grad_dtype
 * (ZERO_F16 / ZERO_BF16 2-byte, ZERO_F32 4-byte aligned); master / exp_avg / exp_avg_sq: S floats each (4-byte aligned);
 * param (may be NULL): host buffer holding flat indices [param_base,
 * param_base + param_numel), which must contain the shard's real range.
 * overflow: 1 = skip (nothing written), 0 = apply, -1 = test the real
 * gradients flat_grad[0, real) for inf/NaN here first.  n_threads (1..1024): host threads, taken from a pool
 * the library keeps between calls (a call made while another one holds that
 * pool starts threads of its own; a process made by fork() builds a pool of
 * its own); the result does not depend on it.  Calls on disjoint buffers
 * may run concurrently.  Returns 0 applied, 1 skipped, or a negative error
 * (ZERO_ENULL, ZERO_EINVAL, ZERO_EALIGN, ZERO_ENOMEM).  Needs no GPU. */
int zero_cpu_adam_step(const zero_plan_t* plan, const zero_adam_hparams_t* hp, int64_t step,
                       double loss_scale, const void* flat_grad, int32_t grad_dtype,
                       float* master, float* exp_avg, float* exp_avg_sq, void* param,
                       int64_t param_base, int64_t param_numel, int32_t param_dtype,
                       int32_t overflow, int32_t n_threads);

/* Name of the host instruction set the update uses: "avx512", "avx2" or
 * "scalar".  The default is the widest the CPU has, except that AMD cores
 * use "avx2" (faster there); the environment variable ZERO_CPU_ISA forces
 * any of the three that the CPU has.  Every path gives the same bits. */
const char* zero_cpu_isa(void);

/* The offloaded step as a pipeline, with the one-step delayed parameter
 * update ([legal] offload list, DPU bullet: the CPU optimizer step of one
 * iteration overlaps the next iteration's forward pass; [genomic] offload
 * list, DPU bullet).  Per step, after zero_flatten_grads on the caller's
 * stream, zero_offload_submit enqueues there a one-thread snapshot (the
 * flag, t + 1 and the scale of this step; then the loss-scale policy on the
 * device state, flag cleared) and the copy of the flat gradient shard into
 * one of two pinned host buffers, and returns.  A library thread then runs
 * the host update of that step (zero_cpu_adam_step's arithmetic) and copies
 * the half parameters to the rank's offset on its own stream, ordered after
 * the caller's release of the previous parameters: the next submit, a
 * zero_offload_wait_params or zero_offload_drain.  The copies and the update
 * go in pieces of at least 2^25 elements (at most 16 pieces): the update of
 * a piece starts when its gradients have arrived, and its parameters go back
 * at once when the release is already recorded (the serialised step), so a
 * step's copies overlap its own update; the update never waits for the
 * release.  (The environment variable ZERO_OFFLOAD_MIN_CHUNK, read at create,
 * lowers the piece size, down to 64 elements, for tests.)  At most two
 * steps are in flight; a submit waits (host) for the older one when needed.
 *
 * A training loop with the delayed update:
 *   for each step: zero_offload_wait_params(o, 1, s);   forward(s); backward(s);
 *                  zero_flatten_grads(..., s);  zero_offload_submit(o, ..., s);
 *   zero_offload_drain(o, s);
 * With lag 0 instead of 1 the step is serialised (no overlap). */
typedef struct zero_offload zero_offload_t;

typedef struct {
    int64_t submitted;      /* steps submitted */
    int64_t processed;      /* steps whose host part is done */
    int64_t applied;        /* of those, updates applied */
    int64_t skipped;        /* of those, overflow-skipped */
    int32_t last_flag;      /* flag of the last processed step */
    int32_t _pad;
    double host_ms_last;    /* host update time of the last applied step */
    double host_ms_total;
    /* where the time outside the host update goes (totals, ms): the worker
     * idle until the next submit, waiting for a step's gradient copy, for
     * the previous parameter copy out of the same pinned buffer, and for the
     * caller's release of the device parameters; the caller's threads
     * blocked in submit / wait_params until the worker finished a step.  A
     * pipeline bound by the host update shows caller waits and almost no
     * worker waits; one bound by the caller shows wait_submit. */
    double wait_submit_ms_total;
    double wait_grad_ms_total;
    double wait_h2d_ms_total;
    double wait_release_ms_total;
    double caller_wait_ms_total;
} zero_offload_stats_t;

/* Creates the pipeline for `plan`, whose device state must already hold t
 * and the scaler (zero_state_upload).  master / exp_avg / exp_avg_sq: HOST
 * fp32 arrays of S elements, owned by the caller and touched only by the
 * library's thread until zero_offload_drain returns.  param_dtype: 0 for no
 * parameter write-back.  grad_dtype: ZERO_F16, ZERO_BF16 or ZERO_F32.
 * Allocates two pinned gradient buffers (S elements of grad_dtype each),
 * two pinned parameter buffers (2 real bytes each), a pool of n_threads - 1
 * host threads (kept for the pipeline's life), a transfer
 * stream and a worker thread.  Errors: ZERO_ENULL, ZERO_EINVAL, ZERO_ESTATE,
 * ZERO_EHIP, ZERO_ENOMEM. */
int zero_offload_create(zero_plan_t* plan, const zero_adam_hparams_t* hp, int32_t grad_dtype,
                        int32_t param_dtype, float* master, float* exp_avg, float* exp_avg_sq,
                        int32_t n_threads, zero_offload_t** out);

/* Submits one step: flat_grad is the device flat gradient shard (S
 * elements of the offload's grad_dtype, 16-byte aligned), normally just
 * flattened on `stream`; param the device parameter buffer holding flat
 * indices [param_base, param_base + param_numel) (may be NULL when
 * param_dtype is 0).  The step's overflow flag follows zero_adam_step's
 * gate: the flattens since the last step when they covered flat_grad,
 * otherwise a scan of its real elements on `stream`.  Errors: ZERO_ENULL,
 * ZERO_EINVAL (flat_grad last flattened in another dtype), ZERO_EALIGN,
 * ZERO_EHIP, ZERO_ESTATE, or the worker's error. */
int zero_offload_submit(zero_offload_t* off, const void* flat_grad, void* param,
                        int64_t param_base, int64_t param_numel, void* stream);

/* Makes `stream` wait (on the device) until the parameters of every
 * submitted step except the last `lag` are in the device buffer; the host
 * waits only for the host update of those steps.  lag is 1 (the one-step
 * delayed update) or 0 (serialised).  Call it before each forward: the
 * parameters it releases are overwritten only after the next submit.
 * Errors: ZERO_ENULL, ZERO_EINVAL, ZERO_ESTATE, ZERO_EHIP, or the worker's. */
int zero_offload_wait_params(zero_offload_t* off, int32_t lag, void* stream);

/* Waits (host) until every submitted step is complete, parameters copied. */
int zero_offload_drain(zero_offload_t* off, void* stream);

/* Counters of the pipeline; returns the worker's error, if any. */
int zero_offload_stats(zero_offload_t* off, zero_offload_stats_t* out);

/* One interval of the pipeline's timeline: piece `piece` of submitted step
 * `step`; kind 0 = its gradient copy (device -> pinned host), 1 = its host
 * update, 2 = its parameter copy (pinned host -> device).  Times in ms on
 * one host clock, from the moment zero_offload_timeline_start returned. */
typedef struct {
    int64_t step;
    int32_t piece;
    int32_t kind;
    double start_ms;
    double end_ms;
} zero_offload_interval_t;

/* Records a timeline of the steps submitted from now on, up to `capacity`
 * intervals (1 .. 2^24), to show how the copies of a step overlap its host
 * update ([legal] offload list, DPU bullet: CPU work of one iteration
 * overlaps GPU work).  The copies are bracketed by timing events on their
 * own streams, the update by host clock readings; a reference event, polled
 * by the host until it completes, puts both on the host clock: its
 * completion is bracketed by two polls, taken at the bracket's midpoint,
 * and a bracket wider than 20 microseconds is retried with a new event.  Costs four timing events per piece
 * and 32 bytes of host memory per interval; off unless called.  Call with no step in flight (after zero_offload_drain, or
 * before the first submit); it drops what an earlier start recorded.
 * Errors: ZERO_ENULL, ZERO_EINVAL (capacity), ZERO_ESTATE (steps in
 * flight), ZERO_EHIP, ZERO_ENOMEM. */
int zero_offload_timeline_start(zero_offload_t* off, int64_t capacity);

/* Copies up to `cap` recorded intervals into `out` (host memory; may be
 * NULL when cap is 0), in the order they were completed, and returns how
 * many are stored (at most the capacity given to zero_offload_timeline_start,
 * fewer if host memory ran out while recording; later intervals are
 * dropped) or a negative error.  Call after
 * zero_offload_drain so that the last steps' parameter copies are included.
 * Errors: ZERO_ENULL, ZERO_EINVAL (cap < 0), ZERO_ESTATE (no timeline
 * started, or another device current). */
int64_t zero_offload_timeline(zero_offload_t* off, zero_offload_interval_t* out, int64_t cap);

/* Completes the submitted steps, then releases the thread, stream and
 * buffers (NULL is a no-op). */
void zero_offload_destroy(zero_offload_t* off);

/* The fp32 scalars of the update for bias-correction steps t_first ..
 * t_first + count - 1 at loss scale loss_scale, ten floats per step in this
 * order: 1/scale, b1, 1-b1, b2, 1-b2, lr/(1-b1^t), 1/sqrt(1-b2^t), eps,
 * 1-lr*wd (AdamW; 1 for Adam-L2), wd -- each formed in double and rounded
 * once ([instr] ZeRO-1 paragraph, momentum and variance; the update of
 * zero_adam_step).  on_device = 0: out is host memory and the scalars are
 * those zero_adam_step and zero_cpu_adam_step form on the host; on_device =
 * 1: out is device memory and a kernel on `stream` forms them as
 * zero_adam_step_async's prologue does, with the device's pow and sqrt
 * (async; the caller waits for `stream`).  out: 10 * count floats, 4-byte
 * aligned.  Errors: ZERO_ENULL, ZERO_EINVAL (t_first < 1, count < 0,
 * loss_scale, hyperparameters), ZERO_EALIGN, ZERO_EHIP. */
int zero_adam_scalars(const zero_adam_hparams_t* hp, int64_t t_first, int64_t count,
                      double loss_scale, float* out, int32_t on_device, void* stream);

/* Message of the calling thread's last error ("" if none). */
const char* zero_last_error(void);

/* Kernel timing with HIP events recorded on the launch stream around each
 * kernel (off by default; skipped while the stream is being captured).  which: 0 flatten (all launches of the last
 * call), 1 overflow scan, 2 fused Adam, 3 parameter write.  *ms receives
 * the last launch's duration; the call waits for that launch to finish.
 * Errors: ZERO_ESTATE if that kernel has not run since timing was enabled. */
int zero_plan_set_timing(zero_plan_t* plan, int32_t on);
int zero_plan_kernel_ms(zero_plan_t* plan, int32_t which, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_MI355X_H */
