"""One data-parallel rank's share of ZeRO's partitioned mixed-precision Adam
step, on an AMD Instinct MI355X.

Every step runs in libzero_mi355x (host planner + HIP kernels for gfx950);
this module only marshals arguments: torch tensors supply device pointers
and the stream.  The functions keep the names of the C ABI
(include/zero_mi355x.h):

    zero_partition_plan(numels, world_size, rank, align_elems, bucket_elems) -> Plan
    zero_flatten_grads(plan, bucket, grads, flat_grad, stream=None)
                                (grads: a list of tensors, or a GradList bound once)
    zero_flatten_invalidate(plan)  (the flat buffer was written after the flattens)
    zero_adam_step(plan, hparams, step, loss_scale, flat_grad, master, exp_avg,
                   exp_avg_sq, param=None, param_base=0, stream=None) -> 0 | 1
    zero_update_loss_scale(scaler, overflow)
    zero_write_param_shard(plan, master, param, param_base=0, stream=None)

and the step without host round trips (graph-capturable):

    zero_state_upload(plan, applied_steps, scaler, stream=None)
    zero_adam_step_async(plan, hparams, flat_grad, master, exp_avg, exp_avg_sq,
                         param=None, param_base=0, stream=None)
    zero_state_download(plan, stream=None) -> DeviceStepState
    zero_state_device_scale(plan) -> device address of the loss scale (double)

and, for callers that cannot allocate, the step with nothing allocated or waited for:

    zero_adam_step_noalloc(plan, hparams, step, loss_scale, flat_grad, master, exp_avg,
                           exp_avg_sq, overflow_out, param=None, param_base=0, stream=None)

and ZeRO-Offload's host-side update (host buffers: numpy arrays or CPU tensors):

    zero_cpu_adam_step(plan, hparams, step, loss_scale, flat_grad, master, exp_avg,
                       exp_avg_sq, param=None, param_base=0, grad_dtype=None,
                       param_dtype=None, overflow=-1, n_threads=None) -> 0 | 1
    zero_cpu_isa() -> "avx512" | "avx2" | "scalar"
    default_host_threads() -> n (n_threads=None: the CPUs of the affinity mask, at most 16)
    zero_adam_scalars(hparams, t_first, count, loss_scale, out=None) -> [count, 10]
                                (the update's fp32 scalars, formed on the host or
                                 on the device as the asynchronous step does)
    Offload(plan, hparams, grad_dtype, param_dtype, master, exp_avg, exp_avg_sq,
            n_threads=None)     .submit / .wait_params / .drain / .stats / .close
                                (zero_offload_* : the pipelined offloaded step with the
                                 one-step delayed parameter update)
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from dataclasses import dataclass
from typing import List, Optional, Sequence

from . import _abi
from ._abi import ZERO_BF16, ZERO_F16, ZERO_F32, ZeroError, check, lib  # noqa: F401

__all__ = ["Plan", "release_all", "AdamHParams", "LossScaler", "DeviceStepState", "ZeroError",
           "zero_partition_plan", "GradList", "zero_flatten_grads", "zero_flatten_invalidate",
           "zero_adam_step",
           "zero_update_loss_scale", "zero_write_param_shard", "zero_state_upload",
           "zero_adam_step_async", "zero_state_download", "zero_state_device_scale",
           "zero_adam_step_noalloc",
           "zero_cpu_adam_step", "zero_cpu_isa", "default_host_threads", "zero_adam_scalars", "SCALAR_FIELDS",
           "Offload", "zero_last_error", "ZERO_F16",
           "ZERO_BF16", "ZERO_F32"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return ZERO_F16
    if t.dtype == torch.bfloat16:
        return ZERO_BF16
    if t.dtype == torch.float32:
        return ZERO_F32
    raise TypeError(f"expected a float16, bfloat16 or float32 tensor, got {t.dtype}")


def _grad_dtypes():
    torch = _torch()
    return (torch.float16, torch.bfloat16, torch.float32)


def _stream_handle(stream, device) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _require(t, name: str, min_numel: int, dtypes) -> None:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs >= {min_numel}")


@dataclass
class AdamHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    adamw: bool = True

    def to_c(self) -> _abi.zero_adam_hparams_t:
        return _abi.zero_adam_hparams_t(self.lr, self.beta1, self.beta2, self.eps,
                                        self.weight_decay, 1 if self.adamw else 0, 0)


class LossScaler:
    """Host state of the dynamic loss scale; the policy runs in the library."""

    def __init__(self, scale: float = 65536.0, dynamic: bool = True, min_scale: float = 1.0,
                 backoff: float = 0.5, growth: float = 2.0, window: int = 1000):
        self.c = _abi.zero_scaler_t(scale, min_scale, backoff, growth, window, 0,
                                    1 if dynamic else 0, 0)

    @property
    def scale(self) -> float:
        return float(self.c.scale)

    @property
    def good_steps(self) -> int:
        return int(self.c.good_steps)


# Library handles not yet released.  release_all() runs from atexit, before
# the interpreter finalizes anything, so no handle is left for a destructor
# to free while the interpreter -- or the HIP runtime after it -- is being
# torn down: pipeline threads are joined and device memory is freed while
# everything is still alive.
_LIVE_PLANS: "weakref.WeakSet[Plan]" = weakref.WeakSet()
_LIVE_OFFLOADS: "weakref.WeakSet[Offload]" = weakref.WeakSet()


def release_all() -> None:
    """Release every live offload pipeline (its worker thread is joined),
    then every live plan (its device block and pinned mirror are freed).
    Registered with atexit; callers may also call it at the end of a run."""
    for o in list(_LIVE_OFFLOADS):
        o.close()
    for p in list(_LIVE_PLANS):
        p.close()


atexit.register(release_all)


class Plan:
    """A partition plan handle (owned): released by close(), by release_all()
    at exit, or when collected before the interpreter finalizes."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        info = _abi.zero_plan_info_t()
        check(lib.zero_plan_info(self._h, ctypes.byref(info)), "zero_plan_info")
        self.info = info
        _LIVE_PLANS.add(self)

    # bound at class creation: module globals may already be gone when a
    # plan is collected at interpreter exit
    _destroy = staticmethod(lib.zero_plan_destroy)
    _finalizing = staticmethod(sys.is_finalizing)

    def close(self) -> None:
        """Release the plan (and first any offload pipeline built on it).
        Later calls that need the plan fail with ZERO_ENULL."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            for o in list(_LIVE_OFFLOADS):
                if o.plan is self:
                    o.close()
            self._destroy(h)
        self._h = ctypes.c_void_p()

    def __del__(self):
        # no HIP call once the interpreter is finalizing: release_all() ran
        # at exit; what is left is reclaimed with the process
        if self._finalizing():
            return
        self.close()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    # sizes
    P = property(lambda self: int(self.info.total_numel))
    P_pad = property(lambda self: int(self.info.padded_numel))
    S = property(lambda self: int(self.info.shard_numel))
    begin = property(lambda self: int(self.info.shard_begin))
    real = property(lambda self: int(self.info.real_numel))
    n_buckets = property(lambda self: int(self.info.n_buckets))
    n_segments = property(lambda self: int(self.info.n_segments))
    n_tensors = property(lambda self: int(self.info.n_tensors))

    def segments(self) -> List[_abi.zero_segment_t]:
        n = int(check(lib.zero_plan_segments(self._h, None, 0), "zero_plan_segments"))
        arr = (_abi.zero_segment_t * max(n, 1))()
        check(lib.zero_plan_segments(self._h, arr, n), "zero_plan_segments")
        return list(arr[:n])

    def tensor_buckets(self) -> List[int]:
        n = self.n_tensors
        arr = (ctypes.c_int32 * max(n, 1))()
        check(lib.zero_plan_tensor_buckets(self._h, arr, n), "zero_plan_tensor_buckets")
        return list(arr[:n])

    def set_timing(self, on: bool) -> None:
        check(lib.zero_plan_set_timing(self._h, 1 if on else 0), "zero_plan_set_timing")

    def kernel_ms(self, which: int) -> float:
        """which: 0 flatten, 1 overflow scan, 2 fused Adam, 3 parameter write."""
        ms = ctypes.c_float(0)
        check(lib.zero_plan_kernel_ms(self._h, which, ctypes.byref(ms)), "zero_plan_kernel_ms")
        return float(ms.value)


def zero_partition_plan(numels: Sequence[int], world_size: int, rank: int,
                        align_elems: int = 64, bucket_elems: int = 1 << 25) -> Plan:
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(n) for n in numels])
    h = ctypes.c_void_p()
    check(lib.zero_partition_plan(arr, len(numels), world_size, rank, align_elems, bucket_elems,
                                  ctypes.byref(h)), "zero_partition_plan")
    plan = Plan(h.value)
    plan._numels = [int(n) for n in numels]
    return plan


class GradList:
    """A plan's gradient tensors, checked once.

    A training loop that keeps its gradient buffers from step to step binds
    them once; zero_flatten_grads then takes the stored pointer array as is,
    with no per-tensor checks on the step path (a model with hundreds of
    tensors otherwise spends about a millisecond per call in them).  The
    list keeps the tensors alive; rebind after reallocating any of them."""

    def __init__(self, plan: Plan, grads: Sequence):
        torch = _torch()
        if len(grads) != plan.n_tensors:
            raise ValueError(f"need {plan.n_tensors} gradient entries, got {len(grads)}")
        numels = _plan_numels(plan)
        self.plan = plan
        self.dtype = None
        self.ptrs = (ctypes.c_void_p * max(len(grads), 1))()
        for i, g in enumerate(grads):
            if g is None:
                continue
            _require(g, f"grads[{i}]", int(numels[i]),
                     (self.dtype,) if self.dtype is not None else _grad_dtypes())
            self.dtype = g.dtype
            self.ptrs[i] = g.data_ptr()
        self._tensors = list(grads)


def zero_flatten_grads(plan: Plan, bucket: int, grads, flat_grad, stream=None) -> None:
    """grads: one entry per tensor (a contiguous fp16/bf16 device tensor, or None for a
    tensor without elements in the requested buckets of this shard), or a GradList
    bound to this plan."""
    torch = _torch()
    _require(flat_grad, "flat_grad", plan.S, _grad_dtypes())
    if isinstance(grads, GradList):
        if grads.plan is not plan:
            raise ValueError("the GradList is bound to another plan")
        if grads.dtype is not None and grads.dtype != flat_grad.dtype:
            raise TypeError(f"gradients are {grads.dtype}, flat_grad is {flat_grad.dtype}")
        ptrs = grads.ptrs
    else:
        if len(grads) != plan.n_tensors:
            raise ValueError(f"need {plan.n_tensors} gradient entries, got {len(grads)}")
        numels = None
        ptrs = (ctypes.c_void_p * max(len(grads), 1))()
        for i, g in enumerate(grads):
            if g is None:
                ptrs[i] = None
                continue
            if numels is None:
                numels = [int(n) for n in _plan_numels(plan)]
            _require(g, f"grads[{i}]", numels[i], (flat_grad.dtype,))
            ptrs[i] = g.data_ptr()
    check(lib.zero_flatten_grads(plan.handle, bucket, ptrs, _dtype_code(flat_grad),
                                 flat_grad.data_ptr(), _stream_handle(stream, flat_grad.device)),
          "zero_flatten_grads")


def zero_flatten_invalidate(plan: Plan) -> None:
    """The flat gradient buffer was written after the flattens: the next
    step scans it instead of trusting their fused inf/NaN test."""
    check(lib.zero_flatten_invalidate(plan.handle), "zero_flatten_invalidate")


def _plan_numels(plan: Plan) -> List[int]:
    cached = getattr(plan, "_numels", None)
    if cached is None:
        raise RuntimeError("plan has no recorded tensor sizes")
    return cached


def zero_adam_step(plan: Plan, hparams: AdamHParams, step: int, loss_scale: float, flat_grad,
                   master, exp_avg, exp_avg_sq, param=None, param_base: int = 0,
                   stream=None) -> int:
    """Returns 0 when the update was applied, 1 when an overflow skipped it."""
    torch = _torch()
    _require(flat_grad, "flat_grad", plan.S, _grad_dtypes())
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _require(t, name, plan.S, (torch.float32,))
    pptr, pnum, pdt = None, 0, 0
    if param is not None:
        _require(param, "param", 0, (torch.float16, torch.bfloat16))
        pptr, pnum, pdt = param.data_ptr(), param.numel(), _dtype_code(param)
    hp = hparams.to_c()
    return check(lib.zero_adam_step(plan.handle, ctypes.byref(hp), int(step), float(loss_scale),
                                    flat_grad.data_ptr(), _dtype_code(flat_grad),
                                    master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(),
                                    pptr, int(param_base), pnum, pdt,
                                    _stream_handle(stream, master.device)), "zero_adam_step")


def zero_update_loss_scale(scaler: LossScaler, overflow: int) -> None:
    check(lib.zero_update_loss_scale(ctypes.byref(scaler.c), int(overflow)),
          "zero_update_loss_scale")


def zero_write_param_shard(plan: Plan, master, param, param_base: int = 0, stream=None) -> None:
    torch = _torch()
    _require(master, "master", plan.real, (torch.float32,))
    _require(param, "param", 0, (torch.float16, torch.bfloat16))
    check(lib.zero_write_param_shard(plan.handle, master.data_ptr(), param.data_ptr(),
                                     int(param_base), param.numel(), _dtype_code(param),
                                     _stream_handle(stream, master.device)),
          "zero_write_param_shard")


@dataclass
class DeviceStepState:
    """The device state of the asynchronous step, as read back."""
    applied_steps: int
    skipped_steps: int
    last_flag: int
    scale: float
    good_steps: int


def zero_state_upload(plan: Plan, applied_steps: int, scaler: LossScaler, stream=None) -> None:
    """Load t (= applied_steps) and the scaler into the plan's device state (waits)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device())
    check(lib.zero_state_upload(plan.handle, int(applied_steps), ctypes.byref(scaler.c),
                                _stream_handle(stream, dev)), "zero_state_upload")


def zero_state_download(plan: Plan, stream=None, scaler: Optional[LossScaler] = None
                        ) -> DeviceStepState:
    """Read the device state back (waits); also refreshes `scaler` when given."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device())
    t = ctypes.c_int64(0)
    skipped = ctypes.c_int64(0)
    last = ctypes.c_int32(0)
    sc = _abi.zero_scaler_t()
    check(lib.zero_state_download(plan.handle, ctypes.byref(t), ctypes.byref(sc),
                                  ctypes.byref(last), ctypes.byref(skipped),
                                  _stream_handle(stream, dev)), "zero_state_download")
    if scaler is not None:
        ctypes.memmove(ctypes.byref(scaler.c), ctypes.byref(sc), ctypes.sizeof(sc))
    return DeviceStepState(int(t.value), int(skipped.value), int(last.value), float(sc.scale),
                           int(sc.good_steps))


def zero_state_device_scale(plan: Plan) -> int:
    """Device address of the current loss scale (a double)."""
    out = ctypes.c_void_p()
    check(lib.zero_state_device_scale(plan.handle, ctypes.byref(out)), "zero_state_device_scale")
    return int(out.value)


def zero_adam_step_async(plan: Plan, hparams: AdamHParams, flat_grad, master, exp_avg,
                         exp_avg_sq, param=None, param_base: int = 0, stream=None) -> None:
    """Enqueue the gated update and the loss-scale policy on the device state;
    returns at once (nothing waits, nothing is allocated)."""
    torch = _torch()
    _require(flat_grad, "flat_grad", plan.S, _grad_dtypes())
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _require(t, name, plan.S, (torch.float32,))
    pptr, pnum, pdt = None, 0, 0
    if param is not None:
        _require(param, "param", 0, (torch.float16, torch.bfloat16))
        pptr, pnum, pdt = param.data_ptr(), param.numel(), _dtype_code(param)
    hp = hparams.to_c()
    check(lib.zero_adam_step_async(plan.handle, ctypes.byref(hp), flat_grad.data_ptr(),
                                   _dtype_code(flat_grad), master.data_ptr(),
                                   exp_avg.data_ptr(), exp_avg_sq.data_ptr(), pptr,
                                   int(param_base), pnum, pdt,
                                   _stream_handle(stream, master.device)),
          "zero_adam_step_async")


def zero_adam_step_noalloc(plan: Plan, hparams: AdamHParams, step: int, loss_scale: float,
                           flat_grad, master, exp_avg, exp_avg_sq, overflow_out, param=None,
                           param_base: int = 0, stream=None) -> None:
    """zero_adam_step with nothing allocated and nothing waited for: the
    flag (1 skipped, 0 applied) lands in overflow_out, an int32 device
    tensor, when the stream reaches it."""
    torch = _torch()
    _require(flat_grad, "flat_grad", plan.S, _grad_dtypes())
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _require(t, name, plan.S, (torch.float32,))
    _require(overflow_out, "overflow_out", 1, (torch.int32,))
    pptr, pnum, pdt = None, 0, 0
    if param is not None:
        _require(param, "param", 0, (torch.float16, torch.bfloat16))
        pptr, pnum, pdt = param.data_ptr(), param.numel(), _dtype_code(param)
    hp = hparams.to_c()
    check(lib.zero_adam_step_noalloc(plan.handle, ctypes.byref(hp), int(step), float(loss_scale),
                                     flat_grad.data_ptr(), _dtype_code(flat_grad),
                                     master.data_ptr(), exp_avg.data_ptr(),
                                     exp_avg_sq.data_ptr(), pptr, int(param_base), pnum, pdt,
                                     overflow_out.data_ptr(),
                                     _stream_handle(stream, master.device)),
          "zero_adam_step_noalloc")


_HALF_CODES = {"f16": ZERO_F16, "bf16": ZERO_BF16, ZERO_F16: ZERO_F16, ZERO_BF16: ZERO_BF16}
_GRAD_CODES = {**_HALF_CODES, "f32": ZERO_F32, ZERO_F32: ZERO_F32}


def _host_buffer(x, name: str, min_numel: int, itemsize: int):
    """(address, numel) of a contiguous host buffer: a numpy array or a CPU tensor."""
    torch = _torch()
    if isinstance(x, torch.Tensor):
        if x.is_cuda:
            raise ValueError(f"{name} must be host memory")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        addr, n, isz = x.data_ptr(), x.numel(), x.element_size()
    else:
        import numpy as np
        if not isinstance(x, np.ndarray) or not x.flags.c_contiguous:
            raise ValueError(f"{name} must be a contiguous numpy array or CPU tensor")
        addr, n, isz = x.ctypes.data, x.size, x.itemsize
    if isz != itemsize:
        raise TypeError(f"{name} has {isz}-byte elements, expected {itemsize}")
    if n < min_numel:
        raise ValueError(f"{name} holds {n} elements, needs >= {min_numel}")
    return addr, n


def _half_code(x, given):
    if given is not None:
        return _HALF_CODES[given]
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.dtype in (torch.float16, torch.bfloat16):
        return _dtype_code(x)
    raise TypeError("pass param_dtype ('f16' or 'bf16') for raw 16-bit buffers")


def _grad_code(x, given):
    if given is not None:
        return _GRAD_CODES[given]
    torch = _torch()
    if isinstance(x, torch.Tensor) and x.dtype in _grad_dtypes():
        return _dtype_code(x)
    import numpy as np
    if isinstance(x, np.ndarray) and x.dtype == np.float32:
        return ZERO_F32
    raise TypeError("pass grad_dtype ('f16', 'bf16' or 'f32') for raw gradient buffers")


def zero_cpu_adam_step(plan: Plan, hparams: AdamHParams, step: int, loss_scale: float, flat_grad,
                       master, exp_avg, exp_avg_sq, param=None, param_base: int = 0,
                       grad_dtype=None, param_dtype=None, overflow: int = -1,
                       n_threads: Optional[int] = None) -> int:
    """ZeRO-Offload's update on host buffers; returns 0 applied, 1 skipped.
    overflow: -1 tests flat_grad here, 0 / 1 pass a known flag."""
    gcode = _grad_code(flat_grad, grad_dtype)
    g, _ = _host_buffer(flat_grad, "flat_grad", plan.S, 4 if gcode == ZERO_F32 else 2)
    ptrs = [_host_buffer(t, name, plan.S, 4)[0] for name, t in
            (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq))]
    pptr, pnum, pdt = None, 0, 0
    if param is not None:
        pptr, pnum = _host_buffer(param, "param", 0, 2)
        pdt = _half_code(param, param_dtype)
    if n_threads is None:
        n_threads = default_host_threads()
    hp = hparams.to_c()
    return check(lib.zero_cpu_adam_step(plan.handle, ctypes.byref(hp), int(step),
                                        float(loss_scale), g, gcode,
                                        *ptrs, pptr, int(param_base), pnum, pdt, int(overflow),
                                        int(n_threads)), "zero_cpu_adam_step")


def default_host_threads() -> int:
    """Threads the host update uses when none are given: the CPUs this
    process may run on (its affinity mask), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def zero_cpu_isa() -> str:
    return lib.zero_cpu_isa().decode()


SCALAR_FIELDS = ("inv_scale", "b1", "omb1", "b2", "omb2", "step", "rsbc2", "eps", "decay", "wd")


def zero_adam_scalars(hparams: AdamHParams, t_first: int, count: int, loss_scale: float,
                      out=None, stream=None):
    """The update's fp32 scalars for steps t_first .. t_first + count - 1,
    shape [count, 10] (columns SCALAR_FIELDS).  out=None: formed on the host
    (a numpy array is returned); out a float32 device tensor of >= 10*count
    elements: formed on the device as the asynchronous step forms them
    (enqueued on `stream`)."""
    hp = hparams.to_c()
    if out is None:
        import numpy as np
        arr = np.zeros((max(count, 0), len(SCALAR_FIELDS)), np.float32)
        check(lib.zero_adam_scalars(ctypes.byref(hp), int(t_first), int(count), float(loss_scale),
                                    arr.ctypes.data, 0, None), "zero_adam_scalars")
        return arr
    torch = _torch()
    _require(out, "out", 10 * count, (torch.float32,))
    check(lib.zero_adam_scalars(ctypes.byref(hp), int(t_first), int(count), float(loss_scale),
                                out.data_ptr(), 1, _stream_handle(stream, out.device)),
          "zero_adam_scalars")
    return out


class Offload:
    """ZeRO-Offload pipeline of one rank (zero_offload_*): host-resident fp32
    master / moments, host update on a library thread, parameters copied
    back with the one-step delayed update.  The plan's device state must be
    uploaded first (zero_state_upload).  The host arrays must stay alive and
    untouched until drain() returns."""

    def __init__(self, plan: Plan, hparams: AdamHParams, grad_dtype, param_dtype, master,
                 exp_avg, exp_avg_sq, n_threads: Optional[int] = None):
        self.plan = plan
        self._keep = (master, exp_avg, exp_avg_sq)
        ptrs = [_host_buffer(t, name, plan.S, 4)[0] for name, t in
                (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq))]
        if n_threads is None:
            n_threads = default_host_threads()
        pdt = 0 if param_dtype is None else _HALF_CODES[param_dtype]
        hp = hparams.to_c()
        h = ctypes.c_void_p()
        check(lib.zero_offload_create(plan.handle, ctypes.byref(hp), _GRAD_CODES[grad_dtype], pdt,
                                      *ptrs, int(n_threads), ctypes.byref(h)),
              "zero_offload_create")
        self._h = h
        self._gcode = _GRAD_CODES[grad_dtype]
        _LIVE_OFFLOADS.add(self)

    def _stream(self, stream):
        torch = _torch()
        return _stream_handle(stream, torch.device("cuda", torch.cuda.current_device()))

    def submit(self, flat_grad, param=None, param_base: int = 0, stream=None) -> None:
        torch = _torch()
        _require(flat_grad, "flat_grad", self.plan.S, _grad_dtypes())
        if _dtype_code(flat_grad) != self._gcode:
            raise TypeError(f"flat_grad has dtype {flat_grad.dtype}; this offload copies "
                            f"gradients of code {self._gcode}")
        pptr, pnum = None, 0
        if param is not None:
            _require(param, "param", 0, (torch.float16, torch.bfloat16))
            pptr, pnum = param.data_ptr(), param.numel()
        check(lib.zero_offload_submit(self._h, flat_grad.data_ptr(), pptr, int(param_base), pnum,
                                      self._stream(stream)), "zero_offload_submit")

    def wait_params(self, lag: int = 1, stream=None) -> None:
        check(lib.zero_offload_wait_params(self._h, int(lag), self._stream(stream)),
              "zero_offload_wait_params")

    def drain(self, stream=None) -> None:
        check(lib.zero_offload_drain(self._h, self._stream(stream)), "zero_offload_drain")

    def stats(self) -> dict:
        st = _abi.zero_offload_stats_t()
        check(lib.zero_offload_stats(self._h, ctypes.byref(st)), "zero_offload_stats")
        return {k: getattr(st, k) for k, _ in st._fields_ if k != "_pad"}

    TIMELINE_KINDS = ("gradient copy", "host update", "parameter copy")

    def timeline_start(self, capacity: int = 1 << 20) -> None:
        """Record the copies and host update of every piece of the steps
        submitted from now on (call with no step in flight)."""
        check(lib.zero_offload_timeline_start(self._h, int(capacity)),
              "zero_offload_timeline_start")

    def timeline(self) -> List[dict]:
        """The recorded intervals (call after drain()): step, piece, kind
        (one of TIMELINE_KINDS), start_ms, end_ms on one host clock."""
        n = int(check(lib.zero_offload_timeline(self._h, None, 0), "zero_offload_timeline"))
        buf = (_abi.zero_offload_interval_t * max(n, 1))()
        kept = min(n, int(check(lib.zero_offload_timeline(self._h, buf, n),
                                "zero_offload_timeline")))  # stored count; it only grows
        return [{"step": r.step, "piece": r.piece, "kind": self.TIMELINE_KINDS[r.kind],
                 "start_ms": r.start_ms, "end_ms": r.end_ms} for r in buf[:kept]]

    _destroy = staticmethod(lib.zero_offload_destroy)
    _finalizing = staticmethod(sys.is_finalizing)

    def close(self) -> None:
        """Complete the submitted steps, join the worker, free the buffers."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
        self._h = ctypes.c_void_p()

    def __del__(self):
        if self._finalizing():
            return
        self.close()


def zero_last_error() -> str:
    return lib.zero_last_error().decode(errors="replace")
