"""ctypes declarations of libzero_mi355x (the C ABI in include/zero_mi355x.h).

The shared library is built in-tree by ``__graft_entry__.build()``.  There is
no fallback: importing this module fails when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzero_mi355x.so")

ZERO_F16 = 1
ZERO_BF16 = 2
ZERO_F32 = 3   # gradients only

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EALIGN = -2
ZERO_ENULL = -3
ZERO_EHIP = -4
ZERO_ENOMEM = -5
ZERO_ESTATE = -6

ERROR_NAMES = {ZERO_EINVAL: "ZERO_EINVAL", ZERO_EALIGN: "ZERO_EALIGN", ZERO_ENULL: "ZERO_ENULL",
               ZERO_EHIP: "ZERO_EHIP", ZERO_ENOMEM: "ZERO_ENOMEM", ZERO_ESTATE: "ZERO_ESTATE"}


class zero_segment_t(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("tensor_off", ctypes.c_int64),
                ("shard_off", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("bucket", ctypes.c_int32), ("_pad", ctypes.c_int32)]


class zero_plan_info_t(ctypes.Structure):
    _fields_ = [("total_numel", ctypes.c_int64), ("padded_numel", ctypes.c_int64),
                ("shard_numel", ctypes.c_int64), ("shard_begin", ctypes.c_int64),
                ("real_numel", ctypes.c_int64), ("align_elems", ctypes.c_int64),
                ("bucket_elems", ctypes.c_int64), ("bytes_stage1", ctypes.c_int64),
                ("bytes_stage2", ctypes.c_int64), ("bytes_stage3", ctypes.c_int64),
                ("world_size", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("n_tensors", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("n_buckets", ctypes.c_int32), ("_pad", ctypes.c_int32)]


class zero_adam_hparams_t(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("adamw", ctypes.c_int32), ("_pad", ctypes.c_int32)]


class zero_offload_stats_t(ctypes.Structure):
    _fields_ = [("submitted", ctypes.c_int64), ("processed", ctypes.c_int64),
                ("applied", ctypes.c_int64), ("skipped", ctypes.c_int64),
                ("last_flag", ctypes.c_int32), ("_pad", ctypes.c_int32),
                ("host_ms_last", ctypes.c_double), ("host_ms_total", ctypes.c_double),
                ("wait_submit_ms_total", ctypes.c_double),
                ("wait_grad_ms_total", ctypes.c_double), ("wait_h2d_ms_total", ctypes.c_double),
                ("wait_release_ms_total", ctypes.c_double),
                ("caller_wait_ms_total", ctypes.c_double)]


class zero_offload_interval_t(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("piece", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("start_ms", ctypes.c_double), ("end_ms", ctypes.c_double)]


class zero_scaler_t(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("min_scale", ctypes.c_double),
                ("backoff", ctypes.c_double), ("growth", ctypes.c_double),
                ("window", ctypes.c_int32), ("good_steps", ctypes.c_int32),
                ("dynamic", ctypes.c_int32), ("_pad", ctypes.c_int32)]


_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

# name -> (restype, argtypes); the same list the header declares
SIGNATURES = {
    "zero_partition_plan": (ctypes.c_int, [_VP, _I32, _I32, _I32, _I64, _I64,
                                           ctypes.POINTER(_VP)]),
    "zero_plan_info": (ctypes.c_int, [_VP, ctypes.POINTER(zero_plan_info_t)]),
    "zero_plan_segments": (_I64, [_VP, ctypes.POINTER(zero_segment_t), _I64]),
    "zero_plan_tensor_buckets": (ctypes.c_int, [_VP, ctypes.POINTER(_I32), _I64]),
    "zero_plan_destroy": (None, [_VP]),
    "zero_flatten_grads": (ctypes.c_int, [_VP, _I32, ctypes.POINTER(_VP), _I32, _VP, _VP]),
    "zero_flatten_invalidate": (ctypes.c_int, [_VP]),
    "zero_adam_step": (ctypes.c_int, [_VP, ctypes.POINTER(zero_adam_hparams_t), _I64,
                                      ctypes.c_double, _VP, _I32, _VP, _VP, _VP, _VP, _I64, _I64,
                                      _I32, _VP]),
    "zero_update_loss_scale": (ctypes.c_int, [ctypes.POINTER(zero_scaler_t), _I32]),
    "zero_write_param_shard": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I32, _VP]),
    "zero_state_upload": (ctypes.c_int, [_VP, _I64, ctypes.POINTER(zero_scaler_t), _VP]),
    "zero_state_download": (ctypes.c_int, [_VP, ctypes.POINTER(_I64), ctypes.POINTER(zero_scaler_t),
                                           ctypes.POINTER(_I32), ctypes.POINTER(_I64), _VP]),
    "zero_state_device_scale": (ctypes.c_int, [_VP, ctypes.POINTER(_VP)]),
    "zero_adam_step_async": (ctypes.c_int, [_VP, ctypes.POINTER(zero_adam_hparams_t), _VP, _I32,
                                            _VP, _VP, _VP, _VP, _I64, _I64, _I32, _VP]),
    "zero_adam_step_noalloc": (ctypes.c_int, [_VP, ctypes.POINTER(zero_adam_hparams_t), _I64,
                                              ctypes.c_double, _VP, _I32, _VP, _VP, _VP, _VP,
                                              _I64, _I64, _I32, _VP, _VP]),
    "zero_cpu_adam_step": (ctypes.c_int, [_VP, ctypes.POINTER(zero_adam_hparams_t), _I64,
                                          ctypes.c_double, _VP, _I32, _VP, _VP, _VP, _VP, _I64,
                                          _I64, _I32, _I32, _I32]),
    "zero_cpu_isa": (ctypes.c_char_p, []),
    "zero_offload_create": (ctypes.c_int, [_VP, ctypes.POINTER(zero_adam_hparams_t), _I32, _I32,
                                           _VP, _VP, _VP, _I32, ctypes.POINTER(_VP)]),
    "zero_offload_submit": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _VP]),
    "zero_offload_wait_params": (ctypes.c_int, [_VP, _I32, _VP]),
    "zero_offload_drain": (ctypes.c_int, [_VP, _VP]),
    "zero_offload_stats": (ctypes.c_int, [_VP, ctypes.POINTER(zero_offload_stats_t)]),
    "zero_offload_timeline_start": (ctypes.c_int, [_VP, _I64]),
    "zero_offload_timeline": (ctypes.c_int64, [_VP, ctypes.POINTER(zero_offload_interval_t),
                                               _I64]),
    "zero_offload_destroy": (None, [_VP]),
    "zero_adam_scalars": (ctypes.c_int, [ctypes.POINTER(zero_adam_hparams_t), _I64, _I64,
                                         ctypes.c_double, _VP, _I32, _VP]),
    "zero_last_error": (ctypes.c_char_p, []),
    "zero_plan_set_timing": (ctypes.c_int, [_VP, _I32]),
    "zero_plan_kernel_ms": (ctypes.c_int, [_VP, _I32, ctypes.POINTER(ctypes.c_float)]),
}


def hip_runtimes_mapped() -> set:
    """Paths of every HIP runtime library mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if line.count("/") else ""
                if os.path.basename(path).startswith("libamdhip64.so"):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: the HIP library must be built (python __graft_entry__.py); "
            "there is no CPU fallback")
    # One HIP runtime per process: torch carries its own libamdhip64 (same
    # SONAME as ROCm's), so load it first and the library binds to it.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class ZeroError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib.zero_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def check(code: int, where: str) -> int:
    if code < 0:
        raise ZeroError(code, where)
    return code
