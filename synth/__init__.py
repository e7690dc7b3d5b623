"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Only random numbers and workload shapes live here: no partitioning, flatten,
overflow test, optimizer arithmetic or half-precision rounding of the
method.  Values are defined by ``synth_host.c`` (counter based SplitMix64
words and a four-term Irwin-Hall normal); ``synth_dev.hip`` implements the
same definition on the GPU.  The last rounding of a value to fp16/bf16 is a
library conversion (numpy / torch), IEEE round-to-nearest-even on both
sides.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, small_sizes  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

STREAM_GRAD = 1
STREAM_MASTER = 2

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise ImportError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, i64, u32, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
        lib.synth_mix64.restype = u64
        lib.synth_mix64.argtypes = [u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u32, u32]
        lib.synth_word.restype = u64
        lib.synth_word.argtypes = [u64, i64]
        lib.synth_fill_f32.restype = None
        lib.synth_fill_f32.argtypes = [ctypes.c_void_p, i64, u64, i64, f32, f32, u32, f32]
        lib.synth_gather_f32.restype = None
        lib.synth_gather_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, u64, f32, f32,
                                         u32, f32]
        lib.synth_small_sizes.restype = None
        lib.synth_small_sizes.argtypes = [ctypes.c_void_p, i64, i64, i64]
        lib.synth_inject.restype = ctypes.c_int
        lib.synth_inject.argtypes = [u64, u32, i64, u32, ctypes.POINTER(i64)]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise ImportError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (bind to torch's HIP runtime: one runtime per process)
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_fill_f32.restype = ctypes.c_int
        lib.synth_dev_fill_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                           ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p]
        _dev = lib
    return _dev


def key(seed: int, stream: int, it: int) -> int:
    return int(_load_host().synth_key(seed, stream, it))


def mix64(z: int) -> int:
    return int(_load_host().synth_mix64(z & 0xFFFFFFFFFFFFFFFF))


def outlier_thresh(p: float) -> int:
    """Threshold for an outlier probability p (compared with 32 hash bits)."""
    return int(round(p * 2.0 ** 32)) if p > 0 else 0


def host_values(k: int, index0: int, n: int, sigma: float, scale: float = 1.0,
                othresh: int = 0, omult: float = 1.0) -> np.ndarray:
    out = np.empty(max(n, 0), dtype=np.float32)
    if n > 0:
        _load_host().synth_fill_f32(out.ctypes.data, n, k, index0, sigma, scale, othresh, omult)
    return out


def host_gather(k: int, idx: np.ndarray, sigma: float, scale: float = 1.0,
                othresh: int = 0, omult: float = 1.0) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    if idx.size:
        _load_host().synth_gather_f32(out.ctypes.data, idx.ctypes.data, idx.size, k, sigma,
                                      scale, othresh, omult)
    return out


def inject(seed: int, it: int, n: int, p: float):
    """Return the injected position in [0, n) for iteration ``it``, or None."""
    pos = ctypes.c_int64(0)
    hit = _load_host().synth_inject(seed, it, n, outlier_thresh(p), ctypes.byref(pos))
    return int(pos.value) if hit else None


def half_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to fp16 / bf16 with a library conversion; return uint16 bits."""
    values = np.ascontiguousarray(values, dtype=np.float32)
    if dtype == "f16":
        return values.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(values).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def grad_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Gradient bits of fp32 values: fp16 / bf16 as half_bits, fp32 ("f32") as they are
    (uint32)."""
    if dtype == "f32":
        return np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).copy()
    return half_bits(values, dtype)


def dev_fill_f32(out, k: int, index0: int, sigma: float, scale: float = 1.0,
                 othresh: int = 0, omult: float = 1.0, stream=None) -> None:
    """Fill a contiguous float32 CUDA tensor with the values of flat indices index0 + j."""
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    rc = _load_dev().synth_dev_fill_f32(out.data_ptr(), out.numel(), k, index0, sigma, scale,
                                        othresh, omult, stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_f32 failed with hipError {rc}")


def dev_fill_half(out, k: int, index0: int, sigma: float, scale: float = 1.0,
                  othresh: int = 0, omult: float = 1.0, chunk: int = 1 << 27) -> None:
    """Fill a contiguous fp16/bf16 CUDA tensor: fp32 values from the device generator,
    rounded by torch's conversion (RNE), in chunks to bound the fp32 scratch.  A float32
    tensor (fp32 gradients) takes the values as they are."""
    import torch
    if out.dtype == torch.float32:           # fp32 gradients: no rounding step
        dev_fill_f32(out.view(-1), k, index0, sigma, scale, othresh, omult)
        return
    flat = out.view(-1)
    n = flat.numel()
    tmp = torch.empty(min(n, chunk), dtype=torch.float32, device=out.device)
    for j0 in range(0, n, chunk):
        j1 = min(n, j0 + chunk)
        t = tmp[: j1 - j0]
        dev_fill_f32(t, k, index0 + j0, sigma, scale, othresh, omult)
        flat[j0:j1].copy_(t)
