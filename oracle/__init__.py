"""CPU oracle for one rank's partitioned mixed-precision Adam step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product package never
imports it.  The arithmetic lives in ``zero_oracle.c`` (plain scalar C,
built by ``__graft_entry__.build()`` into ``liboracle.so``); this module only
marshals numpy arrays.

ZERO_ORACLE_LIB (tests only) names another build of ``zero_oracle.c`` to
load instead of ``liboracle.so``: the mutation tests use it to show that the
oracle's pins fail when a plausible mistake is planted in it.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ZERO_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F16 = 1
BF16 = 2
F32 = 3
DTYPES = {"f16": F16, "bf16": BF16, "f32": F32}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        lib.oracle_plan.restype = ctypes.c_int
        lib.oracle_plan.argtypes = [P, i64, i64, i64, i64, i64, P, P, P, P, P, P]
        lib.oracle_flatten.restype = None
        lib.oracle_flatten.argtypes = [P, P, P, P, P, i64, i64, i64, P]
        lib.oracle_flatten_f32.restype = None
        lib.oracle_flatten_f32.argtypes = [P, P, P, P, P, i64, i64, i64, P]
        lib.oracle_nonfinite.restype = ctypes.c_int
        lib.oracle_nonfinite.argtypes = [P, i64, ctypes.c_int]
        lib.oracle_half_to_float_n.restype = None
        lib.oracle_half_to_float_n.argtypes = [P, i64, ctypes.c_int, P]
        lib.oracle_float_to_half_n.restype = None
        lib.oracle_float_to_half_n.argtypes = [P, i64, ctypes.c_int, P]
        for name in ("oracle_adam_update", "oracle_adam_step"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int if name == "oracle_adam_step" else None
            fn.argtypes = [i64, i64, d, P, ctypes.c_int, P, P, P, d, d, d, d, d, ctypes.c_int]
        lib.oracle_write_param.restype = None
        lib.oracle_write_param.argtypes = [P, i64, i64, i64, P, ctypes.c_int]
        lib.oracle_update_scale.restype = None
        lib.oracle_update_scale.argtypes = [ctypes.POINTER(d), ctypes.POINTER(i32), ctypes.c_int,
                                            ctypes.c_int, d, d, d, i32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


@dataclass
class OraclePlan:
    P: int
    P_pad: int
    S: int
    begin: int
    real: int
    seg_tensor: np.ndarray
    seg_tensor_off: np.ndarray
    seg_shard_off: np.ndarray
    seg_numel: np.ndarray
    tensor_bucket: np.ndarray
    n_buckets: int
    bytes_stage1: int
    bytes_stage2: int
    bytes_stage3: int

    @property
    def n_segments(self) -> int:
        return int(self.seg_tensor.size)


def plan(numels: Sequence[int], world_size: int, rank: int, align: int = 64,
         bucket_elems: int = 1 << 25) -> OraclePlan:
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    n = nums.size
    scal = np.zeros(10, dtype=np.int64)
    bufs = [np.zeros(max(n, 1), dtype=np.int64) for _ in range(5)]
    rc = _load().oracle_plan(_ptr(nums), n, world_size, rank, align, bucket_elems, _ptr(scal),
                             *[_ptr(b) for b in bufs])
    if rc != 0:
        raise ValueError("oracle_plan: invalid arguments")
    nseg = int(scal[5])
    return OraclePlan(P=int(scal[0]), P_pad=int(scal[1]), S=int(scal[2]), begin=int(scal[3]),
                      real=int(scal[4]), seg_tensor=bufs[0][:nseg].copy(),
                      seg_tensor_off=bufs[1][:nseg].copy(), seg_shard_off=bufs[2][:nseg].copy(),
                      seg_numel=bufs[3][:nseg].copy(), tensor_bucket=bufs[4][:n].copy(),
                      n_buckets=int(scal[6]), bytes_stage1=int(scal[7]),
                      bytes_stage2=int(scal[8]), bytes_stage3=int(scal[9]))


def _grad_word(grads) -> type:
    """uint32 when the gradients are fp32 bits (uint32 or float32 arrays), else uint16."""
    for g in grads:
        if g is not None:
            return np.uint32 if np.asarray(g).dtype in (np.uint32, np.float32) else np.uint16
    return np.uint16


def flatten(p: OraclePlan, grads: List[Optional[np.ndarray]],
            dtype: Optional[str] = None) -> np.ndarray:
    """grads[i]: tensor i's gradient bits (None when it has no segment): uint16 arrays of
    fp16 / bf16 bits, or uint32 / float32 arrays of fp32 gradients (then the flat shard
    is uint32).  dtype ("f16", "bf16", "f32") fixes the element width when no array
    gives it."""
    word = _grad_word(grads) if dtype is None else (np.uint32 if dtype == "f32" else np.uint16)
    keep = [None if g is None else
            np.ascontiguousarray(np.asarray(g).view(word) if np.asarray(g).dtype == np.float32
                                 else g, dtype=word) for g in grads]
    ptrs = (ctypes.c_void_p * max(len(keep), 1))()
    for i, g in enumerate(keep):
        ptrs[i] = g.ctypes.data if g is not None else None
    for s in range(p.n_segments):
        g = keep[int(p.seg_tensor[s])]
        if g is None or g.size < p.seg_tensor_off[s] + p.seg_numel[s]:
            raise ValueError(f"gradient of tensor {int(p.seg_tensor[s])} missing or too small")
    flat = np.full(p.S, 0xDEAD, dtype=word)   # every element must be written
    fn = _load().oracle_flatten_f32 if word == np.uint32 else _load().oracle_flatten
    fn(ctypes.addressof(ptrs), _ptr(p.seg_tensor), _ptr(p.seg_tensor_off),
                           _ptr(p.seg_shard_off), _ptr(p.seg_numel), p.n_segments, p.S, p.real,
                           _ptr(flat))
    return flat


def nonfinite(h: np.ndarray, dtype: str) -> bool:
    """h: uint16 bits of fp16 / bf16 gradients, or uint32 bits of fp32 ones (dtype "f32")."""
    h = _grad_bits(h, dtype)
    return bool(_load().oracle_nonfinite(_ptr(h), h.size, DTYPES[dtype]))


def half_to_float(h: np.ndarray, dtype: str) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.size, dtype=np.float32)
    _load().oracle_half_to_float_n(_ptr(h), h.size, DTYPES[dtype], _ptr(out))
    return out


def float_to_half(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    _load().oracle_float_to_half_n(_ptr(x), x.size, DTYPES[dtype], _ptr(out))
    return out


def _grad_bits(g: np.ndarray, dtype: str) -> np.ndarray:
    g = np.asarray(g)
    if dtype == "f32":
        return np.ascontiguousarray(g.view(np.uint32) if g.dtype == np.float32 else g,
                                    dtype=np.uint32)
    return np.ascontiguousarray(g, dtype=np.uint16)


def _adam(fn, t, scale, flat, gdt, master, m, v, lr, b1, b2, eps, wd, adamw):
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    flat = _grad_bits(flat, gdt)
    n = master.size
    assert flat.size == n and m.size == n and v.size == n
    return fn(n, t, scale, _ptr(flat), DTYPES[gdt], _ptr(master), _ptr(m), _ptr(v), lr, b1, b2,
              eps, wd, 1 if adamw else 0)


def adam_step(t: int, scale: float, flat: np.ndarray, gdt: str, master: np.ndarray,
              m: np.ndarray, v: np.ndarray, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01,
              adamw=True) -> int:
    """In place on master/m/v; returns 1 when the step overflowed and was skipped."""
    return int(_adam(_load().oracle_adam_step, t, scale, flat, gdt, master, m, v, lr, b1, b2,
                     eps, wd, adamw))


def adam_update(t: int, scale: float, flat: np.ndarray, gdt: str, master: np.ndarray,
                m: np.ndarray, v: np.ndarray, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01,
                adamw=True) -> None:
    """The update alone (no overflow test), in place."""
    _adam(_load().oracle_adam_update, t, scale, flat, gdt, master, m, v, lr, b1, b2, eps, wd,
          adamw)


def write_param(master: np.ndarray, real: int, begin: int, base: int, param: np.ndarray,
                pdt: str) -> None:
    master = np.ascontiguousarray(master, dtype=np.float32)
    assert param.dtype == np.uint16 and param.flags.c_contiguous
    if real > 0:
        assert begin - base >= 0 and begin + real - base <= param.size and master.size >= real
    _load().oracle_write_param(_ptr(master), real, begin, base, _ptr(param), DTYPES[pdt])


class Scaler:
    """Host loss-scale state driven by the oracle's policy function."""

    def __init__(self, scale: float, dynamic: bool, min_scale: float = 1.0, backoff: float = 0.5,
                 growth: float = 2.0, window: int = 1000):
        self.scale = ctypes.c_double(scale)
        self.good = ctypes.c_int32(0)
        self.dynamic = dynamic
        self.min_scale, self.backoff, self.growth, self.window = min_scale, backoff, growth, window

    def update(self, overflow: int) -> None:
        _load().oracle_update_scale(ctypes.byref(self.scale), ctypes.byref(self.good),
                                    int(overflow), 1 if self.dynamic else 0, self.min_scale,
                                    self.backoff, self.growth, self.window)

    @property
    def value(self) -> float:
        return float(self.scale.value)
