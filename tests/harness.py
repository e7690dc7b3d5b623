"""Shared drivers for the GPU parity tests and the smoke check.

A run is the same sequence of steps on both sides, from the same seeded
inputs:
  GPU    zero_flatten_grads -> zero_adam_step (fused cast) -> zero_update_loss_scale
         through the C ABI of libzero_mi355x;
  oracle oracle.flatten -> oracle.adam_step -> oracle.write_param -> Scaler.update.
Inputs come from ``synth`` (host generator for the oracle, host or device
generator for the GPU side, checked equal bit for bit).  Nothing the GPU
computes is fed to the oracle.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle
import synth
import zero_partitioned_mixed_plan_amd as z

INF_BITS = {"f16": 0x7C00, "bf16": 0x7F80, "f32": 0x7F800000}
GRAD_WORD = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}


# pytest's capture manager, set by conftest.py: progress lines of the long
# GPU tests go around the output capture, so a run under `pytest -q` prints
# them as they happen (a multi-minute test is never silent).
CAPTURE_MANAGER = None


def log(msg: str) -> None:
    if CAPTURE_MANAGER is not None:
        with CAPTURE_MANAGER.global_and_fixture_disabled():
            print(msg, flush=True)
        return
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dt: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]


def to_device_grad(bits: np.ndarray, dt: str, dev):
    """Gradient bits (uint16 for fp16 / bf16, uint32 for fp32) as a device tensor."""
    import torch
    signed = np.int32 if dt == "f32" else np.int16
    return torch.from_numpy(bits.view(signed)).to(dev).view(torch_dtype(dt))


def grad_bits_host(t, dt: str) -> np.ndarray:
    """A device gradient tensor's bits on the host (uint16, or uint32 for fp32)."""
    import torch
    if dt == "f32":
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def flat_offsets(numels: Sequence[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(numels, dtype=np.int64))]).astype(np.int64)


@dataclass
class Case:
    """A parity case: model shapes, partition and optimizer setting."""
    numels: List[int]
    world_size: int
    rank: int
    grad_dtype: str
    param_dtype: str
    steps: int
    align: int = 64
    bucket_elems: int = 1 << 25
    grad_sigma: float = 1e-3
    master_sigma: float = 0.02
    dynamic: bool = False
    init_scale: float = 1.0
    window: int = 1000
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    inject: Dict[int, int] = field(default_factory=dict)   # iteration -> shard-local index
    inject_p: float = 0.0                                  # Bernoulli per iteration
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    adamw: bool = True
    seed: int = 0
    flatten_mode: str = "all"        # "all" | "buckets" | "buckets_shuffled" | "scan"
    param_mode: str = "full"         # "full" | "window" | "none"

    @classmethod
    def from_workload(cls, w, **kw):
        base = dict(numels=w.numels, world_size=w.world_size, rank=w.rank,
                    grad_dtype=w.grad_dtype, param_dtype=w.param_dtype, steps=w.steps,
                    align=w.align, bucket_elems=w.bucket_elems, grad_sigma=w.grad_sigma,
                    master_sigma=w.master_sigma, dynamic=w.dynamic_scale,
                    init_scale=w.init_scale, outlier_p=w.outlier_p,
                    outlier_mult=w.outlier_mult, inject_p=w.inject_p, lr=w.lr,
                    beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                    adamw=w.adamw, seed=w.seed)
        base.update(kw)
        return cls(**base)

    def hparams(self) -> dict:
        return dict(lr=self.lr, b1=self.beta1, b2=self.beta2, eps=self.eps, wd=self.weight_decay,
                    adamw=self.adamw)

    def injection(self, it: int, real: int) -> Optional[int]:
        if it in self.inject:
            return self.inject[it]
        if self.inject_p > 0:
            return synth.inject(self.seed, it, real, self.inject_p)
        return None


def grad_key(case: Case, it: int) -> int:
    return synth.key(case.seed, synth.STREAM_GRAD, it)


def master_key(case: Case) -> int:
    return synth.key(case.seed, synth.STREAM_MASTER, 0)


def host_grad_values(case: Case, it: int, flat0: int, n: int, scale: float) -> np.ndarray:
    return synth.host_values(grad_key(case, it), flat0, n, case.grad_sigma, scale,
                             synth.outlier_thresh(case.outlier_p), case.outlier_mult)


def host_model_grads(case: Case, op, it: int, scale: float) -> List[Optional[np.ndarray]]:
    """Per-tensor gradient bits on the host for the tensors that touch the
    shard (full-size tensors whose part outside the shard is zero; the others
    are None), with this iteration's +inf."""
    offs = flat_offsets(case.numels)
    out: List[Optional[np.ndarray]] = [None] * len(case.numels)
    for s in range(op.n_segments):
        i = int(op.seg_tensor[s])
        g = np.zeros(case.numels[i], GRAD_WORD[case.grad_dtype])
        a, n = int(op.seg_tensor_off[s]), int(op.seg_numel[s])
        vals = host_grad_values(case, it, int(offs[i]) + a, n, scale)
        g[a:a + n] = synth.grad_bits(vals, case.grad_dtype)
        out[i] = g
    pos = case.injection(it, op.real)
    if pos is not None:
        s = int(np.searchsorted(op.seg_shard_off, pos, side="right") - 1)
        t = int(op.seg_tensor[s])
        out[t][int(op.seg_tensor_off[s] + pos - op.seg_shard_off[s])] = INF_BITS[case.grad_dtype]
    return out


def init_master_host(case: Case, begin: int, real: int, S: int) -> np.ndarray:
    m = np.zeros(S, np.float32)
    m[:real] = synth.host_values(master_key(case), begin, real, case.master_sigma)
    return m


PARAM_FILL = 0xFFFF   # a NaN pattern no finite master casts to: any stray write shows


def init_param_host(case: Case, P: int) -> np.ndarray:
    """Initial contents of the full half parameter buffer."""
    return np.full(P, PARAM_FILL, np.uint16)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    """Max distance in units in the last place between half bit patterns
    (sign-magnitude mapped to a monotone integer line)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    if a.size == 0:
        return 0
    return int(np.max(np.abs(key(a) - key(b))))


def max_rel(a: np.ndarray, b: np.ndarray) -> float:
    """max |a - b| / max(|b|, FLT_MIN) over all elements (b is the oracle)."""
    if a.size == 0:
        return 0.0
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    den = np.maximum(np.abs(b64), np.finfo(np.float32).tiny)
    return float(np.max(np.abs(a64 - b64) / den))


REL_TOL = 1e-6   # fp32 master / moments
ULP_TOL = 1      # half parameters


def host_threads() -> int:
    """Host threads for the oracle's chunked work (at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_POOL = None


def pool() -> ThreadPoolExecutor:
    """Threads for elementwise oracle work over chunks (the oracle's C calls
    release the interpreter lock; each chunk is the plain scalar loop)."""
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(host_threads())
    return _POOL


def chunk_ranges(n: int, size: int = 1 << 22):
    return [(lo, min(n, lo + size)) for lo in range(0, n, size)]


def float_to_half_chunked(x: np.ndarray, dtype: str) -> np.ndarray:
    """oracle.float_to_half over chunks on the host threads."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.uint16)

    def one(c):
        out[c[0]:c[1]] = oracle.float_to_half(x[c[0]:c[1]], dtype)
    list(pool().map(one, chunk_ranges(x.size)))
    return out


def cast_library(x: np.ndarray, dtype: str, parallel: bool = True) -> np.ndarray:
    """fp32 -> fp16 / bf16 bits by torch's CPU round-to-nearest-even
    conversion, over chunks on the host threads.  The oracle's own cast
    (oracle.float_to_half, written from IEEE 754) equals this conversion on
    all 2^32 fp32 bit patterns except NaN payloads (tests/test_oracle_cast.py),
    so for the multi-billion-element shards the expected parameters come
    from the oracle's fp32 master through this faster, identical conversion."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.uint16)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16

    def one(c):
        lo, hi = c
        out[lo:hi] = torch.from_numpy(x[lo:hi]).to(tdt).view(torch.int16).numpy().view(
            np.uint16)
    if parallel:
        list(pool().map(one, chunk_ranges(x.size)))
    else:                      # the caller already runs on one of several threads
        one((0, x.size))
    return out


def write_param_chunked(master: np.ndarray, real: int, begin: int, base: int,
                        param: np.ndarray, pdt: str) -> None:
    """oracle.write_param over chunks of the shard on the host threads: chunk
    [lo, hi) of the shard writes param[begin + lo - base, begin + hi - base)."""
    def one(c):
        lo, hi = c
        oracle.write_param(master[lo:hi], hi - lo, begin + lo, base, param, pdt)
    list(pool().map(one, chunk_ranges(max(real, 0))))


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-for-bit equality of two equally typed arrays, over chunks."""
    if a.shape != b.shape:
        return False
    return all(pool().map(lambda c: np.array_equal(a[c[0]:c[1]], b[c[0]:c[1]]),
                          chunk_ranges(a.size)))


class OracleRun:
    """The oracle's side of a case over the whole shard."""

    def __init__(self, case: Case):
        self.case = case
        self.plan = oracle.plan(case.numels, case.world_size, case.rank, case.align,
                                case.bucket_elems)
        p = self.plan
        self.master = init_master_host(case, p.begin, p.real, p.S)
        self.m = np.zeros(p.S, np.float32)
        self.v = np.zeros(p.S, np.float32)
        self.param = init_param_host(case, p.P)
        self.scaler = oracle.Scaler(case.init_scale, dynamic=case.dynamic, window=case.window)
        self.t = 0
        self.flat = None

    def step(self, it: int):
        p, c = self.plan, self.case
        scale = self.scaler.value
        grads = host_model_grads(c, p, it, scale)
        self.flat = oracle.flatten(p, grads)
        ovf = oracle.adam_step(self.t + 1, scale, self.flat, c.grad_dtype, self.master, self.m,
                               self.v, **c.hparams())
        if not ovf:
            self.t += 1
            self._param_stale = True
        self.scaler.update(ovf)
        return ovf, grads, scale

    def params(self) -> np.ndarray:
        """The half parameter buffer.  After an applied step it holds the cast
        of the master as it is now (a skipped step changes neither), so the
        write-back is done once, when the buffer is looked at."""
        if getattr(self, "_param_stale", False):
            p = self.plan
            write_param_chunked(self.master, p.real, p.begin, 0, self.param,
                                self.case.param_dtype)
            self._param_stale = False
        return self.param


class DeviceRun:
    """The GPU side of a case (small and medium sizes: inputs copied from host).

    mode "sync":  zero_adam_step returns the flag; the host runs the scaler.
    mode "async": zero_adam_step_async on the device state; the test reads
                  the state back after every step to compare it."""

    def __init__(self, case: Case, device="cuda:0", mode: str = "sync"):
        import torch
        self.case = case
        self.dev = torch.device(device)
        self.plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                          case.bucket_elems)
        p = self.plan
        self.hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay,
                                case.adamw)
        self.master = torch.from_numpy(init_master_host(case, p.begin, p.real, p.S)).to(self.dev)
        self.m = torch.zeros(p.S, dtype=torch.float32, device=self.dev)
        self.v = torch.zeros(p.S, dtype=torch.float32, device=self.dev)
        pbits = init_param_host(case, p.P)
        self.param_full = torch.from_numpy(pbits.view(np.int16)).to(self.dev).view(
            torch_dtype(case.param_dtype))
        self.flat = torch.empty(max(p.S, 1), dtype=torch_dtype(case.grad_dtype), device=self.dev)
        self.scaler = z.LossScaler(case.init_scale, dynamic=case.dynamic, window=case.window)
        self.t = 0
        self.rng = np.random.default_rng(case.seed + 17)
        self.mode = mode
        if mode == "async":
            z.zero_state_upload(p, 0, self.scaler)

    def _param_args(self):
        p, c = self.plan, self.case
        if c.param_mode == "none":
            return None, 0
        if c.param_mode == "window":
            return self.param_full[p.begin:p.begin + max(p.real, 0)], p.begin
        return self.param_full, 0

    def step(self, it: int, grads_host: List[Optional[np.ndarray]]):
        import torch
        p, c = self.plan, self.case
        grads = [None if g is None else to_device_grad(g, c.grad_dtype, self.dev)
                 for g in grads_host]
        if c.flatten_mode == "all":
            z.zero_flatten_grads(p, -1, grads, self.flat)
        elif c.flatten_mode in ("buckets", "buckets_shuffled"):
            order = list(range(p.n_buckets))
            if c.flatten_mode == "buckets_shuffled":
                self.rng.shuffle(order)
            tb = p.tensor_buckets()
            for b in order:
                # only this bucket's tensors are passed, as a backward hook would
                gb = [g if (g is not None and tb[i] == b) else None for i, g in enumerate(grads)]
                z.zero_flatten_grads(p, b, gb, self.flat)
        elif c.flatten_mode == "scan":
            # fill the flat shard some other way (as a reduce-scatter would);
            # the step must then scan it for overflow before updating
            z.zero_flatten_grads(p, -1, grads, self.flat)
            other = torch.empty_like(self.flat)
            other.copy_(self.flat)
            self.flat = other
        else:
            raise ValueError(c.flatten_mode)
        param, base = self._param_args()
        scale = self.scaler.scale
        if self.mode == "async":
            z.zero_adam_step_async(p, self.hp, self.flat, self.master, self.m, self.v, param, base)
            st = z.zero_state_download(p, scaler=self.scaler)
            ovf = st.last_flag
            assert st.applied_steps == self.t + (1 - ovf)
            self.t = st.applied_steps
            return ovf, scale
        ovf = z.zero_adam_step(p, self.hp, self.t + 1, scale, self.flat, self.master, self.m,
                               self.v, param, base)
        if not ovf:
            self.t += 1
        z.zero_update_loss_scale(self.scaler, ovf)
        return ovf, scale

    def state_host(self):
        import torch
        torch.cuda.synchronize()
        p = self.plan
        return (self.master.cpu().numpy(), self.m.cpu().numpy(), self.v.cpu().numpy(),
                self.param_full.view(torch.int16).cpu().numpy().view(np.uint16),
                grad_bits_host(self.flat[:p.S], self.case.grad_dtype))


def compare_full(case: Case, steps: Optional[int] = None, check_every: int = 1,
                 label: str = "", mode: str = "sync") -> dict:
    """Run a case on both sides and compare after every (check_every-th) step.
    Returns a summary (exact-match flags and the max errors seen)."""
    steps = case.steps if steps is None else steps
    orc = OracleRun(case)
    gpu = DeviceRun(case, mode=mode)
    assert (gpu.plan.S, gpu.plan.begin, gpu.plan.real) == (orc.plan.S, orc.plan.begin,
                                                           orc.plan.real)
    worst = dict(master=0.0, m=0.0, v=0.0, param_ulp=0, bit_exact=True, skipped=0)
    for it in range(1, steps + 1):
        o_ovf, grads, o_scale = orc.step(it)
        g_ovf, g_scale = gpu.step(it, grads)
        assert g_scale == o_scale, f"{label} it={it}: loss scale {g_scale} vs oracle {o_scale}"
        assert g_ovf == o_ovf, f"{label} it={it}: overflow flag {g_ovf} vs oracle {o_ovf}"
        assert gpu.t == orc.t
        assert gpu.scaler.scale == orc.scaler.value
        worst["skipped"] += o_ovf
        if it % check_every and it != steps:
            continue
        compare_state(gpu, orc, worst, f"{label} it={it}")
    return worst


def compare_state(gpu: "DeviceRun", orc: OracleRun, worst: dict, where: str) -> None:
    """Compare the GPU's flat shard, master, moments and parameters with the
    oracle's after the same steps; update the worst-error summary."""
    case = orc.case
    gm, gmo, gv, gp, gf = gpu.state_host()
    S = orc.plan.S
    assert same_bits(gf[:S], orc.flat), f"{where}: flat gradient shard differs"
    for name, a, b in (("master", gm[:S], orc.master), ("m", gmo[:S], orc.m),
                       ("v", gv[:S], orc.v)):
        if same_bits(a.view(np.uint32), b.view(np.uint32)):
            continue                      # identical bits: zero error
        worst["bit_exact"] = False
        err = max_rel(a, b)
        worst[name] = max(worst[name], err)
        assert err <= REL_TOL, f"{where}: {name} max rel err {err}"
    if case.param_mode != "none":
        want = orc.params()
        if not same_bits(gp, want):
            worst["bit_exact"] = False
            du = ulp_diff(gp, want)
            worst["param_ulp"] = max(worst["param_ulp"], du)
            assert du <= ULP_TOL, f"{where}: params differ by {du} ulp"
