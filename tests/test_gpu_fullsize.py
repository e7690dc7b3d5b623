"""GPU vs oracle parity at the workloads' full sizes (and one tensor past 2^31
elements).

Whole shards (the _whole_shard runs): every element of the flat gradients,
master, moments and parameters after every step, and the flag and loss
scale, for the full-length runs of the large workloads in bench.py's launch
configuration: Llama-3-8B rank 3 (20 steps; all buckets at once, bucket by
bucket, graph-replayed; and 6 steps with fp32 gradients), the 20B DNA-LM
rank 2 (50 steps with the workload's injected infs, 25 of them graph-
replayed with the device-side scaler, and 3 steps with a +inf past 2^31),
Llama-2-70B rank 7 (5 steps, synchronous and graph-replayed) when the host
holds the oracle's ~121 GB, and a 5e9-element tensor whose shard starts past
2^31, 10 bytes off a 16-byte boundary.  The device state comes back through
pinned buffers, chunk by chunk, and the oracle runs over the same chunks on
host threads (the step is elementwise once the overflow decision, taken over
the whole shard first, is known).

Sampled windows (the _run_sampled runs): the Llama-2-70B step on any machine with
its device memory (and its graph-replayed step where the host cannot hold the
whole oracle state), the standalone cast and scan at that size, and the
offload pipeline on Llama-3-8B.  The oracle recomputes fixed windows of the
shard -- its head and tail, +-4096 elements around every segment edge, +-64
around every injected +inf, and 16 seeded random windows of 2^24 elements --
from the host generator; the update is elementwise, so a window evolves
exactly as it does inside the whole shard.  The overflow decision is global:
the windows contain every injected position, and the generator's support
(|z| <= 2*sqrt(3)) keeps every other gradient finite, which the test asserts
from the workload's constants, so the window's overflow test equals the
whole shard's.

Bar, after every step: flags, loss scale and applied-step counter equal;
flat gradients, master, moments and parameters bit-identical (within 1e-6
relative error and 1 ulp is the acceptance bound; identical bits are
expected and required).  Expected parameters come from the oracle's fp32
master through torch's round-to-nearest-even conversion, which equals the
oracle's own cast on all 2^32 fp32 inputs (tests/test_oracle_cast.py).

step_mode="graph" runs the step as bench.py's graph line does: flatten +
zero_adam_step_async captured once into a HIP graph and replayed every
iteration, with t and the loss scale held on the device (read back after
each replay only to compare with the oracle).
"""
import gc
import os
import threading
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
import zero_partitioned_mixed_plan_amd as z
from harness import (GRAD_WORD, INF_BITS, PARAM_FILL, ULP_TOL, Case, flat_offsets,
                     cast_library, grad_key, log, master_key, grad_bits_host, max_rel,
                     same_bits, torch_dtype, ulp_diff)
from synth.workloads import get

pytestmark = pytest.mark.gpu

HALF_MAX = {"f16": 65504.0, "bf16": 3.3895313892515355e38, "f32": 3.4028234663852886e38}


def _windows(op, case, n_random=16, rnd_len=1 << 24, seed=1):
    S, real = op.S, op.real
    ranges = [(0, 4096), (max(real - 4096, 0), S)]
    for so in op.seg_shard_off.tolist():
        ranges.append((so - 4096, so + 4096))
    for it in range(1, case.steps + 1):
        pos = case.injection(it, real)
        if pos is not None:
            ranges.append((pos - 64, pos + 64))
    rng = np.random.default_rng(seed)
    for _ in range(n_random):
        a = int(rng.integers(0, max(S - rnd_len, 1)))
        ranges.append((a, a + rnd_len))
    ranges = sorted((max(0, a), min(S, b)) for a, b in ranges if min(S, b) > max(0, a))
    merged = []
    for a, b in ranges:
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], b))
        else:
            merged.append((a, b))
    idx = np.concatenate([np.arange(a, b, dtype=np.int64) for a, b in merged])
    return merged, idx


class WindowOracle:
    """The oracle's step on the sampled windows of a shard, chunk by chunk on
    host threads.  The windows are split into pieces of <= 2^22 elements:
    positions [p0, p1) of the sampled arrays hold shard elements [s0, s0 +
    p1 - p0).  Gradients and the initial master come from the host generator
    at the same flat indices as the device's; the overflow decision is taken
    over every sampled gradient first, then the update runs per piece."""

    def __init__(self, op, case, pool):
        self.case, self.pool = case, pool
        self.S, self.real, self.begin = op.S, op.real, op.begin
        self.windows, self.idx = _windows(op, case)
        n = self.n = self.idx.size
        self.chunks = []
        for a, b in self.windows:
            for s0 in range(a, b, 1 << 22):
                p0 = self.chunks[-1][1] if self.chunks else 0
                self.chunks.append((p0, p0 + min(b, s0 + (1 << 22)) - s0, s0))
        assert self.chunks[-1][1] == n
        self.in_real = self.idx < self.real
        self.master = np.zeros(n, np.float32)
        self.m = np.zeros(n, np.float32)
        self.v = np.zeros(n, np.float32)
        self.flat = np.zeros(n, GRAD_WORD[case.grad_dtype])
        self.scaler = oracle.Scaler(case.init_scale, dynamic=case.dynamic, window=case.window)
        self.t = 0
        self.othresh = synth.outlier_thresh(case.outlier_p)

        def init(c):
            k = self._n_real(c)
            self.master[c[0]:c[0] + k] = synth.host_values(master_key(case), self.begin + c[2],
                                                           k, case.master_sigma)
        self._map(init)

    def _n_real(self, c):
        return max(0, min(c[1] - c[0], self.real - c[2]))

    def _map(self, fn):
        return list(self.pool.map(fn, self.chunks))

    def step(self, it, pos):
        """One iteration at the current scale, +inf at shard index pos (or
        None); returns the overflow flag."""
        case, scale = self.case, self.scaler.value
        key = grad_key(case, it)

        def gen(c):
            k = self._n_real(c)
            vals = synth.host_values(key, self.begin + c[2], k, case.grad_sigma, scale,
                                     self.othresh, case.outlier_mult)
            self.flat[c[0]:c[0] + k] = synth.grad_bits(vals, case.grad_dtype)
            self.flat[c[0] + k:c[1]] = 0
        self._map(gen)
        if pos is not None:
            self.flat[np.searchsorted(self.idx, pos)] = INF_BITS[case.grad_dtype]
        ovf = int(any(self._map(lambda c: oracle.nonfinite(self.flat[c[0]:c[1]],
                                                            case.grad_dtype))))
        if not ovf:
            t = self.t + 1

            def upd(c):
                lo, hi = c[0], c[1]
                oracle.adam_update(t, scale, self.flat[lo:hi], case.grad_dtype,
                                   self.master[lo:hi], self.m[lo:hi], self.v[lo:hi],
                                   **case.hparams())
            self._map(upd)
        self.scaler.update(ovf)
        self.t += 1 - ovf
        return ovf

    def params(self):
        """The half parameters of the windows' real elements: the oracle's
        fp32 master through a conversion equal to the oracle's cast on every
        fp32 input (cast_library)."""
        return cast_library(self.master[self.in_real], self.case.param_dtype)

    def differs(self, got):
        """Pieces where the device's flat / master / m / v (sampled arrays in
        `got`) are not bit-identical to the oracle's."""
        want = {"flat": self.flat, "master": self.master, "m": self.m, "v": self.v}

        def one(c):
            lo, hi = c[0], c[1]
            bad = []
            for name, a in got.items():
                a, b = a[lo:hi], want[name][lo:hi]
                if name == "flat":
                    if not np.array_equal(a, b):
                        bad.append(name)
                elif not np.array_equal(a.view(np.uint32), b.view(np.uint32)):
                    bad.append(f"{name} (max rel err {max_rel(a, b)})")
            return (c[2], bad) if bad else None
        return [r for r in self._map(one) if r is not None]


def _host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _mem_available():
    """Host memory available to a new allocation (MemAvailable), in bytes."""
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


def _run_sampled(case, flatten_mode="all", label="", step_mode="sync"):
    import torch
    dev = torch.device("cuda:0")
    gdt, pdt = torch_dtype(case.grad_dtype), torch_dtype(case.param_dtype)
    # finite by construction: the largest gradient the generator can draw
    bound = case.grad_sigma * 2 * np.sqrt(3) * 1.0001 * max(case.outlier_mult, 1.0) * \
        max(case.init_scale, 1.0)
    assert bound < HALF_MAX[case.grad_dtype]

    op = oracle.plan(case.numels, case.world_size, case.rank, case.align, case.bucket_elems)
    plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                 case.bucket_elems)
    assert (plan.S, plan.begin, plan.real, plan.n_segments) == (op.S, op.begin, op.real,
                                                               op.n_segments)
    S, real, begin = op.S, op.real, op.begin
    pool = ThreadPoolExecutor(_host_threads())
    wo = WindowOracle(op, case, pool)
    idx, n = wo.idx, wo.n
    log(f"[full] {label}: S={S} real={real} segments={op.n_segments} "
        f"windows={len(wo.windows)} sampled={n} pieces={len(wo.chunks)} "
        f"threads={pool._max_workers}")
    offs = flat_offsets(case.numels)

    # ---- GPU state (whole shard)
    master = torch.empty(S, dtype=torch.float32, device=dev)
    master[real:].zero_()
    synth.dev_fill_f32(master[:real], master_key(case), begin, case.master_sigma)
    mom = torch.zeros(S, dtype=torch.float32, device=dev)
    var = torch.zeros(S, dtype=torch.float32, device=dev)
    flat = torch.empty(S, dtype=gdt, device=dev)
    param = torch.full((max(real, 1),), float("nan"), dtype=pdt, device=dev)
    grads = [None] * len(case.numels)
    for s in range(op.n_segments):
        t = int(op.seg_tensor[s])
        if grads[t] is None:
            grads[t] = torch.empty(case.numels[t], dtype=gdt, device=dev)
    hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay, case.adamw)
    g_scaler = z.LossScaler(case.init_scale, dynamic=case.dynamic, window=case.window)
    tb = plan.tensor_buckets()
    d_idx = torch.from_numpy(idx).to(dev)
    d_ridx = d_idx[torch.from_numpy(wo.in_real).to(dev)]

    def flatten():
        if flatten_mode == "buckets":
            for b in range(plan.n_buckets):
                z.zero_flatten_grads(plan, b, [g if (g is not None and tb[i] == b) else None
                                               for i, g in enumerate(grads)], flat)
        else:
            z.zero_flatten_grads(plan, -1, grads, flat)

    graph = None
    if step_mode == "graph":
        z.zero_state_upload(plan, 0, g_scaler)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            flatten()
            z.zero_adam_step_async(plan, hp, flat, master, mom, var, param, begin)
        log(f"[full] {label}: flatten + asynchronous step captured")
    else:
        assert step_mode == "sync", step_mode

    g_t = o_t = skipped = 0
    othresh = synth.outlier_thresh(case.outlier_p)
    for it in range(1, case.steps + 1):
        t_step = time.perf_counter()
        scale = wo.scaler.value
        if graph is not None:
            st = z.zero_state_download(plan)
            assert st.applied_steps == o_t, f"{label} it={it}: t {st.applied_steps} vs {o_t}"
            assert st.scale == scale, f"{label} it={it}: device scale {st.scale} vs {scale}"
        else:
            assert g_scaler.scale == scale, f"{label} it={it}: scale {g_scaler.scale} vs {scale}"
        key = grad_key(case, it)
        pos = case.injection(it, real)
        # GPU inputs: every segment of the shard, drawn on the device
        for s in range(op.n_segments):
            t, a, nn = int(op.seg_tensor[s]), int(op.seg_tensor_off[s]), int(op.seg_numel[s])
            synth.dev_fill_half(grads[t][a:a + nn], key, int(offs[t]) + a, case.grad_sigma,
                                scale, othresh, case.outlier_mult)
        if pos is not None:
            s = int(np.searchsorted(op.seg_shard_off, pos, side="right") - 1)
            t = int(op.seg_tensor[s])
            grads[t][int(op.seg_tensor_off[s] + pos - op.seg_shard_off[s])] = float("inf")
        if graph is not None:
            graph.replay()
            st = z.zero_state_download(plan)
            g_ovf = int(st.last_flag)
            assert st.skipped_steps == skipped + g_ovf, f"{label} it={it}: skip count"
        else:
            flatten()
            g_ovf = z.zero_adam_step(plan, hp, g_t + 1, scale, flat, master, mom, var, param,
                                     begin)
            z.zero_update_loss_scale(g_scaler, g_ovf)

        # the oracle on the windows, from the host generator
        o_ovf = wo.step(it, pos)
        assert g_ovf == o_ovf, f"{label} it={it}: overflow {g_ovf} vs oracle {o_ovf}"
        g_t += 1 - g_ovf
        o_t += 1 - o_ovf
        skipped += o_ovf
        got = {"flat": grad_bits_host(flat.index_select(0, d_idx), case.grad_dtype),
               "master": master.index_select(0, d_idx).cpu().numpy(),
               "m": mom.index_select(0, d_idx).cpu().numpy(),
               "v": var.index_select(0, d_idx).cpu().numpy()}
        wrong = wo.differs(got)
        assert not wrong, f"{label} it={it}: windows differ: {wrong[:4]}"
        del got
        if o_t > 0:
            gp = param.index_select(0, d_ridx).view(torch.int16).cpu().numpy().view(np.uint16)
            op_bits = wo.params()
            if not same_bits(gp, op_bits):
                du = ulp_diff(gp, op_bits)
                assert du <= ULP_TOL, f"{label} it={it}: params differ by {du} ulp"
                raise AssertionError(f"{label} it={it}: params not bit-identical ({du} ulp)")
        log(f"[full] {label}: it={it} t={o_t} scale={scale} overflow={o_ovf}: windows equal "
            f"({time.perf_counter() - t_step:.1f} s)")
    pool.shutdown()
    if graph is not None:
        st = z.zero_state_download(plan)
        assert (st.applied_steps, st.scale) == (o_t, wo.scaler.value), f"{label}: final state"
    log(f"[full] {label}: done, skipped {skipped} of {case.steps}")
    del graph, master, mom, var, flat, param, grads, d_idx, d_ridx
    gc.collect()
    torch.cuda.empty_cache()
    return skipped


def _whole_70b_fits():
    """Whether this host holds the oracle's whole 70B-class shard (~121 GB of
    host memory) beside the device state (~160 GB)."""
    import torch
    free, _ = torch.cuda.mem_get_info()
    return _mem_available() >= 140e9 and free >= 170e9


def test_llama3_8b_rank3_bucketed_flatten():
    # one flatten call per bucket (19 buckets touch this shard), all 20 steps
    case = Case.from_workload(get("llama3_8b"))
    assert _whole_shard(case, "llama3_8b buckets", flatten_mode="buckets") == 0


def test_llama3_8b_rank3_fp32_gradients():
    # gradients kept in fp32 at full size: 4-byte flatten and update path
    case = Case.from_workload(get("llama3_8b"), grad_dtype="f32", steps=6)
    assert _whole_shard(case, "llama3_8b fp32 grads") == 0


def test_dna_20b_rank2_dynamic_scale_with_injected_overflows():
    # all 50 steps: fp16 at the dynamic scale, the workload's injected infs
    case = Case.from_workload(get("dna_20b"))
    expect = sum(case.injection(it, 2_498_481_408) is not None for it in range(1, case.steps + 1))
    assert _whole_shard(case, "dna_20b") == expect and expect >= 1


def test_llama3_8b_rank3_graph_replayed_step():
    case = Case.from_workload(get("llama3_8b"))
    assert _whole_shard(case, "llama3_8b graph", step_mode="graph") == 0


def test_dna_20b_rank2_graph_replayed_step_with_device_scaler():
    # the loss-scale policy runs on the device: skips and halvings at full
    # size; 25 of the workload's 50 steps hold all three of its injections
    case = Case.from_workload(get("dna_20b"), steps=25)
    expect = sum(case.injection(it, 2_498_481_408) is not None for it in range(1, case.steps + 1))
    assert _whole_shard(case, "dna_20b graph", step_mode="graph") == expect and expect >= 1


def test_llama2_70b_rank7_full_shard():
    # sampled windows: runs on any machine with the device memory
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 170e9:
        pytest.skip(f"needs ~160 GB of free device memory, {free / 1e9:.0f} GB free")
    case = Case.from_workload(get("llama2_70b"))
    _run_sampled(case, label="llama2_70b")


def test_llama2_70b_rank7_graph_replayed_step():
    # every element when the host holds the oracle's whole shard, else windows
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 170e9:
        pytest.skip(f"needs ~160 GB of free device memory, {free / 1e9:.0f} GB free")
    case = Case.from_workload(get("llama2_70b"))
    if _whole_70b_fits():
        assert _whole_shard(case, "llama2_70b graph", step_mode="graph") == 0
    else:
        _run_sampled(case, label="llama2_70b graph", step_mode="graph")


def test_llama2_70b_rank7_standalone_cast_and_scan():
    """The two kernels bench.py also times on their own, at the 70B shard's
    size: zero_write_param_shard, and the scan that zero_adam_step runs when
    its gradient buffer did not come from zero_flatten_grads (here it is
    filled directly).  A +inf 12,345 elements before the shard's end (past
    2^33) must skip the step with every sampled state and parameter bit
    unchanged; without it the step must match the oracle."""
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 150e9:
        pytest.skip(f"needs ~140 GB of free device memory, {free / 1e9:.0f} GB free")
    dev = torch.device("cuda:0")
    w = get("llama2_70b")
    op = oracle.plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
    S, real, begin = op.S, op.real, op.begin
    pos = S - 12_345
    assert pos > 1 << 33 and S == real
    case = Case.from_workload(w, steps=1, inject={1: pos})
    plan = z.zero_partition_plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
    pool = ThreadPoolExecutor(_host_threads())
    wo = WindowOracle(op, case, pool)
    idx = wo.idx
    log(f"[full] 70b cast+scan: S={S} windows={len(wo.windows)} sampled={idx.size}")
    d_idx = torch.from_numpy(idx).to(dev)
    pdt, gdt = torch_dtype(w.param_dtype), torch_dtype(w.grad_dtype)

    master = torch.empty(S, dtype=torch.float32, device=dev)
    synth.dev_fill_f32(master, master_key(case), begin, case.master_sigma)
    mom = torch.zeros(S, dtype=torch.float32, device=dev)
    var = torch.zeros(S, dtype=torch.float32, device=dev)
    fill = int(np.array(PARAM_FILL, np.uint16).view(np.int16))
    param = torch.full((S,), fill, dtype=torch.int16, device=dev).view(pdt)

    def bits16(t):
        return t.index_select(0, d_idx).view(torch.int16).cpu().numpy().view(np.uint16)

    def bits32(t):
        return t.index_select(0, d_idx).cpu().numpy().view(np.uint32)

    # standalone cast of the fp32 master shard to its window of the parameters
    z.zero_write_param_shard(plan, master, param, begin)
    want_p = wo.params()
    assert same_bits(bits16(param), want_p), "standalone cast differs"
    log("[full] 70b cast+scan: standalone cast ok")

    # gradients written straight into the flat buffer: the step must scan
    key = grad_key(case, 1)
    flat = torch.empty(S, dtype=gdt, device=dev)
    synth.dev_fill_half(flat, key, begin, case.grad_sigma)
    good = flat[pos].clone()
    flat[pos] = float("inf")
    hp = z.AdamHParams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.adamw)
    before = (bits32(master), bits32(mom), bits32(var))
    assert z.zero_adam_step(plan, hp, 1, 1.0, flat, master, mom, var, param, begin) == 1
    for name, a, b in zip(("master", "m", "v"), before, (bits32(master), bits32(mom),
                                                         bits32(var))):
        assert same_bits(a, b), f"skipped step changed {name}"
    assert same_bits(bits16(param), want_p), "skipped step changed the parameters"
    log("[full] 70b cast+scan: +inf found by the scan, step skipped")

    flat[pos] = good
    assert z.zero_adam_step(plan, hp, 1, 1.0, flat, master, mom, var, param, begin) == 0
    assert wo.step(1, None) == 0          # the oracle's step on the same (clean) gradients
    wrong = wo.differs({"flat": bits16(flat), "master": master.index_select(0, d_idx).cpu()
                        .numpy(), "m": mom.index_select(0, d_idx).cpu().numpy(),
                        "v": var.index_select(0, d_idx).cpu().numpy()})
    assert not wrong, f"the scanned step differs: {wrong[:4]}"
    assert same_bits(bits16(param), wo.params())
    log("[full] 70b cast+scan: scanned step ok")
    pool.shutdown()
    del master, mom, var, param, flat, d_idx
    gc.collect()
    torch.cuda.empty_cache()


def test_tensor_beyond_2_31_elements():
    # Rank 1 of 2 over tensors of 3, 4,999,999,990 and 7 elements: the shard
    # starts 2,499,999,997 elements into the middle tensor (past 2^31, and 10
    # bytes past a 16-byte boundary), so the flatten's source offsets need 64
    # bits and take the realigned path; the 7-element tensor puts a piece
    # edge inside the last tile.  The +inf of iteration 2 sits past 2^31 in
    # the shard.  About 50 GB of device memory.
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 60e9:
        pytest.skip(f"needs ~50 GB of free device memory, {free / 1e9:.0f} GB free")
    case = Case(numels=[3, 4_999_999_990, 7], world_size=2, rank=1, grad_dtype="bf16",
                param_dtype="bf16", steps=3, inject={2: 2_300_000_000})
    assert _whole_shard(case, "5e9-element tensor") == 1


def _offload_sampled(case, lag, label, n_threads=8):
    """The ZeRO-Offload pipeline over a full-size shard, checked on the same
    sampled windows: each iteration's stand-in forward must see exactly the
    oracle's parameters after iteration it - 1 - lag, and after the drain the
    host master / moments and the device parameters must equal the oracle's
    bit for bit there."""
    import torch
    dev = torch.device("cuda:0")
    gdt, pdt = torch_dtype(case.grad_dtype), torch_dtype(case.param_dtype)
    op = oracle.plan(case.numels, case.world_size, case.rank, case.align, case.bucket_elems)
    plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                 case.bucket_elems)
    S, real, begin = op.S, op.real, op.begin
    assert (plan.S, plan.begin, plan.real) == (S, begin, real)
    pool = ThreadPoolExecutor(_host_threads())
    wo = WindowOracle(op, case, pool)
    idx = wo.idx
    ridx = idx[wo.in_real]
    log(f"[full] {label}: S={S} real={real} lag={lag} threads={n_threads} "
        f"windows={len(wo.windows)} sampled={idx.size}")
    offs = flat_offsets(case.numels)

    # ---- host state of the offloaded step (drawn by the device generator,
    # cross-checked against the host one elsewhere), device buffers
    dm = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.dev_fill_f32(dm[:real], master_key(case), begin, case.master_sigma)
    master = dm.cpu().numpy()
    del dm
    mom = np.zeros(S, np.float32)
    var = np.zeros(S, np.float32)
    param = torch.zeros(max(real, 1), dtype=pdt, device=dev)   # window at shard_begin
    flat = torch.empty(S, dtype=gdt, device=dev)
    grads = [None] * len(case.numels)
    for s in range(op.n_segments):
        t = int(op.seg_tensor[s])
        if grads[t] is None:
            grads[t] = torch.empty(case.numels[t], dtype=gdt, device=dev)
    hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay, case.adamw)
    z.zero_state_upload(plan, 0, z.LossScaler(case.init_scale, dynamic=case.dynamic,
                                              window=case.window))
    off = z.Offload(plan, hp, case.grad_dtype, case.param_dtype, master, mom, var,
                    n_threads=n_threads)
    d_ridx = torch.from_numpy(ridx).to(dev)
    skipped = 0
    othresh = synth.outlier_thresh(case.outlier_p)
    hist = [np.zeros(ridx.size, np.uint16)]   # the windows' parameters after iteration k
    for it in range(1, case.steps + 1):
        off.wait_params(lag)
        seen = param.index_select(0, d_ridx).view(torch.int16).cpu().numpy().view(np.uint16)
        assert same_bits(seen, hist[max(it - 1 - lag, 0)]), \
            f"{label} it={it}: the forward saw other parameters than iteration {it - 1 - lag}'s"
        scale = wo.scaler.value
        st = z.zero_state_download(plan)
        assert st.scale == scale, f"{label} it={it}: device scale {st.scale} vs {scale}"
        key = grad_key(case, it)
        pos = case.injection(it, real)
        for s in range(op.n_segments):
            t, a, n = int(op.seg_tensor[s]), int(op.seg_tensor_off[s]), int(op.seg_numel[s])
            synth.dev_fill_half(grads[t][a:a + n], key, int(offs[t]) + a, case.grad_sigma, scale,
                                othresh, case.outlier_mult)
        if pos is not None:
            s = int(np.searchsorted(op.seg_shard_off, pos, side="right") - 1)
            t = int(op.seg_tensor[s])
            grads[t][int(op.seg_tensor_off[s] + pos - op.seg_shard_off[s])] = float("inf")
        z.zero_flatten_grads(plan, -1, grads, flat)
        off.submit(flat, param, begin)
        o_ovf = wo.step(it, pos)
        skipped += o_ovf
        hist.append(hist[-1] if o_ovf else wo.params())
        log(f"[full] {label}: it={it} submitted, oracle overflow {o_ovf}")
    off.drain()
    stats = off.stats()
    assert stats["applied"] == wo.t and stats["skipped"] == skipped, stats
    st = z.zero_state_download(plan)
    assert (st.applied_steps, st.skipped_steps, st.scale) == (wo.t, skipped, wo.scaler.value)
    wrong = wo.differs({"master": master[idx], "m": mom[idx], "v": var[idx]})
    assert not wrong, f"{label}: host state differs: {wrong[:4]}"
    final = param.index_select(0, d_ridx).view(torch.int16).cpu().numpy().view(np.uint16)
    assert same_bits(final, hist[-1]), f"{label}: final parameters differ"
    off.close()
    pool.shutdown()
    log(f"[full] {label}: ok, applied {wo.t}, skipped {skipped}, "
        f"host ms last {stats['host_ms_last']:.1f}")
    del param, flat, grads, d_ridx, master, mom, var
    gc.collect()
    torch.cuda.empty_cache()
    return skipped


@pytest.mark.parametrize("lag", [1, 0])
def test_llama3_8b_rank3_offload(lag):
    # bench.py's offload workload at its full size (16 pieces of the shard),
    # with a +inf at iteration 3 so one step is skipped
    case = Case.from_workload(get("llama3_8b"), steps=5, inject={3: 700_000_001})
    assert _offload_sampled(case, lag, f"llama3_8b offload lag={lag}") == 1


def _whole_shard(case, label, step_mode="sync", flatten_mode="all"):
    """Every element of the shard after every step: the flat gradients,
    master, moments and parameters bit for bit, and the overflow flag and
    loss scale.  The oracle runs over contiguous chunks of the shard on host
    threads (the step is elementwise once the overflow decision, taken over
    the whole shard first, is known); its gradients come from the host
    generator at the same flat indices as the device's, with the same +inf.
    The device's state comes back through pinned buffers, chunk by chunk.
    step_mode="graph": flatten + zero_adam_step_async replayed from a HIP
    graph, t and the scale on the device.  flatten_mode="buckets": one
    zero_flatten_grads call per bucket, each given only that bucket's
    gradient tensors, as backward hooks would call it."""
    import torch
    dev = torch.device("cuda:0")
    gdt, pdt = torch_dtype(case.grad_dtype), torch_dtype(case.param_dtype)
    op = oracle.plan(case.numels, case.world_size, case.rank, case.align, case.bucket_elems)
    plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                 case.bucket_elems)
    S, real, begin = op.S, op.real, op.begin
    assert (plan.S, plan.begin, plan.real) == (S, begin, real)
    chunk = 1 << 24
    chunks = [(lo, min(S, lo + chunk)) for lo in range(0, S, chunk)]
    pool = ThreadPoolExecutor(_host_threads())
    log(f"[whole] {label}: S={S} real={real} chunks={len(chunks)} threads={pool._max_workers}")
    offs = flat_offsets(case.numels)
    othresh = synth.outlier_thresh(case.outlier_p)

    master = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.dev_fill_f32(master[:real], master_key(case), begin, case.master_sigma)
    mom = torch.zeros(S, dtype=torch.float32, device=dev)
    var = torch.zeros(S, dtype=torch.float32, device=dev)
    flat = torch.empty(S, dtype=gdt, device=dev)
    param = torch.empty(max(real, 1), dtype=pdt, device=dev)   # window at shard_begin
    grads = [None] * len(case.numels)
    for s in range(op.n_segments):
        t = int(op.seg_tensor[s])
        if grads[t] is None:
            grads[t] = torch.empty(case.numels[t], dtype=gdt, device=dev)
    hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay, case.adamw)
    g_scaler = z.LossScaler(case.init_scale, dynamic=case.dynamic, window=case.window)
    tb = plan.tensor_buckets()

    def flatten():
        if flatten_mode == "buckets":
            for b in range(plan.n_buckets):
                z.zero_flatten_grads(plan, b, [g if (g is not None and tb[i] == b) else None
                                               for i, g in enumerate(grads)], flat)
        else:
            assert flatten_mode == "all", flatten_mode
            z.zero_flatten_grads(plan, -1, grads, flat)

    graph = None
    if step_mode == "graph":
        z.zero_state_upload(plan, 0, g_scaler)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            flatten()
            z.zero_adam_step_async(plan, hp, flat, master, mom, var, param, begin)
    else:
        assert step_mode == "sync", step_mode

    o_master = np.zeros(S, np.float32)
    o_m = np.zeros(S, np.float32)
    o_v = np.zeros(S, np.float32)
    word = GRAD_WORD[case.grad_dtype]           # uint16, or uint32 for fp32 gradients
    flat_bits = torch.int32 if case.grad_dtype == "f32" else torch.int16
    bits = np.zeros(S, word)

    def init(c):
        lo, hi = c[0], min(c[1], real)
        if hi > lo:
            o_master[lo:hi] = synth.host_values(master_key(case), begin + lo, hi - lo,
                                                case.master_sigma)

    list(pool.map(init, chunks))
    o_scaler = oracle.Scaler(case.init_scale, dynamic=case.dynamic, window=case.window)
    staging = threading.local()

    def fetch(t, name):
        """A device slice's contents on the host, through a pinned buffer of
        the calling thread (synchronous copy)."""
        bufs = getattr(staging, "bufs", None)
        if bufs is None:
            bufs = staging.bufs = {}
        buf = bufs.get(name)
        if buf is None:
            buf = bufs[name] = torch.empty(chunk, dtype=t.dtype, pin_memory=True)
        dst = buf[:t.numel()]
        dst.copy_(t)
        return dst.numpy()

    g_t = o_t = skipped = 0
    for it in range(1, case.steps + 1):
        t_step = time.perf_counter()
        scale = o_scaler.value
        if graph is not None:
            st = z.zero_state_download(plan)
            assert (st.applied_steps, st.scale) == (o_t, scale), f"{label} it={it}: state"
        else:
            assert g_scaler.scale == scale, f"{label} it={it}: scale {g_scaler.scale} vs {scale}"
        key = grad_key(case, it)
        pos = case.injection(it, real)
        for s in range(op.n_segments):
            t, a, n = int(op.seg_tensor[s]), int(op.seg_tensor_off[s]), int(op.seg_numel[s])
            synth.dev_fill_half(grads[t][a:a + n], key, int(offs[t]) + a, case.grad_sigma, scale,
                                othresh, case.outlier_mult)
        if pos is not None:
            s = int(np.searchsorted(op.seg_shard_off, pos, side="right") - 1)
            t = int(op.seg_tensor[s])
            grads[t][int(op.seg_tensor_off[s] + pos - op.seg_shard_off[s])] = float("inf")
        if graph is not None:
            graph.replay()
            g_ovf = int(z.zero_state_download(plan).last_flag)
        else:
            flatten()
            g_ovf = z.zero_adam_step(plan, hp, g_t + 1, scale, flat, master, mom, var, param,
                                     begin)
            z.zero_update_loss_scale(g_scaler, g_ovf)

        def gen(c):
            lo, hi = c[0], min(c[1], real)
            if hi > lo:
                bits[lo:hi] = synth.grad_bits(
                    synth.host_values(key, begin + lo, hi - lo, case.grad_sigma, scale, othresh,
                                      case.outlier_mult), case.grad_dtype)
                if pos is not None and lo <= pos < hi:
                    bits[pos] = INF_BITS[case.grad_dtype]
            return oracle.nonfinite(bits[c[0]:c[1]], case.grad_dtype)

        o_ovf = int(any(list(pool.map(gen, chunks))))
        if not o_ovf:
            def upd(c):
                lo, hi = c
                oracle.adam_update(o_t + 1, scale, bits[lo:hi], case.grad_dtype,
                                   o_master[lo:hi], o_m[lo:hi], o_v[lo:hi], **case.hparams())
            list(pool.map(upd, chunks))
        o_scaler.update(o_ovf)
        assert g_ovf == o_ovf, f"{label} it={it}: overflow {g_ovf} vs oracle {o_ovf}"
        g_t += 1 - g_ovf
        o_t += 1 - o_ovf
        skipped += o_ovf
        torch.cuda.synchronize(dev)

        def check(c):
            lo, hi = c
            bad = []
            got = fetch(flat[lo:hi].view(flat_bits), "flat").view(word)
            if not np.array_equal(got, bits[lo:hi]):
                bad.append("flat")
            for name, d, o in (("master", master, o_master), ("m", mom, o_m), ("v", var, o_v)):
                got = fetch(d[lo:hi], name)
                if not np.array_equal(got.view(np.uint32), o[lo:hi].view(np.uint32)):
                    bad.append(f"{name} (max rel err {max_rel(got, o[lo:hi])})")
            hi = min(hi, real)
            if o_t > 0 and hi > lo:
                got = fetch(param[lo:hi].view(torch.int16), "param").view(np.uint16)
                if not np.array_equal(got, cast_library(o_master[lo:hi], case.param_dtype,
                                                        parallel=False)):
                    bad.append("param")
            return (lo, bad) if bad else None

        wrong = [r for r in pool.map(check, chunks) if r is not None]
        assert not wrong, f"{label} it={it}: chunks differ: {wrong[:4]}"
        log(f"[whole] {label}: it={it} t={o_t} scale={scale} overflow={o_ovf}: "
            f"every element equal ({time.perf_counter() - t_step:.1f} s)")
    pool.shutdown()
    del staging
    if graph is not None:
        st = z.zero_state_download(plan)
        assert (st.applied_steps, st.skipped_steps, st.scale) == (o_t, skipped, o_scaler.value)
    del graph, master, mom, var, flat, param, grads
    gc.collect()
    torch.cuda.empty_cache()
    return skipped


def test_llama3_8b_rank3_whole_shard_every_step():
    # all 20 steps of the workload, with its 1% x100 outliers
    case = Case.from_workload(get("llama3_8b"))
    assert case.steps == 20
    assert _whole_shard(case, "llama3_8b") == 0


def test_dna_20b_rank2_whole_shard_every_step():
    # fp16 gradients at the dynamic scale, 300 pieces, a +inf at iteration 2
    case = Case.from_workload(get("dna_20b"), steps=3, inject_p=0.0,
                              inject={2: 2_000_000_017})
    assert _whole_shard(case, "dna_20b") == 1


@pytest.mark.timeout(1200)
def test_llama2_70b_rank7_whole_shard_every_step():
    """Every element of the 8.6e9-element shard after each of the workload's
    5 steps.  The oracle's state (fp32 master, moments, gradient bits) takes
    ~121 GB of host memory and the device ~155 GB."""
    if not _whole_70b_fits():
        pytest.skip(f"needs ~140 GB of available host memory and ~170 GB of free device "
                    f"memory ({_mem_available() / 1e9:.0f} GB available on the host)")
    case = Case.from_workload(get("llama2_70b"))
    assert case.steps == 5
    assert _whole_shard(case, "llama2_70b") == 0
