"""Throughput of one rank's partitioned mixed-precision Adam step on one MI355X.

A step is the whole hot path over one batch of gradients already resident in
HBM: bucketed flatten of the half gradients into the rank's flat shard (with
the fused inf/NaN test), the gated fused unscale + AdamW + bf16 cast, and the
loss-scale update.  Default workload: Llama-2-70B shaped parameters (80
layers, d=8192, ffn 28672, 8 kv heads, vocab 32000; 68,976,648,192 elements),
R=8, rank 7, whose shard holds 8,622,081,024 elements (~138 GB of model
state on the GPU); bf16 gradients N(0, 1e-3), fp32 master N(0, 0.02).

Prints one JSON line.  ``value`` is shard parameters updated per second over
the timed steps (wall clock, synchronized on both sides).  ``roofline``
prices the fused Adam kernel at 28 algorithmic bytes per shard element
against 8 TB/s, from HIP events recorded around the kernel on its launch
stream; its ``traffic`` is the counter-measured HBM bytes per launch from
the committed rocprofv3 summary under profiles/, reported only while the
kernel source is the one that summary measured.  ``cpu_baseline`` times the
oracle (single thread) on a bounded window of the same shard.
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ADAM_BYTES_PER_ELEM = 28      # read grad 2 + master/m/v 12; write master/m/v 12 + param 2
FLATTEN_BYTES_PER_ELEM = 4    # read 2 + write 2
GRAD_BYTES = {"f16": 2, "bf16": 2, "f32": 4}


def adam_bytes(gdt: str) -> int:
    """Algorithmic bytes per element of the fused update: the gradient, 12 B of
    fp32 state read and written, the half parameter written."""
    return ADAM_BYTES_PER_ELEM - 2 + GRAD_BYTES[gdt]


def flatten_bytes(gdt: str) -> int:
    return 2 * GRAD_BYTES[gdt]


METRIC = "shard params/sec per Adam step + achieved HBM GB/s (% of peak), 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _ensure_built():
    libs = [os.path.join(ROOT, "zero_partitioned_mixed_plan_amd", "libzero_mi355x.so"),
            os.path.join(ROOT, "synth", "libsynth_dev.so"),
            os.path.join(ROOT, "synth", "libsynth_host.so"),
            os.path.join(ROOT, "oracle", "liboracle.so")]
    if not all(os.path.exists(p) for p in libs):
        import __graft_entry__
        __graft_entry__.build()


def setup(w, device):
    """Allocate and fill the shard state and the gradient tensors on the GPU."""
    import torch

    import synth
    import zero_partitioned_mixed_plan_amd as z

    plan = z.zero_partition_plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
    S, real, begin = plan.S, plan.real, plan.begin
    gdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.grad_dtype]
    pdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.param_dtype]
    segs = plan.segments()
    touched = sorted({s.tensor for s in segs})
    grad_elems = sum(w.numels[i] for i in touched)
    gb = GRAD_BYTES[w.grad_dtype]
    need = S * (12 + gb) + real * 2 + grad_elems * gb + (1 << 29)
    free, total = torch.cuda.mem_get_info(device)
    log(f"[bench] {w.name}: S={S} real={real} segments={len(segs)} buckets={plan.n_buckets} "
        f"device bytes needed ~{need / 1e9:.1f} GB, free {free / 1e9:.1f} GB")
    if need > free:
        raise SystemExit(f"not enough device memory: need {need / 1e9:.1f} GB, "
                         f"free {free / 1e9:.1f} GB")
    master = torch.empty(S, dtype=torch.float32, device=device)
    m = torch.zeros(S, dtype=torch.float32, device=device)
    v = torch.zeros(S, dtype=torch.float32, device=device)
    flat = torch.empty(S, dtype=gdt, device=device)
    param = torch.empty(max(real, 1), dtype=pdt, device=device)
    master[real:].zero_()
    synth.dev_fill_f32(master[:real], synth.key(w.seed, synth.STREAM_MASTER, 0), begin,
                       w.master_sigma)
    grads = [None] * len(w.numels)
    offs = [0]
    for n in w.numels:
        offs.append(offs[-1] + n)
    gkey = synth.key(w.seed, synth.STREAM_GRAD, 1)
    scale = w.init_scale if w.dynamic_scale else 1.0
    for s in segs:
        i = s.tensor
        if grads[i] is None:
            grads[i] = torch.empty(w.numels[i], dtype=gdt, device=device)
        part = grads[i][s.tensor_off:s.tensor_off + s.numel]
        synth.dev_fill_half(part, gkey, offs[i] + s.tensor_off, w.grad_sigma, scale,
                            synth.outlier_thresh(w.outlier_p), w.outlier_mult)
    torch.cuda.synchronize(device)
    # bound once, as a training loop that keeps its gradient buffers does
    return plan, master, m, v, flat, param, z.GradList(plan, grads)


def run_gpu(w, steps, warmup, device, step_log=None):
    """The synchronous step, `steps` timed after `warmup`.  step_log: a file
    that receives one JSON line per timed step (t, overflow, scale, kernel
    times and rates)."""
    import torch

    import zero_partitioned_mixed_plan_amd as z

    plan, master, m, v, flat, param, grads = setup(w, device)
    hp = z.AdamHParams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.adamw)
    scaler = z.LossScaler(w.init_scale if w.dynamic_scale else 1.0, dynamic=w.dynamic_scale)
    plan.set_timing(True)
    state = {"t": 0, "skipped": 0}

    def one_step(times=None):
        z.zero_flatten_grads(plan, -1, grads, flat)
        scale_used = scaler.scale
        ovf = z.zero_adam_step(plan, hp, state["t"] + 1, scale_used, flat, master, m, v,
                               param, plan.begin)
        z.zero_update_loss_scale(scaler, ovf)
        if ovf:
            state["skipped"] += 1
        else:
            state["t"] += 1
        if times is not None:
            # kernel statistics over applied steps only: a skipped step's update
            # kernel returns at once (the per-step log keeps every step)
            fl, ad = plan.kernel_ms(0), plan.kernel_ms(2)
            if not ovf:
                times["flatten"].append(fl)
                times["adam"].append(ad)
            times["rec"].append((state["t"], int(ovf), scale_used, scaler.scale, fl, ad))

    for i in range(warmup):
        one_step()
        log(f"[bench] warmup step {i + 1}/{warmup} done")
    torch.cuda.synchronize(device)
    times = {"flatten": [], "adam": [], "rec": []}
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(times)
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    log(f"[bench] timed {steps} steps in {wall:.3f} s; skipped {state['skipped']}")
    if step_log is not None:   # written after the timed region
        ab, fb = adam_bytes(w.grad_dtype), flatten_bytes(w.grad_dtype)
        for i, (t, ovf, sc_used, sc_next, fl, ad) in enumerate(times["rec"], 1):
            gbs = ab * plan.S / (ad * 1e-3) / 1e9
            step_log.write(json.dumps({
                "step": i, "t": t, "overflow": ovf, "scale_used": sc_used, "scale_next": sc_next,
                "flatten_ms": fl, "adam_ms": ad, "params_per_s": plan.S / (ad * 1e-3),
                "adam_gbps": gbs, "adam_pct_peak": 100.0 * gbs / HBM_PEAK_GBS,
                "flatten_gbps": fb * plan.S / (fl * 1e-3) / 1e9}) + "\n")
        step_log.flush()
    return plan, wall, times, state, (plan, master, m, v, flat, param, grads, hp, scaler)


def run_graph(bufs, steps, warmup, device):
    """The same step without host round trips: the state goes to the device,
    flatten + zero_adam_step_async are captured once into a HIP graph, and
    `steps` replays are timed (synchronized on both sides)."""
    import torch

    import zero_partitioned_mixed_plan_amd as z

    plan, master, m, v, flat, param, grads, hp, scaler = bufs
    z.zero_state_upload(plan, 0, scaler)
    before = z.zero_state_download(plan)

    def step():
        z.zero_flatten_grads(plan, -1, grads, flat)
        z.zero_adam_step_async(plan, hp, flat, master, m, v, param, plan.begin)

    # eager asynchronous steps first: their update kernel (scalars read from
    # device memory) is timed with HIP events like the synchronous one
    dev_ms = []
    for _ in range(max(warmup, 2)):
        step()
        dev_ms.append(plan.kernel_ms(2))
    torch.cuda.synchronize(device)
    # captured without the plan's timing events, as a caller would capture it
    plan.set_timing(False)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize(device)
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    after = z.zero_state_download(plan)
    done = (after.applied_steps + after.skipped_steps) - (before.applied_steps +
                                                          before.skipped_steps)
    assert done == steps + warmup + max(warmup, 2), (done, steps, warmup)
    plan.set_timing(True)
    log(f"[bench] graph: {steps} replays in {wall:.3f} s; skipped {after.skipped_steps}")
    return wall, sum(dev_ms[1:]) / len(dev_ms[1:])


def time_bucketed_flatten(bufs, reps=5):
    """The flatten as a training loop overlapping backward would call it:
    one call per bucket of the shard, in bucket order (the reverse of
    registration order), bracketed as a whole by HIP events on the stream
    the calls are enqueued on.  Returns the call count and the median time
    of the whole sequence."""

    import torch

    import zero_partitioned_mixed_plan_amd as z

    plan, master, m, v, flat, param, grads, hp, scaler = bufs
    buckets = sorted({s.bucket for s in plan.segments()})
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    plan.set_timing(False)  # no per-call timing events: two of them cost ~7 us a call
    for r in range(reps + 1):
        e0.record()
        for b in buckets:
            z.zero_flatten_grads(plan, b, grads, flat)
        e1.record()
        e1.synchronize()
        if r:
            times.append(e0.elapsed_time(e1))
    plan.set_timing(True)
    # the bookkeeping now says every bucket was flattened into `flat`, as the
    # one-call flatten leaves it
    return len(buckets), statistics.median(times)


def time_standalone_kernels(bufs, reps=5):
    """The kernels the default step does not run, median of `reps` launches
    each: the standalone parameter cast (6 B/element) and the overflow scan
    of a flat shard that was not flattened this step (2 B/element; it runs
    inside a zero_adam_step, whose update is timed separately)."""
    import zero_partitioned_mixed_plan_amd as z

    plan, master, m, v, flat, param, grads, hp, scaler = bufs
    write_ms, scan_ms = [], []
    for _ in range(reps):
        z.zero_write_param_shard(plan, master, param, plan.begin)
        write_ms.append(plan.kernel_ms(3))
    for _ in range(reps):
        z.zero_adam_step(plan, hp, 1, scaler.scale, flat, master, m, v, param, plan.begin)
        scan_ms.append(plan.kernel_ms(1))
    return statistics.median(write_ms), statistics.median(scan_ms)


def forward_stand_in(forward_ms, device):
    """A fixed amount of GPU work that stands in for a step's forward and
    backward passes: a chain of 8192 x 8192 x 8192 bf16 products on the
    current stream, sized from a timed sample to take about forward_ms.
    Returns (run, gemms, measured ms per run)."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=device, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=device, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=device, dtype=torch.bfloat16)

    def gemms(k):
        for _ in range(k):
            torch.mm(a, b, out=c)

    def timed(k):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gemms(k)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1)

    gemms(3)
    per = timed(20) / 20
    k = max(1, round(forward_ms / per))
    return (lambda: gemms(k)), k, timed(k)


def _merged(iv):
    """Union of [start, end) intervals as sorted disjoint ones."""
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _length(iv):
    return sum(b - a for a, b in _merged(iv))


def _overlap(x, y):
    """Length of the intersection of two interval sets."""
    x, y = _merged(x), _merged(y)
    i = j = 0
    tot = 0.0
    while i < len(x) and j < len(y):
        a, b = max(x[i][0], y[j][0]), min(x[i][1], y[j][1])
        tot += max(0.0, b - a)
        if x[i][1] < y[j][1]:
            i += 1
        else:
            j += 1
    return tot


def timeline_summary(tl):
    """Per submitted step, from the pipeline's own timeline: time spent
    copying (gradients to the host, parameters back), updating on the host,
    and how much of the copying ran while the host update of the same step
    ran; medians over the steps after the first."""
    steps = sorted({r["step"] for r in tl})
    rows = []
    for j in steps:
        g = [(r["start_ms"], r["end_ms"]) for r in tl
             if r["step"] == j and r["kind"] == "gradient copy"]
        u = [(r["start_ms"], r["end_ms"]) for r in tl
             if r["step"] == j and r["kind"] == "host update"]
        h = [(r["start_ms"], r["end_ms"]) for r in tl
             if r["step"] == j and r["kind"] == "parameter copy"]
        if not u:
            continue
        allv = g + u + h
        rows.append({"gradient_copy_ms": _length(g), "host_update_ms": _length(u),
                     "parameter_copy_ms": _length(h),
                     "copies_during_update_ms": _overlap(g + h, u),
                     "span_ms": max(b for _, b in allv) - min(a for a, _ in allv),
                     "pieces": len(u)})
    rows = rows[1:] if len(rows) > 1 else rows
    if not rows:
        return None
    return {k: statistics.median(r[k] for r in rows) for k in rows[0]} | {"steps": len(rows)}


def run_offload(w, steps, warmup, device, n_threads, forward_ms=0.0, timeline_file=None):
    """ZeRO-Offload: fp32 master / moments in host memory, the update on the
    host cores, gradients and parameters crossing PCIe; timed with the
    one-step delayed update (lag 1) and serialised (lag 0).  forward_ms > 0
    puts a stand-in for the forward and backward passes on the GPU before
    each step, which the delayed update overlaps with the host update."""
    import numpy as np
    import torch

    import zero_partitioned_mixed_plan_amd as z

    plan, dmaster, dm, dv, flat, param, grads = setup(w, device)
    del dm, dv
    S, real, begin = plan.S, plan.real, plan.begin
    master = np.zeros(S, np.float32)
    master[:real] = dmaster[:real].cpu().numpy()
    del dmaster
    torch.cuda.empty_cache()
    hp = z.AdamHParams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.adamw)
    out = {"isa": z.zero_cpu_isa(), "host_threads": n_threads}
    forward = None
    if forward_ms > 0:
        forward, k, measured = forward_stand_in(forward_ms, device)
        out["forward"] = {"what": "8192^3 bf16 torch.mm chain before each step, standing in "
                                  "for the forward and backward passes",
                          "gemms_per_step": k, "ms_alone": measured}
    timelines = {}
    # the host's own streaming rate, taken before and after the timed lags
    # (host rates drift within a run); past the caches at every shard size
    ceiling_bytes = min(max(14 * S, 1 << 30), 4 << 30)
    before = host_stream_ceiling(ceiling_bytes, n_threads)
    for lag in (1, 0):
        m = np.zeros(S, np.float32)
        v = np.zeros(S, np.float32)
        scaler = z.LossScaler(w.init_scale if w.dynamic_scale else 1.0, dynamic=w.dynamic_scale)
        z.zero_state_upload(plan, 0, scaler)
        off = z.Offload(plan, hp, w.grad_dtype, w.param_dtype, master, m, v, n_threads=n_threads)

        def step():
            off.wait_params(lag)
            if forward is not None:
                forward()
            z.zero_flatten_grads(plan, -1, grads, flat)
            off.submit(flat, param, begin)

        for _ in range(warmup):
            step()
        off.drain()
        # short steps: time enough of them (>= 0.5 s) that refilling the
        # pipeline after the drain does not weigh on the average
        n = steps
        while True:
            if timeline_file:
                off.timeline_start()
            s0 = off.stats()
            t0 = time.perf_counter()
            for _ in range(n):
                step()
            off.drain()
            wall = time.perf_counter() - t0
            if wall >= 0.5 or n >= 5000:
                break
            n = min(5000, max(n + 1, int(n * 0.6 / max(wall, 1e-6))))
        st = off.stats()
        host_ms = (st["host_ms_total"] - s0["host_ms_total"]) / n
        tl = off.timeline() if timeline_file else None
        off.close()
        out[f"lag{lag}"] = {"timed_steps": n,
                            "ms_per_step": wall * 1000.0 / n, "host_update_ms": host_ms,
                            "value": real / (wall / n),
                            "host_update_params_per_s": S / (host_ms * 1e-3),
                            "host_update_gbps": adam_bytes(w.grad_dtype) * S / (host_ms * 1e-3) / 1e9,
                            # per step: where the worker and the caller wait
                            "waits_ms": {k[:-len("_ms_total")]: (st[k] - s0[k]) / n
                                         for k in ("wait_submit_ms_total",
                                                   "wait_grad_ms_total", "wait_h2d_ms_total",
                                                   "wait_release_ms_total",
                                                   "caller_wait_ms_total")}}
        if tl is not None:
            out[f"lag{lag}"]["timeline"] = timeline_summary(tl)
            timelines[f"lag{lag}"] = tl
        log(f"[bench] offload lag={lag}: {out[f'lag{lag}']}")
    if timeline_file:
        with open(timeline_file, "w") as f:
            json.dump({"workload": w.name, "forward_ms": forward_ms, **timelines}, f)
    after = host_stream_ceiling(ceiling_bytes, n_threads)
    best = max(before["gbps"], after["gbps"])
    out["host_ceiling"] = {"what": before["what"], "bytes": before["bytes"],
                           "threads": n_threads, "gbps_before": before["gbps"],
                           "gbps_after": after["gbps"], "gbps": best}
    for lag in (1, 0):
        out[f"lag{lag}"]["host_update_frac"] = out[f"lag{lag}"]["host_update_gbps"] / best
    return plan, out


def host_stream_ceiling(nbytes, n_threads, reps=7):
    """The host DRAM rate that the host update's traffic can reach on the same
    threads. The update reads 14 and writes 14 bytes per element, and every
    state line it reads it writes back. An in-place fp32 scale has the same
    mix: each line is read once and written back once, with no read for
    ownership. nbytes of memory are split into n_threads contiguous chunks,
    which are first touched and then scaled by the threads at once (numpy's
    ufunc loops release the GIL). A pass moves 2 * nbytes. Returns the median
    rate over reps passes, after one untimed pass."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    n = nbytes // 4 // n_threads * n_threads
    a = np.empty(n, np.float32)
    chunks = np.split(a, n_threads)
    one = np.float32(1.0)

    def touch(c):
        np.copyto(c, one)

    def scale(c):
        np.multiply(c, one, out=c)

    times = []
    with ThreadPoolExecutor(n_threads) as ex:
        list(ex.map(touch, chunks))
        for _ in range(reps + 1):
            t0 = time.perf_counter()
            list(ex.map(scale, chunks))
            times.append(time.perf_counter() - t0)
    assert a[0] == 1.0 and a[-1] == 1.0
    med = statistics.median(times[1:])
    return {"what": f"in-place fp32 scale of {n * 4} bytes on {n_threads} threads (each line "
                    f"read once and written once), median of {reps} passes",
            "bytes": n * 4, "ms": med * 1e3, "gbps": 2 * n * 4 / med / 1e9}


def host_info():
    """CPU model and core counts of the host the bench runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    quota = None
    try:  # cgroup v2 CPU quota: "max" or "<quota> <period>"
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    usable = affinity
    for cap in (quota, os.environ.get("OMP_NUM_THREADS")):
        if cap:
            usable = min(usable, int(cap))
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity,
            "cgroup_quota_cpus": quota, "usable_cpus": max(1, usable)}


def cpu_baseline_all_cores(w, plan_S, plan_begin, n_threads, target_s=8.0, window=1 << 22):
    """The same oracle calls on n_threads host threads at once, each on its own
    window of the shard (the step is elementwise, so the windows are
    independent; ctypes releases the GIL inside the oracle's C code).  Rate =
    elements processed by all threads / wall time of the concurrent run."""
    import threading

    import numpy as np

    import oracle
    import synth

    n_threads = max(1, min(n_threads, plan_S // window if plan_S >= window else 1))
    n = min(window, plan_S)
    op = oracle.plan([n], 1, 0, 1)
    hp = dict(lr=w.lr, b1=w.beta1, b2=w.beta2, eps=w.eps, wd=w.weight_decay, adamw=w.adamw)
    gkey = synth.key(w.seed, synth.STREAM_GRAD, 1)
    mkey = synth.key(w.seed, synth.STREAM_MASTER, 0)
    bufs = []
    for t in range(n_threads):
        i0 = plan_begin + t * n
        vals = synth.host_values(gkey, i0, n, w.grad_sigma, 1.0,
                                 synth.outlier_thresh(w.outlier_p), w.outlier_mult)
        bufs.append((synth.grad_bits(vals, w.grad_dtype),
                     synth.host_values(mkey, i0, n, w.master_sigma),
                     np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)))
    start = threading.Barrier(n_threads + 1)
    counts = [0] * n_threads
    stop_at = [0.0]

    def work(t):
        gbits, master, mm, vv, param = bufs[t]
        start.wait()
        while True:
            flat = oracle.flatten(op, [gbits])
            ovf = oracle.adam_step(counts[t] + 1, 1.0, flat, w.grad_dtype, master, mm, vv, **hp)
            if not ovf:
                oracle.write_param(master, n, 0, 0, param, w.param_dtype)
            counts[t] += 1
            if time.perf_counter() >= stop_at[0]:
                break

    threads = [threading.Thread(target=work, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    t0 = time.perf_counter()
    stop_at[0] = t0 + target_s
    start.wait()
    for th in threads:
        th.join()
    el = time.perf_counter() - t0
    rate = n * sum(counts) / el
    return {"value": rate, "unit": "params/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{n_threads} host threads at once, each running the oracle (scalar C) "
                      f"flatten + overflow test + AdamW + {w.param_dtype} cast on its own "
                      f"{n}-element window of the shard; {sum(counts)} window-steps in {el:.1f} s"}


def cpu_baseline(w, plan_S, plan_begin, target_s=12.0, window=1 << 24):
    """The oracle (single thread, as it stands) on a bounded window of the same
    shard: flatten + overflow test + AdamW + half cast, repeated until about
    target_s seconds of CPU work."""
    import numpy as np

    import oracle
    import synth

    n = min(window, plan_S)
    op = oracle.plan([n], 1, 0, 1)
    gkey = synth.key(w.seed, synth.STREAM_GRAD, 1)
    vals = synth.host_values(gkey, plan_begin, n, w.grad_sigma, 1.0,
                             synth.outlier_thresh(w.outlier_p), w.outlier_mult)
    gbits = synth.grad_bits(vals, w.grad_dtype)
    master = synth.host_values(synth.key(w.seed, synth.STREAM_MASTER, 0), plan_begin, n,
                               w.master_sigma)
    mm = np.zeros(n, np.float32)
    vv = np.zeros(n, np.float32)
    param = np.zeros(n, np.uint16)
    hp = dict(lr=w.lr, b1=w.beta1, b2=w.beta2, eps=w.eps, wd=w.weight_decay, adamw=w.adamw)
    steps = 0
    t0 = time.perf_counter()
    while True:
        flat = oracle.flatten(op, [gbits])
        ovf = oracle.adam_step(steps + 1, 1.0, flat, w.grad_dtype, master, mm, vv, **hp)
        if not ovf:
            oracle.write_param(master, n, 0, 0, param, w.param_dtype)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or steps >= 50:
            break
    rate = n * steps / el
    return {"value": rate, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle (scalar C, 1 thread) flatten + overflow test + AdamW + "
                      f"{w.param_dtype} cast over the shard's first {n} elements "
                      f"(flat [{plan_begin}, {plan_begin + n})), {steps} steps, {el:.1f} s",
            "gbps_equiv": rate * (adam_bytes(w.grad_dtype) + flatten_bytes(w.grad_dtype)) / 1e9}


PROFILES_DIR = os.path.join(ROOT, "profiles")
KERNELS_SRC = os.path.join(ROOT, "zero_partitioned_mixed_plan_amd", "csrc", "kernels.hip")
# Bytes per L2-to-memory request on MI355X, shown by a copy of known size
# (profiles/*_hbm_requests.md): a read that is not a 32-byte request moves a
# 128-byte line, a write request moves 64 bytes (or 32).
READ_LINE_BYTES = 128


def kernels_digest(path=KERNELS_SRC):
    """SHA-256 of the kernel source with // comments and blank lines removed,
    so that a comment edit does not count as a kernel change."""
    import hashlib
    import re
    lines = []
    for line in open(path).read().splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line.strip():
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def request_bytes(rdreq, rdreq_32b, wrreq, wrreq_64b):
    """HBM bytes of TCC/EA request counts: reads at 128 (32) bytes, writes at
    64 (32) bytes per request."""
    reads = READ_LINE_BYTES * (rdreq - rdreq_32b) + 32 * rdreq_32b
    writes = 64 * wrreq_64b + 32 * (wrreq - wrreq_64b)
    return reads + writes


def counted_traffic(workload_name, grad_dtype="bf16", kernel="adam"):
    """HBM bytes per launch of the update (kernel="adam") or per call of the
    flatten (kernel="flatten"), from the raw request counts in the committed
    rocprofv3 summary for this workload and gradient dtype; None when there is
    none, or the kernels have changed since it was taken."""
    import glob
    import re
    digest = kernels_digest()
    for path in sorted(glob.glob(os.path.join(PROFILES_DIR, "*_hbm_requests.md"))):
        vals = dict(re.findall(r"^(\w+) = (\S+)$", open(path).read(), flags=re.M))
        if (vals.get("workload") == workload_name and vals.get("grad_dtype") == grad_dtype
                and vals.get("kernels_sha256") == digest):
            return request_bytes(*(int(vals[f"{kernel}_{c}"])
                                   for c in ("rdreq", "rdreq_32b", "wrreq", "wrreq_64b")))
    return None


def copy_probe(nbytes, reps, device):
    """A plain device copy of known size (for scaling the HBM byte counters)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize(device)
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def placement_probe(S, ballasts_gb, device, reps=10):
    """The fused update on one S-element shard placed anew for every trial:
    before each trial a ballast allocation of the given size moves where the
    arrays land, and the arrays are either five allocations ("separate") or
    carved back to back from one ("one").  The caching allocator is emptied
    between trials, so even a repeated virtual address gets its physical
    pages afresh.  Prints one line per trial and a JSON summary."""
    import torch

    import zero_partitioned_mixed_plan_amd as z
    plan = z.zero_partition_plan([S], 1, 0, 64, 1 << 25)
    plan.set_timing(True)
    hp = z.AdamHParams()
    out = {}
    for gb in ballasts_gb:
        for layout in ("separate", "one"):
            ballast = (torch.empty(int(gb * 1e9), dtype=torch.uint8, device=device)
                       if gb > 0 else None)
            if layout == "separate":
                master, m, v = (torch.empty(S, device=device) for _ in range(3))
                g = torch.empty(S, dtype=torch.bfloat16, device=device)
                param = torch.empty(S, dtype=torch.bfloat16, device=device)
                buf = None
            else:
                buf = torch.empty(16 * S, dtype=torch.uint8, device=device)
                master, m, v = (buf[4 * S * i:4 * S * (i + 1)].view(torch.float32)
                                for i in range(3))
                g = buf[12 * S:14 * S].view(torch.bfloat16)
                param = buf[14 * S:16 * S].view(torch.bfloat16)
            g.normal_(0, 1e-3)
            master.normal_(0, 0.02)
            m.zero_()
            v.zero_()
            t = []
            for i in range(reps + 2):
                assert z.zero_adam_step(plan, hp, 1, 1.0, g, master, m, v, param, 0) == 0
                if i >= 2:
                    t.append(plan.kernel_ms(2))
            med = statistics.median(t)
            out.setdefault(layout, []).append(med)
            print(f"[placement] ballast {gb:g} GB, {layout}: update {med:.3f} ms "
                  f"(min {min(t):.3f}, max {max(t):.3f}) = {28 * S / med / 8e9 * 100:.2f}% of "
                  f"8 TB/s; master at {master.data_ptr():#x}", flush=True)
            del master, m, v, g, param, buf, ballast
            torch.cuda.empty_cache()
    summary = {k: {"min_ms": min(v), "max_ms": max(v), "median_ms": statistics.median(v),
                   "spread_pct": (max(v) / min(v) - 1) * 100} for k, v in out.items()}
    print(json.dumps({"placement_probe_elems": S, "ballasts_gb": ballasts_gb,
                      "reps": reps, "layouts": summary}), flush=True)
    plan.close()


def main(argv=None):
    try:
        return _main(argv)
    finally:
        # plans and pipelines are released here, while the HIP runtime and
        # any profiler attached to it are fully alive, not by destructors
        # during interpreter shutdown
        z = sys.modules.get("zero_partitioned_mixed_plan_amd")
        if z is not None:
            z.release_all()


def _main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama2_70b")
    ap.add_argument("--grad-dtype", choices=["f16", "bf16", "f32"], default=None,
                    help="override the workload's gradient dtype (f32: gradients kept in fp32, "
                         "30 B/element in the update)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--step-log", default=None,
                    help="write one JSON line per timed step (t, overflow, scale, kernel times "
                         "and rates) to this file")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay measurement of the same step")
    ap.add_argument("--mode", choices=["device", "offload"], default="device",
                    help="device: the whole step on the GPU (default); offload: ZeRO-Offload "
                         "(host-resident state, host update, one-step delayed update)")
    ap.add_argument("--host-threads", type=int, default=None,
                    help="threads of the offload host update (default: every usable CPU; "
                         "the pipeline's caller thread mostly waits)")
    ap.add_argument("--forward-ms", type=float, default=0.0,
                    help="offload mode: run about this many ms of bf16 products on the GPU "
                         "before each step, a stand-in for the forward and backward passes "
                         "that the one-step delayed update overlaps")
    ap.add_argument("--timeline", default=None, metavar="FILE",
                    help="offload mode: record the pipeline's timeline of the timed steps "
                         "(every piece's copies and host update), summarise it in the JSON "
                         "line and write the intervals to FILE")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="run only a plain copy of this many bytes (counter calibration)")
    ap.add_argument("--placement-probe", default=None, metavar="GB,GB,...",
                    help="run only the update on the workload's shard size, placed anew "
                         "after ballast allocations of these sizes (GB)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: it runs one rank's real-sized shard on a "
              "single MI355X; --gpus must be 1", file=sys.stderr)
        return 2
    _ensure_built()
    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(args.copy_probe, 5, device)
        return 0

    import dataclasses

    from synth.workloads import get
    w = get(args.workload)
    if args.grad_dtype:
        w = dataclasses.replace(w, grad_dtype=args.grad_dtype)
    if args.placement_probe:
        import zero_partitioned_mixed_plan_amd as z
        wplan = z.zero_partition_plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
        S = wplan.S
        wplan.close()
        placement_probe(S, [float(x) for x in args.placement_probe.split(",")], device)
        return 0
    if args.mode == "offload":
        threads = args.host_threads or host_info()["usable_cpus"]
        plan, res = run_offload(w, args.steps, args.warmup, device, threads, args.forward_ms,
                                args.timeline)
        print(json.dumps({
            "metric": METRIC, "value": res["lag1"]["value"], "unit": "params/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["lag1"]["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": w.description, "mode": "offload (ZeRO-Offload, host update, "
                       "one-step delayed parameter update)", "shard_elems": plan.S,
                       "real_elems": plan.real},
            "offload": res}), flush=True)
        return 0
    step_log = open(args.step_log, "w") if args.step_log else None
    plan, wall, times, state, bufs = run_gpu(w, args.steps, args.warmup, device, step_log)
    if step_log is not None:
        step_log.close()
    write_ms, scan_ms = time_standalone_kernels(bufs)
    n_buckets, bflat_ms = time_bucketed_flatten(bufs)
    graph_wall, devsc_ms = (None, None) if args.no_graph else run_graph(bufs, args.steps,
                                                                        args.warmup, device)
    S, real, begin = plan.S, plan.real, plan.begin
    ms_per_step = wall * 1000.0 / args.steps
    if not times["adam"]:
        raise SystemExit("every timed step was skipped (overflow): no update time to report")
    adam_ms = sum(times["adam"]) / len(times["adam"])
    flat_ms = sum(times["flatten"]) / len(times["flatten"])
    ab, fb = adam_bytes(w.grad_dtype), flatten_bytes(w.grad_dtype)
    adam_gbs = ab * S / (adam_ms * 1e-3) / 1e9
    flat_gbs = fb * S / (flat_ms * 1e-3) / 1e9
    step_gbs = (ab + fb) * S / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": real / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.description, "shard_elems": S, "real_elems": real,
                   "shard_begin": begin, "world_size": w.world_size, "rank": w.rank,
                   "grad_dtype": w.grad_dtype, "param_dtype": w.param_dtype,
                   "segments": plan.n_segments, "flatten": "all buckets, one call"},
        "hbm_gbps_step": step_gbs,
        "pct_peak_step": 100.0 * step_gbs / HBM_PEAK_GBS,
        "kernels": {
            "adam_fused": {"avg_ms": adam_ms, "median_ms": statistics.median(times["adam"]),
                           "min_ms": min(times["adam"]),
                           "bytes_per_elem": ab, "gbps": adam_gbs,
                           "params_per_s": S / (adam_ms * 1e-3)},
            "flatten": {"avg_ms": flat_ms, "median_ms": statistics.median(times["flatten"]),
                        "min_ms": min(times["flatten"]),
                        "bytes_per_elem": fb, "gbps": flat_gbs,
                        "traffic": counted_traffic(w.name, w.grad_dtype, "flatten")},
            "flatten_by_bucket": {"calls": n_buckets, "ms": bflat_ms, "bytes_per_elem": fb,
                                  "gbps": fb * S / (bflat_ms * 1e-3) / 1e9,
                                  "what": "one zero_flatten_grads call per bucket of the shard, "
                                          "timed as a whole"},
            "write_param": {"ms": write_ms, "bytes_per_elem": 6,
                            "gbps": 6 * real / (write_ms * 1e-3) / 1e9},
            "scan": {"ms": scan_ms, "bytes_per_elem": GRAD_BYTES[w.grad_dtype],
                     "gbps": GRAD_BYTES[w.grad_dtype] * S / (scan_ms * 1e-3) / 1e9},
        },
        "skipped_steps": state["skipped"],   # over warm-up and timed steps; kernel times
                                             # above are over the applied timed steps
        "graph_replay": None if graph_wall is None else {
            "ms_per_step": graph_wall * 1000.0 / args.steps,
            "value": real / (graph_wall / args.steps),
            "adam_device_scalars_ms": devsc_ms,
            "what": "flatten + zero_adam_step_async (device-resident t and loss scale) captured "
                    "once into a HIP graph, replayed per step; no host round trip"},
        "roofline": {"bound": "hbm", "achieved": adam_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": adam_gbs / HBM_PEAK_GBS,
                     "traffic": counted_traffic(w.name, w.grad_dtype)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cb = cpu_baseline(w, S, begin, target_s=args.cpu_seconds)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        host = host_info()
        out["cpu_baseline"]["host"] = host
        log(f"[bench] timing the oracle on {host['usable_cpus']} host threads")
        out["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(
            w, S, begin, host["usable_cpus"], target_s=max(2.0, args.cpu_seconds * 2 / 3))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
