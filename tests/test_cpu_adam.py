"""ZeRO-Offload's host-side update (zero_cpu_adam_step) against the oracle,
on the CPU: every instruction-set path (forced with ZERO_CPU_ISA), several
thread counts, fp16, bf16 and fp32 gradients, Adam-L2 and AdamW, padding, skipped steps and
a sweep of fp32 patterns through the parameter cast.  Bar: bit-identical
master / moments / parameters (the same arithmetic as the device update)."""
import os

import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_plan_amd as z

ISAS = ["avx512", "avx2", "scalar"]


@pytest.fixture(params=ISAS)
def isa(request, monkeypatch):
    monkeypatch.setenv("ZERO_CPU_ISA", request.param)
    if request.param != "scalar" and z.zero_cpu_isa() != request.param:
        pytest.skip(f"this host has no {request.param}")
    assert z.zero_cpu_isa() == request.param
    return request.param


def _grads(rng, n, dt, scale, sigma=1e-2):
    vals = (rng.normal(0, sigma, n) * scale).astype(np.float32)
    if dt == "f32":
        return vals
    if dt == "f16":
        return vals.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("gdt,pdt,adamw", [("f16", "f16", True), ("bf16", "bf16", True),
                                           ("bf16", "f16", False), ("f16", "bf16", False),
                                           ("f32", "bf16", True), ("f32", "f16", False)])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_host_update_equals_oracle(isa, gdt, pdt, adamw, threads):
    numels = [1000, 37, 5, 2049, 1]          # P = 3092; R = 3, A = 8 -> S = 1032, padding on rank 2
    rng = np.random.default_rng(7)
    for r in range(3):
        plan = z.zero_partition_plan(numels, 3, r, 8)
        S, real, begin = plan.S, plan.real, plan.begin
        master = np.zeros(S, np.float32)
        master[:real] = rng.normal(0, 0.02, real).astype(np.float32)
        om, omo, ov = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
        gm, gmo, gv = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
        P = sum(numels)
        oparam = np.full(P, 0xABCD, np.uint16)
        gparam = oparam.copy()
        hp = z.AdamHParams(weight_decay=0.05, adamw=adamw)
        scale = 1024.0 if gdt == "f16" else 1.0
        for t in range(1, 5):
            flat = np.zeros(S, np.float32 if gdt == "f32" else np.uint16)
            flat[:real] = _grads(rng, real, gdt, scale)
            o = oracle.adam_step(t, scale, flat, gdt, om, omo, ov, lr=hp.lr, b1=hp.beta1,
                                 b2=hp.beta2, eps=hp.eps, wd=hp.weight_decay, adamw=adamw)
            oracle.write_param(om, real, begin, 0, oparam, pdt)
            g = z.zero_cpu_adam_step(plan, hp, t, scale, flat, gm, gmo, gv, gparam, 0,
                                     grad_dtype=gdt, param_dtype=pdt, n_threads=threads)
            assert g == o == 0
            for a, b in ((gm, om), (gmo, omo), (gv, ov)):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (isa, r, t)
            assert np.array_equal(gparam, oparam), (isa, r, t)


def test_overflow_skips_and_leaves_state_untouched(isa):
    plan = z.zero_partition_plan([5000], 1, 0, 1)
    rng = np.random.default_rng(1)
    for bad in (0x7C00, 0xFC00, 0x7E00, 0x7C01):
        for pos in (0, 17, 4095, 4999):
            flat = _grads(rng, 5000, "f16", 1.0)
            flat[pos] = bad
            m0 = rng.normal(0, 0.02, 5000).astype(np.float32)
            master, mo, v = m0.copy(), np.ones(5000, np.float32), np.ones(5000, np.float32)
            param = np.zeros(5000, np.uint16)
            assert z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, mo, v, param,
                                        grad_dtype="f16", param_dtype="f16") == 1
            assert np.array_equal(master, m0) and np.all(mo == 1) and np.all(v == 1)
            assert not param.any()
    # a known flag overrides the test; the largest finite value does not trip
    flat = np.full(5000, 0x7BFF, np.uint16)
    master = np.zeros(5000, np.float32)
    z1, z2 = np.zeros(5000, np.float32), np.zeros(5000, np.float32)
    assert z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, z1, z2,
                                grad_dtype="f16", overflow=1) == 1
    assert z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, z1, z2,
                                grad_dtype="f16") == 0


def test_f32_overflow_skips_and_leaves_state_untouched(isa):
    n = 5001                                  # a masked / scalar tail on every path
    plan = z.zero_partition_plan([n], 1, 0, 1)
    rng = np.random.default_rng(2)
    for bad in (0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001):
        for pos in (0, 17, 4095, 4999, 5000):
            flat = _grads(rng, n, "f32", 1.0).view(np.uint32).copy()
            flat[pos] = bad
            m0 = rng.normal(0, 0.02, n).astype(np.float32)
            master, mo, v = m0.copy(), np.ones(n, np.float32), np.ones(n, np.float32)
            param = np.zeros(n, np.uint16)
            assert z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, flat.view(np.float32),
                                        master, mo, v, param, grad_dtype="f32",
                                        param_dtype="bf16", n_threads=3) == 1, (bad, pos)
            assert np.array_equal(master, m0) and np.all(mo == 1) and np.all(v == 1)
            assert not param.any()
    flat = np.full(n, 0x7F7FFFFF, np.uint32).view(np.float32)   # largest finite: no skip
    z0 = [np.zeros(n, np.float32) for _ in range(3)]
    assert z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, *z0) == 0


def test_fp32_subnormals_are_kept(isa):
    """g*g and the variance in the fp32 subnormal range, a master of subnormals:
    no flush to zero on any path, bit for bit with the oracle."""
    n = 4099
    plan = z.zero_partition_plan([n], 1, 0, 1)
    rng = np.random.default_rng(9)
    g = (rng.normal(0, 1e-20, n)).astype(np.float32)
    m0 = (rng.normal(0, 1e-39, n)).astype(np.float32)
    tiny = np.finfo(np.float32).tiny
    assert np.any((np.abs(m0) > 0) & (np.abs(m0) < tiny))
    gm, gmo, gv = m0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    om, omo, ov = m0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 4):
        # lr 1e-25: the master moves by subnormal amounts and stays subnormal
        assert z.zero_cpu_adam_step(plan, z.AdamHParams(lr=1e-25, weight_decay=0.1), t, 1.0, g,
                                    gm, gmo, gv, grad_dtype="f32", n_threads=3) == 0
        assert oracle.adam_step(t, 1.0, g, "f32", om, omo, ov, lr=1e-25, wd=0.1) == 0
    for x in (ov, om):
        assert np.any((np.abs(x) > 0) & (np.abs(x) < tiny)), "no fp32 subnormals reached"
    for a, b in ((gm, om), (gmo, omo), (gv, ov)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("pdt", ["f16", "bf16"])
def test_parameter_cast_sweep(isa, pdt):
    """lr = 0 and zero gradients leave the master unchanged, so the written
    parameters are the cast of the master: every fp32 exponent, both
    parities of the last kept bit, ties and their neighbours."""
    lows = []
    for b in range(8):
        for lo in (0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0ABC, 0x1555):
            lows.append((b << 13) | lo)
    lows = np.array(sorted(set(lows)), dtype=np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    x = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    n = x.size
    plan = z.zero_partition_plan([n], 1, 0, 1)
    master = x.copy()
    param = np.zeros(n, np.uint16)
    flat = np.zeros(n, np.uint16)
    hp = z.AdamHParams(lr=0.0, weight_decay=0.0)
    assert z.zero_cpu_adam_step(plan, hp, 1, 1.0, flat, master, np.zeros(n, np.float32),
                                np.zeros(n, np.float32), param, grad_dtype="bf16",
                                param_dtype=pdt, overflow=0, n_threads=4) == 0
    nan = np.isnan(x)
    assert np.array_equal(master[~nan].view(np.uint32), x[~nan].view(np.uint32))
    exp = oracle.float_to_half(x, pdt)
    assert np.array_equal(param[~nan], exp[~nan])
    emask, frac = (0x7C00, 0x03FF) if pdt == "f16" else (0x7F80, 0x007F)
    assert np.all((param[nan] & emask) == emask) and np.all((param[nan] & frac) != 0)


def test_argument_errors():
    plan = z.zero_partition_plan([100], 1, 0, 1)
    f = np.zeros(100, np.float32)
    g = np.zeros(100, np.uint16)
    with pytest.raises(z.ZeroError):
        z.zero_cpu_adam_step(plan, z.AdamHParams(), 0, 1.0, g, f, f.copy(), f.copy(),
                             grad_dtype="bf16")
    with pytest.raises(z.ZeroError):
        z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, g, f, f.copy(), f.copy(),
                             grad_dtype="bf16", overflow=2)
    with pytest.raises(z.ZeroError):
        z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, g, f, f.copy(), f.copy(),
                             np.zeros(10, np.uint16), grad_dtype="bf16", param_dtype="bf16")
    with pytest.raises(ValueError):
        z.zero_cpu_adam_step(plan, z.AdamHParams(), 1, 1.0, g[:10], f, f.copy(), f.copy(),
                             grad_dtype="bf16")


@pytest.mark.skipif(os.environ.get("ZERO_EXHAUSTIVE") != "1",
                    reason="about 4 minutes on 8 cores; set ZERO_EXHAUSTIVE=1 to run")
@pytest.mark.parametrize("pdt", ["f16", "bf16"])
def test_parameter_cast_all_2_32_patterns(pdt, monkeypatch):
    """The host update's half cast on every instruction-set path over all 2^32
    fp32 patterns (lr = 0 and zero gradients leave the master as it is, so the
    parameters are its cast), against the oracle computed once per chunk on
    all cores: every non-NaN input bit for bit, NaN to a NaN.  Opt-in: the
    4.2M-pattern sweep above covers every sign / exponent / high-fraction
    pattern with the tie and neighbour low bits of both formats by default."""
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 26
    workers = max(1, min(16, os.cpu_count() or 1))
    sub = chunk // workers
    plan = z.zero_partition_plan([chunk], 1, 0, 1)
    hp = z.AdamHParams(lr=0.0, weight_decay=0.0)
    flat = np.zeros(chunk, np.uint16)
    mo = np.zeros(chunk, np.float32)
    va = np.zeros(chunk, np.float32)
    param = np.empty(chunk, np.uint16)
    emask, frac = (0x7C00, 0x03FF) if pdt == "f16" else (0x7F80, 0x007F)
    isas = [i for i in ISAS if i == "scalar" or _has_isa(i, monkeypatch)]
    with ThreadPoolExecutor(workers) as ex:
        for c in range((1 << 32) // chunk):
            u = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint32)
            x = u.view(np.float32)
            exp = np.concatenate(list(ex.map(
                lambda i: oracle.float_to_half(x[i * sub:(i + 1) * sub], pdt), range(workers))))
            nan = np.isnan(x)
            for isa in isas:
                monkeypatch.setenv("ZERO_CPU_ISA", isa)
                master = x.copy()
                assert z.zero_cpu_adam_step(plan, hp, 1, 1.0, flat, master, mo, va, param,
                                            grad_dtype="bf16", param_dtype=pdt, overflow=0,
                                            n_threads=workers) == 0
                bad = np.flatnonzero((param != exp) & ~nan)
                assert bad.size == 0, (isa, pdt, [hex(int(u[i])) for i in bad[:4]])
                pn = param[nan]
                assert np.all((pn & emask) == emask) and np.all((pn & frac) != 0), (isa, c)


def _has_isa(isa, monkeypatch):
    monkeypatch.setenv("ZERO_CPU_ISA", isa)
    ok = z.zero_cpu_isa() == isa
    monkeypatch.delenv("ZERO_CPU_ISA")
    return ok



def _forked_host_step(conn, flats):
    """Runs in a child made by fork(): repeat the parent's host steps and
    send back the resulting state."""
    try:
        conn.send(_pool_steps(flats))
    finally:
        conn.close()


def _pool_steps(flats):
    plan = z.zero_partition_plan([flats[0].size], 1, 0, 1)
    master = np.random.default_rng(5).normal(0, 0.02, plan.S).astype(np.float32)
    mo, v = np.zeros_like(master), np.zeros_like(master)
    param = np.zeros(plan.S, np.uint16)
    for t, (flat, threads) in enumerate(zip(flats, (4, 4, 2)), 1):
        assert z.zero_cpu_adam_step(plan, z.AdamHParams(), t, 1.0, flat, master, mo, v, param,
                                    grad_dtype="bf16", param_dtype="bf16",
                                    n_threads=threads) == 0
    return master.view(np.uint32), mo.view(np.uint32), v.view(np.uint32), param


def test_host_step_in_a_forked_child():
    # The library keeps a pool of host threads between calls.  A child made
    # by fork() inherits that pool without its threads: it must build its
    # own (not wait on threads that are not there) and compute the same.
    # The child makes no torch call (torch's own threads do not survive a
    # fork either); the gradients are drawn here.
    import multiprocessing as mp
    rng = np.random.default_rng(6)
    flats = [_grads(rng, 70001, "bf16", 1.0) for _ in range(3)]
    want = _pool_steps(flats)     # the parent now holds a 2-thread pool
    ctx = mp.get_context("fork")
    parent, child = ctx.Pipe(duplex=False)
    proc = ctx.Process(target=_forked_host_step, args=(child, flats))
    proc.start()
    child.close()
    try:
        assert parent.poll(60), "host step in the forked child did not finish"
        got = parent.recv()
    finally:
        proc.join(10)
        if proc.is_alive():
            proc.kill()
            proc.join()
    assert proc.exitcode == 0
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


_NO_THREADS_CHILD = r"""
import json, mmap, re, resource, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import zero_partitioned_mixed_plan_amd as z

n = 70001
plan = z.zero_partition_plan([n], 1, 0, 64)
S = plan.S
rng = np.random.default_rng(5)
g = (rng.normal(0, 1e-2, S).astype(np.float32)).astype(np.float16).view(np.uint16)
m0 = rng.normal(0, 0.02, S).astype(np.float32)
hp = z.AdamHParams(weight_decay=0.05, adamw=True)
bufs = {}
for name, threads in (("want", 1), ("got", 16)):
    bufs[name] = [m0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32),
                  np.zeros(S, np.uint16)]
rc1 = z.zero_cpu_adam_step(plan, hp, 1, 1.0, g, *bufs["want"], 0, grad_dtype="f16",
                           param_dtype="bf16", overflow=0, n_threads=1)
# leave less address space than 16 thread stacks need
vm = int(re.search(r"VmSize:\s+(\d+) kB", open("/proc/self/status").read()).group(1)) << 10
soft, hard = resource.getrlimit(resource.RLIMIT_AS)
resource.setrlimit(resource.RLIMIT_AS, (vm + (40 << 20), hard))
try:
    mmap.mmap(-1, 16 * resource.getrlimit(resource.RLIMIT_STACK)[0])
    bites = False
except OSError:
    bites = True
rc16 = z.zero_cpu_adam_step(plan, hp, 1, 1.0, g, *bufs["got"], 0, grad_dtype="f16",
                            param_dtype="bf16", overflow=-1, n_threads=16)
resource.setrlimit(resource.RLIMIT_AS, (soft, hard))
same = all(np.array_equal(a, b) for a, b in zip(bufs["want"], bufs["got"]))
print(json.dumps({"rc1": rc1, "rc16": rc16, "bites": bites, "same": same}))
"""


def test_host_step_when_threads_cannot_be_started():
    # Thread creation can fail (here: too little address space left for
    # the threads' stacks).  The call must neither abort the process nor
    # fail: the calling thread takes the ranges that got no thread, and the
    # result is the one-thread result.
    import json
    import resource
    import subprocess
    import sys
    if resource.getrlimit(resource.RLIMIT_STACK)[0] in (resource.RLIM_INFINITY, 0):
        pytest.skip("thread stacks are not sized by RLIMIT_STACK here")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, ZERO_CPU_ISA="scalar")
    r = subprocess.run([sys.executable, "-c", _NO_THREADS_CHILD, root], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["bites"], "the address-space limit left room for 16 thread stacks"
    assert d == {"rc1": 0, "rc16": 0, "bites": True, "same": True}
