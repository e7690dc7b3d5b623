"""The overflow gate's rules on the GPU, through the C ABI.

* A step trusts the fused test of the flattens that covered its buffer: a
  value written into that buffer afterwards is not tested again (the
  documented rule), and is consumed as a gradient -- unless the caller
  declares the write with zero_flatten_invalidate, which makes the step scan.
* A flatten into another buffer starts the flag over, so a step on the
  second buffer does not inherit what was found in the first.
* A scan decides a step whose buffer was not (fully) flattened, and it tests
  the real elements only: nonfinite padding does not skip the step.
* The offloaded step gates like the device step: an unflattened buffer with
  an inf is scanned and the step skipped; a buffer flattened in another
  dtype than the pipeline's is refused.
* The asynchronous step forms its fp32 scalars on the device with the
  device's pow and sqrt; they equal the host's bit for bit for t = 1..10^6.

Every applied step is compared with the oracle bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_plan_amd as z
from harness import to_device_grad, torch_dtype
from zero_partitioned_mixed_plan_amd import _abi

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
INF = {"f16": 0x7C00, "bf16": 0x7F80, "f32": 0x7F800000}
NUMELS = [3000, 1, 7, 100003, 65, 2048, 511, 30000, 13, 4099]


def _bits(t):
    import torch
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _grads(dt, seed, numels=NUMELS):
    from synth import grad_bits
    rng = np.random.default_rng(seed)
    return [grad_bits(rng.normal(0, 1e-2, n).astype(np.float32), dt) for n in numels]


def _state(S, seed):
    import torch
    m0 = np.random.default_rng(seed).normal(0, 0.02, S).astype(np.float32)
    return (m0, torch.from_numpy(m0.copy()).to(DEV), torch.zeros(S, device=DEV),
            torch.zeros(S, device=DEV))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_write_after_covering_flatten_is_not_retested(dt):
    """flatten (all buckets) -> write +inf into the flat buffer -> step: the
    gate uses the flatten's clean result, so the step is applied and the inf
    enters the update at that element (NaN master there, as in the oracle's
    ungated update); every other element equals the oracle's."""
    import torch
    plan = z.zero_partition_plan(NUMELS, 2, 1, 8, 20000)
    op = oracle.plan(NUMELS, 2, 1, 8, 20000)
    host = _grads(dt, 1)
    flat = torch.empty(op.S, dtype=torch_dtype(dt), device=DEV)
    z.zero_flatten_grads(plan, -1, [to_device_grad(h, dt, DEV) for h in host], flat)
    pos = op.real // 3
    bits = oracle.flatten(op, host)
    bits[pos] = INF[dt]
    flat[pos:pos + 1].copy_(to_device_grad(bits[pos:pos + 1].copy(), dt, DEV))
    m0, master, mo, va = _state(op.S, 2)
    assert z.zero_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, mo, va) == 0
    om, omo, ov = m0.copy(), np.zeros(op.S, np.float32), np.zeros(op.S, np.float32)
    oracle.adam_update(1, 1.0, bits, dt, om, omo, ov)
    got = master.cpu().numpy()
    assert np.isnan(got[pos]) and np.isnan(om[pos])
    keep = np.arange(op.S) != pos
    assert np.array_equal(got.view(np.uint32)[keep], om.view(np.uint32)[keep])
    assert np.array_equal(_bits(va)[keep], ov.view(np.uint32)[keep])


@pytest.mark.parametrize("mode", ["sync", "async"])
def test_invalidate_makes_the_step_scan(mode):
    """The same write after a covering flatten, declared with
    zero_flatten_invalidate: the step scans the buffer, finds the inf and is
    skipped, leaving the state unchanged."""
    import torch
    plan = z.zero_partition_plan(NUMELS, 2, 1, 8, 20000)
    op = oracle.plan(NUMELS, 2, 1, 8, 20000)
    host = _grads("bf16", 7)
    flat = torch.empty(op.S, dtype=torch.bfloat16, device=DEV)
    z.zero_flatten_grads(plan, -1, [to_device_grad(h, "bf16", DEV) for h in host], flat)
    pos = op.real // 5
    flat[pos] = float("inf")
    z.zero_flatten_invalidate(plan)
    m0, master, mo, va = _state(op.S, 8)
    if mode == "sync":
        assert z.zero_adam_step(plan, z.AdamHParams(), 1, 1.0, flat, master, mo, va) == 1
    else:
        z.zero_state_upload(plan, 0, z.LossScaler(1.0, dynamic=False))
        z.zero_adam_step_async(plan, z.AdamHParams(), flat, master, mo, va)
        assert z.zero_state_download(plan).last_flag == 1
    assert np.array_equal(_bits(master), m0.view(np.uint32))
    assert not _bits(va).any()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_flatten_into_another_buffer_starts_the_flag_over(dt):
    """Gradients with an inf flattened into buffer A, then clean gradients
    into buffer B, then a step on B: applied, and equal to the oracle's;
    then the same with the inf in B's gradients: skipped."""
    import torch
    plan = z.zero_partition_plan(NUMELS, 2, 0, 8, 20000)
    op = oracle.plan(NUMELS, 2, 0, 8, 20000)
    clean = _grads(dt, 3)
    dirty = [h.copy() for h in clean]
    t0 = int(op.seg_tensor[0])
    dirty[t0][int(op.seg_tensor_off[0])] = INF[dt]
    dev = {k: [to_device_grad(h, dt, DEV) for h in v] for k, v in (("clean", clean),
                                                                   ("dirty", dirty))}
    hp = z.AdamHParams()
    for first, second, want in (("dirty", "clean", 0), ("clean", "dirty", 1)):
        a = torch.empty(op.S, dtype=torch_dtype(dt), device=DEV)
        b = torch.empty(op.S, dtype=torch_dtype(dt), device=DEV)
        z.zero_flatten_grads(plan, -1, dev[first], a)
        z.zero_flatten_grads(plan, -1, dev[second], b)
        m0, master, mo, va = _state(op.S, 4)
        assert z.zero_adam_step(plan, hp, 1, 1.0, b, master, mo, va) == want, (first, second)
        om, omo, ov = m0.copy(), np.zeros(op.S, np.float32), np.zeros(op.S, np.float32)
        src = clean if second == "clean" else dirty
        assert oracle.adam_step(1, 1.0, oracle.flatten(op, src), dt, om, omo, ov) == want
        assert np.array_equal(_bits(master), om.view(np.uint32))
        assert np.array_equal(_bits(va), ov.view(np.uint32))


@pytest.mark.parametrize("mode", ["sync", "async", "cpu"])
def test_scan_tests_the_real_elements_only(mode):
    """A flat buffer filled directly (no flatten), with +inf and NaN in the
    padding [real, S): the step is applied, and the real elements equal the
    oracle's step on the same gradients with a zero padding."""
    import torch
    numels = [1000, 37, 5]                     # P = 1042, R = 4, A = 64: S = 320
    plan = z.zero_partition_plan(numels, 4, 3, 64)
    op = oracle.plan(numels, 4, 3, 64)
    S, real = op.S, op.real
    assert 0 < real < S
    rng = np.random.default_rng(6)
    from synth import grad_bits
    bits = grad_bits(rng.normal(0, 1e-2, S).astype(np.float32), "bf16")
    bits[real:] = 0
    dirty = bits.copy()
    dirty[real] = INF["bf16"]
    dirty[S - 1] = 0x7FC1
    m0 = rng.normal(0, 0.02, S).astype(np.float32)
    hp = z.AdamHParams()
    om, omo, ov = m0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    assert oracle.adam_step(1, 1.0, bits, "bf16", om, omo, ov) == 0
    if mode == "cpu":
        master, mo, va = m0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
        flag = z.zero_cpu_adam_step(plan, hp, 1, 1.0, dirty, master, mo, va,
                                    grad_dtype="bf16", n_threads=2)
        got_m, got_v = master, va
    else:
        flat = to_device_grad(dirty, "bf16", DEV)
        _, master, mo, va = _state(S, 0)
        master.copy_(torch.from_numpy(m0))
        if mode == "sync":
            flag = z.zero_adam_step(plan, hp, 1, 1.0, flat, master, mo, va)
        else:
            z.zero_state_upload(plan, 0, z.LossScaler(1.0, dynamic=False))
            z.zero_adam_step_async(plan, hp, flat, master, mo, va)
            flag = z.zero_state_download(plan).last_flag
        got_m, got_v = master.cpu().numpy(), va.cpu().numpy()
    assert flag == 0
    assert np.array_equal(got_m[:real].view(np.uint32), om[:real].view(np.uint32))
    assert np.array_equal(got_v[:real].view(np.uint32), ov[:real].view(np.uint32))


def test_offload_scans_an_unflattened_buffer():
    """zero_offload_submit on a buffer written directly: an inf among the real
    gradients skips the step (host state unchanged, scale halved); a clean
    buffer is applied exactly as the oracle applies it."""
    numels = [5000, 300, 17]
    plan = z.zero_partition_plan(numels, 2, 1, 64)
    op = oracle.plan(numels, 2, 1, 64)
    S, real = op.S, op.real
    from synth import grad_bits
    rng = np.random.default_rng(8)
    bits = grad_bits(rng.normal(0, 1e-2, S).astype(np.float32) * 1024, "f16")
    bits[real:] = 0
    dirty = bits.copy()
    dirty[real // 2] = INF["f16"]
    m0 = rng.normal(0, 0.02, S).astype(np.float32)
    master, mo, va = m0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    hp = z.AdamHParams()
    z.zero_state_upload(plan, 0, z.LossScaler(1024.0, dynamic=True))
    off = z.Offload(plan, hp, "f16", None, master, mo, va, n_threads=2)
    off.submit(to_device_grad(dirty, "f16", DEV))
    off.drain()
    st = off.stats()
    assert (st["applied"], st["skipped"]) == (0, 1)
    assert np.array_equal(master.view(np.uint32), m0.view(np.uint32))
    assert z.zero_state_download(plan).scale == 512.0
    off.submit(to_device_grad(bits, "f16", DEV))
    off.drain()
    assert off.stats()["applied"] == 1
    om, omo, ov = m0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    assert oracle.adam_step(1, 512.0, bits, "f16", om, omo, ov) == 0
    assert np.array_equal(master.view(np.uint32), om.view(np.uint32))
    assert np.array_equal(va.view(np.uint32), ov.view(np.uint32))
    off.close()


def test_offload_refuses_a_buffer_flattened_in_another_dtype():
    import torch
    numels = [5000, 300, 17]
    plan = z.zero_partition_plan(numels, 2, 1, 64)
    S = plan.S
    master, mo, va = (np.zeros(S, np.float32) for _ in range(3))
    z.zero_state_upload(plan, 0, z.LossScaler(1.0, dynamic=False))
    off = z.Offload(plan, z.AdamHParams(), "bf16", None, master, mo, va, n_threads=2)
    flat32 = torch.zeros(S, dtype=torch.float32, device=DEV)
    grads = [torch.zeros(n, dtype=torch.float32, device=DEV) for n in numels]
    z.zero_flatten_grads(plan, -1, grads, flat32)
    with pytest.raises(TypeError):
        off.submit(flat32)                       # the binding checks the dtype
    rc = _abi.lib.zero_offload_submit(off._h, flat32.data_ptr(), None, 0, 0,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == _abi.ZERO_EINVAL and "dtype" in z.zero_last_error()
    rc = _abi.lib.zero_offload_submit(off._h, flat32.data_ptr() + 4, None, 0, 0,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == _abi.ZERO_EALIGN
    off.drain()
    assert off.stats()["submitted"] == 0
    off.close()


@pytest.mark.parametrize("hp,scale", [
    (z.AdamHParams(), 1.0),
    (z.AdamHParams(lr=3e-4, beta1=0.95, beta2=0.98, eps=1e-6, weight_decay=0.1), 65536.0),
    (z.AdamHParams(lr=1.0, beta1=0.5, beta2=0.9999, eps=1e-12, weight_decay=0.0,
                   adamw=False), 3.0),
    (z.AdamHParams(lr=7e-5, beta1=0.0, beta2=0.999999, weight_decay=1e-4), 2.0 ** -20),
])
def test_device_scalars_equal_the_host_scalars(hp, scale):
    """t = 1 .. 10^6: every fp32 scalar the asynchronous step forms on the
    device equals, bit for bit, the one the synchronous step forms on the
    host -- and the host's equal a float64 evaluation of their definitions
    rounded once (Python's math library), sampled every 997th step."""
    import torch
    n = 1_000_000
    out = torch.empty(10 * n, dtype=torch.float32, device=DEV)
    z.zero_adam_scalars(hp, 1, n, scale, out=out)
    torch.cuda.synchronize()
    dev = out.cpu().numpy().reshape(n, 10)
    host = z.zero_adam_scalars(hp, 1, n, scale)
    diff = np.nonzero((dev.view(np.uint32) != host.view(np.uint32)).any(axis=1))[0]
    assert diff.size == 0, f"device and host scalars differ at t = {(diff[:8] + 1).tolist()}"
    for t in range(1, n + 1, 997):
        want = np.array([1.0 / scale, hp.beta1, 1.0 - hp.beta1, hp.beta2, 1.0 - hp.beta2,
                         hp.lr / (1.0 - math.pow(hp.beta1, t)),
                         1.0 / math.sqrt(1.0 - math.pow(hp.beta2, t)), hp.eps,
                         1.0 - hp.lr * hp.weight_decay if hp.adamw else 1.0,
                         hp.weight_decay], np.float64).astype(np.float32)
        assert np.array_equal(host[t - 1].view(np.uint32), want.view(np.uint32)), t
