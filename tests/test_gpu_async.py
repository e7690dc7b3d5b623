"""GPU parity of the step without host round trips (step count and loss
scale kept on the device, zero_adam_step_async) against the oracle: step by
step, and replayed from a HIP graph that holds the flatten and the step.

Bar as for the synchronous step: flags, applied-step count and the loss-scale
trajectory identical; flat shard bit-identical; master / moments within 1e-6
relative and parameters within 1 ulp (expected: identical bits).  Graph tests
replay the captured step many times with eager work (new gradients, state
read-back) between replays and check every replay.
"""
import ctypes

import pytest

import zero_partitioned_mixed_plan_amd as z
from harness import (Case, DeviceRun, OracleRun, compare_full, compare_state, log, to_device_grad,
                     torch_dtype)
from synth.workloads import get

pytestmark = pytest.mark.gpu

RAGGED = [3000, 1, 7, 100003, 65, 2048, 511, 300000, 13, 0, 4099, 77777]


def _run(case, label, **kw):
    log(f"[async] {label}: P={sum(case.numels)} R={case.world_size} r={case.rank} "
        f"grads={case.grad_dtype} flatten={case.flatten_mode} param={case.param_mode} "
        f"steps={case.steps}")
    worst = compare_full(case, label=label, mode="async", **kw)
    log(f"[async] {label}: {worst}")
    return worst


def test_async_tiny_ten_steps_with_overflow_at_step_four():
    case = Case.from_workload(get("tiny"), inject={4: 2624 // 2})
    worst = _run(case, "tiny")
    assert worst["skipped"] == 1 and worst["bit_exact"]


@pytest.mark.parametrize("flatten_mode", ["all", "buckets_shuffled", "scan"])
def test_async_scaler_growth_and_backoff(flatten_mode):
    case = Case(numels=RAGGED, world_size=2, rank=0, grad_dtype="f16", param_dtype="f16",
                steps=9, dynamic=True, init_scale=256.0, window=2, bucket_elems=50000,
                inject={3: 10, 4: 70000, 8: 0}, flatten_mode=flatten_mode)
    worst = _run(case, f"scaler/{flatten_mode}")
    assert worst["skipped"] == 3 and worst["bit_exact"]


@pytest.mark.parametrize("adamw,param_mode", [(False, "full"), (True, "window"), (True, "none")])
def test_async_adam_variants_and_param_targets(adamw, param_mode):
    case = Case(numels=RAGGED, world_size=3, rank=2, grad_dtype="bf16", param_dtype="bf16",
                steps=4, grad_sigma=1e-2, adamw=adamw, weight_decay=0.1, param_mode=param_mode)
    assert _run(case, f"adamw={adamw} param={param_mode}")["bit_exact"]


def test_async_gpt2_small_thirty_steps():
    case = Case.from_workload(get("gpt2_small"), steps=30)
    assert _run(case, "gpt2_small", check_every=1)["bit_exact"]


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipMemcpy.restype = ctypes.c_int
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return lib


def _device_double(addr: int) -> float:
    out = ctypes.c_double(0)
    rc = _hip().hipMemcpy(ctypes.addressof(out), addr, 8, 2)   # device to host
    assert rc == 0, rc
    return out.value


def _graph_run(case, label, check_every=1):
    """Capture flatten + asynchronous step once; per iteration copy that
    iteration's gradients into the captured gradient buffers, replay, read the
    device state back and compare with the oracle."""
    import torch
    orc = OracleRun(case)
    gpu = DeviceRun(case, mode="async")
    p = gpu.plan
    gdt = torch_dtype(case.grad_dtype)
    touched = sorted({int(t) for t in orc.plan.seg_tensor})
    grads_dev = [None] * len(case.numels)
    for i in touched:
        grads_dev[i] = torch.zeros(case.numels[i], dtype=gdt, device=gpu.dev)
    param, base = gpu._param_args()
    scale_addr = z.zero_state_device_scale(p)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if case.flatten_mode == "buckets":
            tb = p.tensor_buckets()
            for b in range(p.n_buckets):
                z.zero_flatten_grads(p, b, [g if (g is not None and tb[i] == b) else None
                                            for i, g in enumerate(grads_dev)], gpu.flat)
        else:
            z.zero_flatten_grads(p, -1, grads_dev, gpu.flat)
        z.zero_adam_step_async(p, gpu.hp, gpu.flat, gpu.master, gpu.m, gpu.v, param, base)
    log(f"[graph] {label}: captured; S={p.S} real={p.real} segments={p.n_segments}")

    worst = dict(master=0.0, m=0.0, v=0.0, param_ulp=0, bit_exact=True, skipped=0)
    for it in range(1, case.steps + 1):
        before = z.zero_state_download(p)
        o_ovf, grads_host, o_scale = orc.step(it)
        assert before.scale == o_scale, f"{label} it={it}: scale {before.scale} vs {o_scale}"
        assert _device_double(scale_addr) == o_scale
        for i in touched:
            grads_dev[i].copy_(to_device_grad(grads_host[i], case.grad_dtype, gpu.dev))
        graph.replay()
        st = z.zero_state_download(p)
        assert st.last_flag == o_ovf, f"{label} it={it}: flag {st.last_flag} vs {o_ovf}"
        assert st.applied_steps == orc.t and st.skipped_steps == worst["skipped"] + o_ovf
        worst["skipped"] += o_ovf
        if it % check_every == 0 or it == case.steps:
            compare_state(gpu, orc, worst, f"{label} replay {it}")
    log(f"[graph] {label}: {worst}")
    return worst


def test_graph_replay_tiny_dynamic_scale_with_overflow():
    case = Case.from_workload(get("tiny"), inject={4: 2624 // 2})
    worst = _graph_run(case, "tiny")
    assert worst["skipped"] == 1 and worst["bit_exact"]


def test_graph_replay_ragged_scaler_growth_and_backoff():
    case = Case(numels=RAGGED, world_size=2, rank=1, grad_dtype="f16", param_dtype="f16",
                steps=10, dynamic=True, init_scale=512.0, window=2,
                inject={2: 5, 3: 100000, 7: 1})
    worst = _graph_run(case, "ragged")
    assert worst["skipped"] == 3 and worst["bit_exact"]


def test_graph_replay_fp32_gradients_dynamic_scale():
    case = Case(numels=RAGGED, world_size=2, rank=1, grad_dtype="f32", param_dtype="bf16",
                steps=8, dynamic=True, init_scale=512.0, window=2, grad_sigma=1e-2,
                inject={2: 5, 5: 100000})
    worst = _graph_run(case, "fp32 grads")
    assert worst["skipped"] == 2 and worst["bit_exact"]


def test_async_fp32_gradients():
    case = Case(numels=RAGGED, world_size=3, rank=0, grad_dtype="f32", param_dtype="f16",
                steps=5, dynamic=True, init_scale=1024.0, window=2, bucket_elems=50000,
                inject={3: 77}, flatten_mode="buckets_shuffled")
    worst = _run(case, "fp32 grads")
    assert worst["skipped"] == 1 and worst["bit_exact"]


def test_graph_replay_gpt2_small():
    case = Case.from_workload(get("gpt2_small"), steps=12)
    worst = _graph_run(case, "gpt2_small", check_every=1)
    assert worst["bit_exact"]


def test_async_needs_uploaded_state():
    import torch
    plan = z.zero_partition_plan([1000], 1, 0, 8)
    flat = torch.zeros(1000, dtype=torch.bfloat16, device="cuda:0")
    st = torch.zeros(1000, device="cuda:0")
    with pytest.raises(z.ZeroError) as e:
        z.zero_adam_step_async(plan, z.AdamHParams(), flat, st, st.clone(), st.clone())
    assert e.value.code == z._abi.ZERO_ESTATE
    with pytest.raises(z.ZeroError):
        z.zero_state_download(plan)
    bad = z.LossScaler(0.0)
    with pytest.raises(z.ZeroError):
        z.zero_state_upload(plan, 0, bad)


@pytest.mark.parametrize("seed", range(40))
def test_graph_replay_random_configuration(seed):
    """The seeded random configurations of the device parity sweep, captured
    once (flatten of all buckets, or bucket by bucket in order, inside the
    capture) and replayed step by step."""
    import dataclasses

    from test_gpu_random_parity import random_case
    case = random_case(seed)
    case = dataclasses.replace(case, flatten_mode="buckets" if seed % 2 else "all")
    label = (f"graph random seed={seed} numels={case.numels} R={case.world_size} "
             f"r={case.rank} A={case.align} grads={case.grad_dtype} params={case.param_dtype} "
             f"param={case.param_mode} flatten={case.flatten_mode}")
    worst = _graph_run(case, label)
    assert worst["bit_exact"], worst
