"""Host-side checks of libzero_mi355x (CPU only, no device compute).

* the library loads and exports every function include/*.h declares;
* its planner agrees with the oracle's on every rank of every workload, on
  random small models, and on generated ones with tensors of up to 2^40
  elements (sizes, segments, buckets, byte accounting);
* its loss-scale policy agrees with the oracle's on random sequences;
* argument errors are reported before any device work.
"""
import ctypes
import glob
import os
import random
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
import zero_partitioned_mixed_plan_amd as z
from zero_partitioned_mixed_plan_amd import _abi
from synth.workloads import WORKLOADS, get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"zero_partition_plan", "zero_flatten_grads", "zero_adam_step",
            "zero_update_loss_scale", "zero_write_param_shard"} <= names
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    # and the binding declares a signature for each
    assert names == set(_abi.SIGNATURES)


def _compare(numels, R, r, A, B):
    op = oracle.plan(numels, R, r, A, B)
    zp = z.zero_partition_plan(numels, R, r, A, B)
    assert (zp.P, zp.P_pad, zp.S, zp.begin, zp.real) == (op.P, op.P_pad, op.S, op.begin, op.real)
    assert zp.n_buckets == op.n_buckets and zp.n_segments == op.n_segments
    segs = zp.segments()
    got = [(s.tensor, s.tensor_off, s.shard_off, s.numel) for s in segs]
    exp = list(zip(op.seg_tensor.tolist(), op.seg_tensor_off.tolist(), op.seg_shard_off.tolist(),
                   op.seg_numel.tolist()))
    assert got == exp
    tb = zp.tensor_buckets()
    assert tb == op.tensor_bucket.tolist()
    assert [s.bucket for s in segs] == [tb[t] for t, *_ in got]
    i = zp.info
    assert (i.bytes_stage1, i.bytes_stage2, i.bytes_stage3) == (
        op.bytes_stage1, op.bytes_stage2, op.bytes_stage3)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_planner_matches_oracle_on_workloads(name):
    w = get(name)
    for r in range(w.world_size):
        for B in (w.bucket_elems, 1 << 20):
            _compare(w.numels, w.world_size, r, w.align, B)


@pytest.mark.parametrize("seed", range(60))
def test_planner_matches_oracle_random(seed):
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 2, 7, 64, 100, 4097]) for _ in range(rng.randint(0, 12))]
    R = rng.randint(1, 9)
    A = rng.choice([1, 3, 8, 64])
    B = rng.choice([1, 50, 1000, 1 << 25])
    for r in range(R):
        _compare(numels, R, r, A, B)


@settings(max_examples=400, deadline=None, derandomize=True, database=None)
@given(numels=st.lists(st.one_of(st.integers(0, 70), st.integers(0, 1 << 40)), max_size=24),
       R=st.integers(1, 64), A=st.sampled_from([1, 2, 3, 8, 64, 128, 4096]),
       B=st.one_of(st.integers(1, 100), st.integers(1, 1 << 42)), data=st.data())
def test_planner_matches_oracle_at_any_size(numels, R, A, B, data):
    # sizes up to 2^40 elements a tensor and 64 ranks: the int64 offsets,
    # padding and bucket sums far beyond the workloads
    _compare(numels, R, data.draw(st.integers(0, R - 1)), A, B)


@pytest.mark.parametrize("seed", range(20))
def test_loss_scale_policy_matches_oracle(seed):
    rng = random.Random(seed)
    dynamic = rng.random() < 0.8
    init = rng.choice([1.0, 1024.0, 65536.0])
    window = rng.randint(1, 5)
    zs = z.LossScaler(init, dynamic=dynamic, window=window, min_scale=1.0)
    os_ = oracle.Scaler(init, dynamic=dynamic, window=window, min_scale=1.0)
    for _ in range(200):
        ovf = 1 if rng.random() < 0.3 else 0
        z.zero_update_loss_scale(zs, ovf)
        os_.update(ovf)
        assert zs.scale == os_.value
        assert zs.good_steps == os_.good.value


def test_argument_errors_before_device_work():
    lib = _abi.lib
    h = ctypes.c_void_p()
    bad_plans = [([4], 0, 0, 1, 1), ([4], 2, 2, 1, 1), ([4], 1, 0, 0, 1), ([4], 1, 0, 1, 0),
                 ([-3], 1, 0, 1, 1)]
    for numels, R, r, A, B in bad_plans:
        arr = (ctypes.c_int64 * 1)(*numels)
        assert lib.zero_partition_plan(arr, 1, R, r, A, B, ctypes.byref(h)) == _abi.ZERO_EINVAL
        assert z.zero_last_error() != ""
    assert lib.zero_partition_plan(None, 1, 1, 0, 1, 1, ctypes.byref(h)) == _abi.ZERO_ENULL
    assert lib.zero_partition_plan(None, 0, 1, 0, 1, 1, None) == _abi.ZERO_ENULL
    # total size overflow
    arr = (ctypes.c_int64 * 2)(1 << 62, 1 << 62)
    assert lib.zero_partition_plan(arr, 2, 1, 0, 1, 1, ctypes.byref(h)) == _abi.ZERO_EINVAL

    plan = z.zero_partition_plan([1000], 2, 0, 8)
    hp = z.AdamHParams().to_c()
    fake = 1 << 20  # 16-byte aligned, never dereferenced on these error paths
    args = dict(step=1, scale=1.0, g=fake, gdt=z.ZERO_BF16, p=fake, m=fake, v=fake)

    def step(**kw):
        a = dict(args, **kw)
        return lib.zero_adam_step(plan.handle, ctypes.byref(hp), a["step"], a["scale"], a["g"],
                                  a["gdt"], a["p"], a["m"], a["v"], None, 0, 0, 0, None)
    assert step(step=0) == _abi.ZERO_EINVAL
    assert step(scale=0.0) == _abi.ZERO_EINVAL
    assert step(scale=float("inf")) == _abi.ZERO_EINVAL
    assert step(gdt=7) == _abi.ZERO_EINVAL
    assert step(g=None) == _abi.ZERO_ENULL
    assert step(m=fake + 2) == _abi.ZERO_EALIGN
    assert step(g=fake + 8) == _abi.ZERO_EALIGN
    bad_hp = z.AdamHParams(beta1=1.0).to_c()
    assert lib.zero_adam_step(plan.handle, ctypes.byref(bad_hp), 1, 1.0, fake, z.ZERO_BF16, fake,
                              fake, fake, None, 0, 0, 0, None) == _abi.ZERO_EINVAL
    # a parameter window that misses the shard
    assert lib.zero_adam_step(plan.handle, ctypes.byref(hp), 1, 1.0, fake, z.ZERO_BF16, fake,
                              fake, fake, fake, 10, 100, z.ZERO_BF16, None) == _abi.ZERO_EINVAL
    assert lib.zero_write_param_shard(plan.handle, fake, fake, 0, 10, z.ZERO_BF16,
                                      None) == _abi.ZERO_EINVAL
    assert lib.zero_write_param_shard(plan.handle, fake + 2, fake, 0, 1000, z.ZERO_BF16,
                                      None) == _abi.ZERO_EALIGN
    ptrs = (ctypes.c_void_p * 1)(None)
    assert lib.zero_flatten_grads(plan.handle, 5, ptrs, z.ZERO_BF16, fake,
                                  None) == _abi.ZERO_EINVAL
    assert lib.zero_flatten_grads(plan.handle, -1, ptrs, z.ZERO_BF16, fake,
                                  None) == _abi.ZERO_ENULL
    ptrs = (ctypes.c_void_p * 1)(fake + 1)
    assert lib.zero_flatten_grads(plan.handle, -1, ptrs, z.ZERO_BF16, fake,
                                  None) == _abi.ZERO_EALIGN
    assert lib.zero_flatten_grads(plan.handle, -1, ptrs, z.ZERO_BF16, fake + 2,
                                  None) == _abi.ZERO_EALIGN
    # fp32 gradients: 4-byte sources
    ptrs = (ctypes.c_void_p * 1)(fake + 2)
    assert lib.zero_flatten_grads(plan.handle, -1, ptrs, z.ZERO_F32, fake,
                                  None) == _abi.ZERO_EALIGN
    assert lib.zero_flatten_grads(plan.handle, -1, ptrs, 4, fake, None) == _abi.ZERO_EINVAL
    assert step(gdt=z.ZERO_F32, g=fake + 4) == _abi.ZERO_EALIGN
    bad = _abi.zero_scaler_t(0.0, 1.0, 0.5, 2.0, 10, 0, 1, 0)
    assert lib.zero_update_loss_scale(ctypes.byref(bad), 0) == _abi.ZERO_EINVAL
    assert lib.zero_update_loss_scale(None, 0) == _abi.ZERO_ENULL
    assert lib.zero_flatten_invalidate(None) == _abi.ZERO_ENULL
    assert lib.zero_offload_timeline_start(None, 16) == _abi.ZERO_ENULL
    assert lib.zero_offload_timeline(None, None, 0) == _abi.ZERO_ENULL
    assert lib.zero_flatten_invalidate(plan.handle) == _abi.ZERO_OK


def test_async_step_argument_errors_before_device_work():
    """The asynchronous step validates its arguments, then refuses to run on a
    plan whose device state was never uploaded -- all before any device call."""
    lib = _abi.lib
    plan = z.zero_partition_plan([1000], 2, 0, 8)
    hp = z.AdamHParams().to_c()
    fake = 1 << 20  # 16-byte aligned, never dereferenced on these error paths

    def step(g=fake, gdt=z.ZERO_BF16, m=fake, hpp=hp, param=None, base=0, numel=0, pdt=0):
        return lib.zero_adam_step_async(plan.handle, ctypes.byref(hpp), g, gdt, fake, m, fake,
                                        param, base, numel, pdt, None)
    assert step(gdt=4) == _abi.ZERO_EINVAL
    assert step(g=None) == _abi.ZERO_ENULL
    assert step(g=fake + 4) == _abi.ZERO_EALIGN
    assert step(m=fake + 1) == _abi.ZERO_EALIGN
    assert step(hpp=z.AdamHParams(eps=0.0).to_c()) == _abi.ZERO_EINVAL
    assert step(param=fake, base=10, numel=100, pdt=z.ZERO_BF16) == _abi.ZERO_EINVAL
    assert step() == _abi.ZERO_ESTATE
    assert "zero_state_upload" in z.zero_last_error()
    assert lib.zero_adam_step_async(None, ctypes.byref(hp), fake, z.ZERO_BF16, fake, fake, fake,
                                    None, 0, 0, 0, None) == _abi.ZERO_ENULL
    out = ctypes.c_void_p()
    assert lib.zero_state_device_scale(plan.handle, ctypes.byref(out)) == _abi.ZERO_ESTATE
    assert lib.zero_state_download(plan.handle, None, None, None, None, None) == _abi.ZERO_ESTATE
    sc = _abi.zero_scaler_t(1024.0, 1.0, 0.5, 2.0, 0, 0, 1, 0)        # window 0
    assert lib.zero_state_upload(plan.handle, 0, ctypes.byref(sc), None) == _abi.ZERO_EINVAL
    sc = _abi.zero_scaler_t(1024.0, 1.0, 0.5, 2.0, 10, 0, 1, 0)
    assert lib.zero_state_upload(plan.handle, -1, ctypes.byref(sc), None) == _abi.ZERO_EINVAL
    assert lib.zero_state_upload(None, 0, ctypes.byref(sc), None) == _abi.ZERO_ENULL


def test_grad_list_checks_when_bound():
    import torch
    plan = z.zero_partition_plan([1000, 24], 2, 0, 8)
    with pytest.raises(ValueError, match="need 2 gradient entries"):
        z.GradList(plan, [None])
    with pytest.raises(ValueError, match="device tensor"):
        z.GradList(plan, [torch.zeros(1000, dtype=torch.bfloat16), None])
    with pytest.raises(TypeError, match="torch tensor"):
        z.GradList(plan, [np.zeros(1000, np.uint16), None])
    empty = z.GradList(plan, [None, None])   # nothing bound: no dtype to check
    assert empty.dtype is None and list(empty.ptrs) == [None, None]


def test_offload_argument_errors_before_device_work():
    lib = _abi.lib
    plan = z.zero_partition_plan([1000], 2, 0, 8)
    hp = z.AdamHParams().to_c()
    fake = 1 << 20
    out = ctypes.c_void_p()
    create = lib.zero_offload_create
    assert create(plan.handle, ctypes.byref(hp), z.ZERO_BF16, z.ZERO_BF16, fake, fake, fake, 4,
                  None) == _abi.ZERO_ENULL
    assert create(plan.handle, ctypes.byref(hp), 9, z.ZERO_BF16, fake, fake, fake, 4,
                  ctypes.byref(out)) == _abi.ZERO_EINVAL
    assert create(plan.handle, ctypes.byref(hp), z.ZERO_BF16, 7, fake, fake, fake, 4,
                  ctypes.byref(out)) == _abi.ZERO_EINVAL
    assert create(plan.handle, ctypes.byref(hp), z.ZERO_BF16, z.ZERO_BF16, fake, fake, fake, 0,
                  ctypes.byref(out)) == _abi.ZERO_EINVAL
    assert create(plan.handle, ctypes.byref(hp), z.ZERO_BF16, z.ZERO_BF16, None, fake, fake, 4,
                  ctypes.byref(out)) == _abi.ZERO_ENULL
    for bad in (z.AdamHParams(lr=float("inf")), z.AdamHParams(eps=float("inf")),
                z.AdamHParams(beta2=1.0), z.AdamHParams(weight_decay=-1.0)):
        bhp = bad.to_c()
        assert create(plan.handle, ctypes.byref(bhp), z.ZERO_BF16, z.ZERO_BF16, fake, fake, fake,
                      4, ctypes.byref(out)) == _abi.ZERO_EINVAL
    # the device state must be uploaded first
    assert create(plan.handle, ctypes.byref(hp), z.ZERO_BF16, z.ZERO_BF16, fake, fake, fake, 4,
                  ctypes.byref(out)) == _abi.ZERO_ESTATE
    assert out.value is None
    assert lib.zero_offload_submit(None, fake, fake, 0, 1, None) == _abi.ZERO_ENULL
    assert lib.zero_offload_wait_params(None, 1, None) == _abi.ZERO_ENULL
    assert lib.zero_offload_drain(None, None) == _abi.ZERO_ENULL
    lib.zero_offload_destroy(None)


def test_adam_scalars_on_the_host():
    """zero_adam_scalars(on_device=0) gives the scalars zero_adam_step forms:
    each definition evaluated in float64 (Python's math library) and rounded
    once to fp32; argument errors are reported."""
    import math
    for hp, scale in ((z.AdamHParams(), 1024.0),
                      (z.AdamHParams(lr=0.5, beta1=0.99, beta2=0.95, eps=1e-3, weight_decay=0.2,
                                     adamw=False), 0.25)):
        got = z.zero_adam_scalars(hp, 1, 20000, scale)
        assert got.shape == (20000, len(z.SCALAR_FIELDS))
        for t in range(1, 20001):
            want = np.array([1.0 / scale, hp.beta1, 1.0 - hp.beta1, hp.beta2, 1.0 - hp.beta2,
                             hp.lr / (1.0 - math.pow(hp.beta1, t)),
                             1.0 / math.sqrt(1.0 - math.pow(hp.beta2, t)), hp.eps,
                             1.0 - hp.lr * hp.weight_decay if hp.adamw else 1.0,
                             hp.weight_decay], np.float64).astype(np.float32)
            assert np.array_equal(got[t - 1].view(np.uint32), want.view(np.uint32)), t
        # a window starting later is the same rows
        assert np.array_equal(z.zero_adam_scalars(hp, 777, 5, scale), got[776:781])
    lib = _abi.lib
    hp = z.AdamHParams().to_c()
    buf = np.zeros(40, np.float32)
    ptr = buf.ctypes.data
    assert lib.zero_adam_scalars(None, 1, 1, 1.0, ptr, 0, None) == _abi.ZERO_ENULL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 0, 1, 1.0, ptr, 0, None) == _abi.ZERO_EINVAL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, -1, 1.0, ptr, 0, None) == _abi.ZERO_EINVAL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, 1, 0.0, ptr, 0, None) == _abi.ZERO_EINVAL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, 1, 1.0, ptr, 2, None) == _abi.ZERO_EINVAL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, 1, 1.0, None, 0, None) == _abi.ZERO_ENULL
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, 1, 1.0, ptr + 2, 0, None) == _abi.ZERO_EALIGN
    assert lib.zero_adam_scalars(ctypes.byref(hp), 1, 0, 1.0, None, 0, None) == _abi.ZERO_OK
    bad = z.AdamHParams(beta2=1.0).to_c()
    assert lib.zero_adam_scalars(ctypes.byref(bad), 1, 1, 1.0, ptr, 0, None) == _abi.ZERO_EINVAL


def test_plans_are_released_explicitly_and_at_exit():
    """close() releases a plan once (later calls fail with ZERO_ENULL);
    release_all() releases every live plan; the binding registers it with
    atexit, so nothing is left for a destructor during interpreter
    finalization."""
    import atexit
    a = z.zero_partition_plan([1000, 24], 2, 0, 8)
    b = z.zero_partition_plan([77], 1, 0, 1)
    a.close()
    a.close()                                    # idempotent
    with pytest.raises(z.ZeroError):
        a.segments()
    assert b in z._LIVE_PLANS
    z.release_all()
    with pytest.raises(z.ZeroError):
        b.tensor_buckets()
    # the hook is registered: unregister returns quietly only for a known one
    atexit.unregister(z.release_all)
    atexit.register(z.release_all)


_EXIT_SCRIPT = r"""
import atexit, sys
sys.path.insert(0, {root!r})
import zero_partitioned_mixed_plan_amd as z
calls = []
real = z.Plan._destroy
def spy(h):
    print("destroy finalizing=%d" % sys.is_finalizing(), flush=True)
    real(h)
z.Plan._destroy = staticmethod(spy)
if {unhook}:
    atexit.unregister(z.release_all)
KEEP = [z.zero_partition_plan([1000, 24], 2, 0, 8) for _ in range(3)]
print("exiting", flush=True)
"""


@pytest.mark.parametrize("unhook", [False, True])
def test_no_library_call_during_interpreter_finalization(unhook):
    """Plans still referenced at exit: with the atexit hook they are released
    before finalization (three destroys, none while finalizing); without it
    their destructors make no library call at all while finalizing."""
    import subprocess
    import sys
    code = _EXIT_SCRIPT.format(root=ROOT, unhook=unhook)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = r.stdout.split()
    assert "exiting" in lines
    out = r.stdout.splitlines()
    destroys = [x for x in out if x.startswith("destroy")]
    if unhook:
        assert destroys == []
    else:
        assert destroys == ["destroy finalizing=0"] * 3
