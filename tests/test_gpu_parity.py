"""GPU vs oracle parity over whole shards (the HIP library through its C ABI).

Bar (checked after every step): overflow flags, loss-scale trajectory and
the applied-step counter identical; the flat gradient shard bit-identical;
fp32 master / momentum / variance within a max relative error of 1e-6
(the pinned operation order makes the expected difference zero); half
parameters within 1 ulp (expected zero).
"""
import pytest

from harness import Case, compare_full, log
from synth.workloads import get

pytestmark = pytest.mark.gpu


def _run(case, label, **kw):
    log(f"[parity] {label}: P={sum(case.numels)} R={case.world_size} r={case.rank} "
        f"A={case.align} grads={case.grad_dtype} params={case.param_dtype} "
        f"flatten={case.flatten_mode} param={case.param_mode} steps={case.steps}")
    worst = compare_full(case, label=label, **kw)
    log(f"[parity] {label}: {worst}")
    return worst


def test_tiny_workload_ten_steps_with_overflow_at_step_four():
    w = get("tiny")
    # +inf at shard-local index real // 2 on iteration 4 (real = 2624 at A = 64)
    case = Case.from_workload(w, inject={4: 2624 // 2})
    worst = _run(case, "tiny")
    assert worst["skipped"] == 1
    assert worst["bit_exact"]


RAGGED = [3000, 1, 7, 100003, 65, 2048, 511, 300000, 13, 0, 4099, 77777]


@pytest.mark.parametrize("align", [1, 8, 64])
@pytest.mark.parametrize("gdt,pdt", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f16")])
def test_ragged_model_every_rank(align, gdt, pdt):
    for r in range(3):
        case = Case(numels=RAGGED, world_size=3, rank=r, grad_dtype=gdt, param_dtype=pdt,
                    steps=3, align=align, bucket_elems=50000, grad_sigma=1e-2,
                    dynamic=(gdt == "f16"), init_scale=(1024.0 if gdt == "f16" else 1.0),
                    inject={2: 1234} if gdt == "f16" else {},
                    flatten_mode="buckets_shuffled" if r == 1 else "all",
                    param_mode="window" if r == 2 else "full")
        worst = _run(case, f"ragged A={align} {gdt}/{pdt} r={r}")
        assert worst["bit_exact"]


@pytest.mark.parametrize("adamw", [True, False])
def test_adam_l2_and_adamw(adamw):
    case = Case(numels=RAGGED, world_size=2, rank=1, grad_dtype="bf16", param_dtype="bf16",
                steps=4, align=64, grad_sigma=1e-2, adamw=adamw, weight_decay=0.1)
    assert _run(case, f"adamw={adamw}")["bit_exact"]


def test_scan_path_when_flatten_did_not_fill_the_buffer():
    case = Case(numels=RAGGED, world_size=2, rank=0, grad_dtype="f16", param_dtype="f16",
                steps=4, align=64, grad_sigma=1e-2, dynamic=True, init_scale=4096.0,
                inject={3: 50001}, flatten_mode="scan")
    worst = _run(case, "scan")
    assert worst["skipped"] == 1 and worst["bit_exact"]


def test_no_param_write():
    case = Case(numels=RAGGED, world_size=4, rank=3, grad_dtype="bf16", param_dtype="bf16",
                steps=2, param_mode="none")
    assert _run(case, "no-param")["bit_exact"]


def test_rank_with_only_padding_and_empty_model():
    # P = 5 < R*A: ranks past the end own padding only
    for r in range(4):
        case = Case(numels=[2, 3], world_size=4, rank=r, grad_dtype="bf16", param_dtype="bf16",
                    steps=2, align=8)
        assert _run(case, f"pad-only r={r}")["bit_exact"]
    case = Case(numels=[], world_size=2, rank=1, grad_dtype="bf16", param_dtype="bf16", steps=1)
    _run(case, "empty")


def test_dynamic_scale_growth_and_backoff():
    case = Case(numels=RAGGED, world_size=2, rank=0, grad_dtype="f16", param_dtype="f16",
                steps=9, dynamic=True, init_scale=256.0, window=2,
                inject={3: 10, 4: 70000, 8: 0})
    worst = _run(case, "scaler")
    assert worst["skipped"] == 3 and worst["bit_exact"]


@pytest.mark.parametrize("align", [1, 64])
@pytest.mark.parametrize("pdt", ["bf16", "f16"])
def test_fp32_gradients_every_rank(align, pdt):
    """Gradients kept in fp32 (4-byte flatten, binary32 overflow test, no
    conversion in the update), with a dynamic scale: every flatten mode."""
    for r, mode in enumerate(["all", "buckets_shuffled", "scan"]):
        case = Case(numels=RAGGED, world_size=3, rank=r, grad_dtype="f32", param_dtype=pdt,
                    steps=5, align=align, bucket_elems=50000, grad_sigma=1e-2, dynamic=True,
                    init_scale=1024.0, window=2, inject={2: 1234, 4: 50001},
                    flatten_mode=mode, param_mode="window" if r == 2 else "full")
        worst = _run(case, f"fp32 grads A={align} {pdt} r={r} {mode}")
        assert worst["skipped"] == 2 and worst["bit_exact"]


def test_fp32_gradients_gpt2_small():
    case = Case.from_workload(get("gpt2_small"), grad_dtype="f32", steps=6)
    worst = _run(case, "gpt2_small fp32 grads", check_every=1)
    assert worst["bit_exact"]


def _has_subnormals(x):
    import numpy as np
    a = np.abs(x)
    return bool(np.any((a > 0) & (a < np.finfo(np.float32).tiny)))


@pytest.mark.parametrize("gdt,scale,sigma", [("f32", 1.0, 1e-20), ("f16", 2.0 ** 40, 1e-20),
                                             ("bf16", 1.0, 1e-20)])
def test_fp32_subnormals_are_kept(gdt, scale, sigma):
    """Gradients so small that g*g and the variance are fp32 subnormals, and a
    master of subnormals: the update must keep them (no flush to zero), as the
    oracle does, bit for bit."""
    from harness import DeviceRun, OracleRun, compare_state
    # lr 1e-25: each step moves the master by a subnormal amount, so it stays
    # subnormal and every step computes on subnormals
    case = Case(numels=RAGGED, world_size=2, rank=0, grad_dtype=gdt, param_dtype="bf16",
                steps=3, grad_sigma=sigma, master_sigma=1e-39, init_scale=scale,
                weight_decay=0.1, adamw=(gdt != "bf16"), lr=1e-25)
    orc, gpu = OracleRun(case), DeviceRun(case)
    worst = dict(master=0.0, m=0.0, v=0.0, param_ulp=0, bit_exact=True, skipped=0)
    for it in range(1, case.steps + 1):
        o_ovf, grads, _ = orc.step(it)
        g_ovf, _ = gpu.step(it, grads)
        assert g_ovf == o_ovf == 0
        compare_state(gpu, orc, worst, f"subnormals {gdt} it={it}")
    assert _has_subnormals(orc.v) and _has_subnormals(orc.master), \
        "the case no longer reaches fp32 subnormals"
    assert worst["bit_exact"]
    log(f"[parity] subnormals {gdt}: {worst}")


@pytest.mark.parametrize("label,hp", [
    ("no momentum (beta1 = beta2 = 0)", dict(beta1=0.0, beta2=0.0)),
    ("lr = 0 (AdamW leaves the master as it is)", dict(lr=0.0)),
    ("lr = 0, Adam-L2", dict(lr=0.0, adamw=False, weight_decay=0.5)),
    ("no decay (wd = 0)", dict(weight_decay=0.0)),
    ("large eps (1.0)", dict(eps=1.0)),
    ("beta2 close to 1", dict(beta2=0.999999)),
])
def test_degenerate_hyperparameters(label, hp):
    """Boundary settings the update must still compute exactly as the oracle."""
    base = dict(numels=RAGGED, world_size=2, rank=1, grad_dtype="bf16", param_dtype="bf16",
                steps=3, grad_sigma=1e-2)
    base.update(hp)
    worst = _run(Case(**base), label)
    assert worst["bit_exact"]


def test_gpt2_small_full_shard_all_steps():
    w = get("gpt2_small")
    case = Case.from_workload(w)
    worst = _run(case, "gpt2_small", check_every=1)
    assert worst["bit_exact"]
