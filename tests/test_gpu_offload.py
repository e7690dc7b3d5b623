"""ZeRO-Offload pipeline (zero_offload_*) on the GPU against the oracle.

Each iteration: wait_params(lag), a stand-in "forward" that copies the
device parameter buffer, the gradients of the iteration copied to the
device, zero_flatten_grads, submit.  Checked:
  * what the forward of iteration it sees is exactly the oracle's parameters
    after iteration it - 1 - lag (lag 1: the one-step delayed update; lag 0:
    the serialised step) -- so the parameter copy never lands early or late;
  * the device loss scale before each iteration equals the oracle's;
  * after drain: host master / moments and the device parameters equal the
    oracle's bit for bit, and the applied / skipped counts match;
  * where a timeline is recorded: every piece's copies and update in the
    order the pipeline must run them (an update after its gradient arrived,
    a parameter copy after its update).
"""
import numpy as np
import pytest

import zero_partitioned_mixed_plan_amd as z
from harness import Case, OracleRun, init_master_host, init_param_host, log, \
    to_device_grad, torch_dtype
from synth.workloads import get

pytestmark = pytest.mark.gpu

RAGGED = [3000, 1, 7, 100003, 65, 2048, 511, 300000, 13, 0, 4099, 77777]


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


_EPS_MS = 0.05  # clock mapping of the timeline: the host's polling of one reference event


def _check_timeline(tl, steps, skipped_steps, write_params, real, S, label):
    """The recorded intervals against what the pipeline must do: every step
    copies every gradient piece in order; every applied step updates every
    piece after its gradient arrived, in order, and copies back the pieces
    holding real parameters only after their update."""
    by = {}
    for r in tl:
        assert r["end_ms"] >= r["start_ms"] - _EPS_MS, (label, r)
        by.setdefault((r["step"], r["kind"]), {})[r["piece"]] = (r["start_ms"], r["end_ms"])
    grads0 = by.get((0, "gradient copy"), {})
    n = len(grads0)
    assert n >= 1 and sorted(grads0) == list(range(n)), (label, sorted(grads0))
    sent_pieces = None
    for j in range(steps):
        g = by.get((j, "gradient copy"), {})
        assert sorted(g) == list(range(n)), (label, j, "gradient pieces")
        for c in range(1, n):
            assert g[c][0] >= g[c - 1][1] - _EPS_MS, (label, j, c, "gradient copies out of order")
        u = by.get((j, "host update"), {})
        h = by.get((j, "parameter copy"), {})
        if j in skipped_steps:
            assert not u and not h, (label, j, "a skipped step updated or copied")
            continue
        assert sorted(u) == list(range(n)), (label, j, "update pieces")
        for c in range(n):
            assert u[c][0] >= g[c][1] - _EPS_MS, (label, j, c, "update before its gradient")
            if c:
                assert u[c][0] >= u[c - 1][1] - _EPS_MS, (label, j, c, "updates out of order")
        if not write_params or real == 0:
            assert not h, (label, j, "parameters copied without param_dtype")
            continue
        assert h and sorted(h) == list(range(len(h))), (label, j, sorted(h))
        assert len(h) == n if real == S else len(h) <= n, (label, j, len(h), n)
        sent_pieces = len(h) if sent_pieces is None else sent_pieces
        assert len(h) == sent_pieces, (label, j, "parameter pieces vary between steps")
        for c in h:
            assert h[c][0] >= u[c][1] - _EPS_MS, (label, j, c, "parameters sent before the update")


def _offload_run(case, lag, label, write_params=True, n_threads=4, timeline=False):
    import torch
    dev = torch.device("cuda:0")
    orc = OracleRun(case)
    op = orc.plan
    plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                 case.bucket_elems)
    S, real, begin = plan.S, plan.real, plan.begin
    hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay, case.adamw)
    scaler = z.LossScaler(case.init_scale, dynamic=case.dynamic, window=case.window)
    z.zero_state_upload(plan, 0, scaler)
    master = init_master_host(case, begin, real, S)
    mom = np.zeros(S, np.float32)
    var = np.zeros(S, np.float32)
    gdt = torch_dtype(case.grad_dtype)
    param = torch.from_numpy(init_param_host(case, op.P).view(np.int16)).to(dev).view(
        torch_dtype(case.param_dtype))
    flat = torch.empty(max(S, 1), dtype=gdt, device=dev)
    off = z.Offload(plan, hp, case.grad_dtype, case.param_dtype if write_params else None,
                    master, mom, var, n_threads=n_threads)
    if timeline:
        off.timeline_start()
    hist = [orc.params().copy()]       # oracle parameters after iteration k
    skipped = 0
    skipped_steps = set()
    log(f"[offload] {label}: S={S} real={real} lag={lag} steps={case.steps}")
    for it in range(1, case.steps + 1):
        off.wait_params(lag)
        seen = param.clone()          # the forward of this iteration reads the parameters
        st = z.zero_state_download(plan)
        o_ovf, grads, o_scale = orc.step(it)
        assert st.scale == o_scale, f"{label} it={it}: device scale {st.scale} vs {o_scale}"
        grads_dev = [None if g is None else to_device_grad(g, case.grad_dtype, dev)
                     for g in grads]
        z.zero_flatten_grads(plan, -1, grads_dev, flat)
        off.submit(flat, param if write_params else None, 0)
        skipped += o_ovf
        if o_ovf:
            skipped_steps.add(it - 1)
        hist.append(orc.params().copy())
        if write_params:
            want = hist[max(it - 1 - lag, 0)]
            assert np.array_equal(_bits(seen), want), \
                f"{label} it={it}: the forward saw other parameters than iteration {it - 1 - lag}'s"
    off.drain()
    if timeline:
        _check_timeline(off.timeline(), case.steps, skipped_steps, write_params, real, S, label)
    stats = off.stats()
    assert stats["applied"] == orc.t and stats["skipped"] == skipped, stats
    assert stats["submitted"] == stats["processed"] == case.steps, stats
    for k in ("host_ms_total", "wait_submit_ms_total", "wait_grad_ms_total",
              "wait_h2d_ms_total", "wait_release_ms_total", "caller_wait_ms_total"):
        assert np.isfinite(stats[k]) and stats[k] >= 0.0, (k, stats)
    st = z.zero_state_download(plan)
    assert (st.applied_steps, st.skipped_steps, st.scale) == (orc.t, skipped, orc.scaler.value)
    for name, a, b in (("master", master, orc.master), ("m", mom, orc.m), ("v", var, orc.v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{label}: {name} differs"
    final = _bits(param)
    if write_params:
        assert np.array_equal(final, hist[-1]), f"{label}: final parameters differ"
    else:
        assert np.array_equal(final, hist[0]), f"{label}: parameters written without param_dtype"
    off.close()
    log(f"[offload] {label}: ok, applied {orc.t}, skipped {skipped}, "
        f"host ms last {stats['host_ms_last']:.2f}")
    return skipped


@pytest.mark.parametrize("lag", [1, 0])
def test_offload_tiny_with_overflow_at_step_four(lag):
    case = Case.from_workload(get("tiny"), inject={4: 2624 // 2})
    assert _offload_run(case, lag, f"tiny lag={lag}") == 1


@pytest.mark.parametrize("lag", [1, 0])
def test_offload_ragged_scaler_growth_and_backoff(lag):
    case = Case(numels=RAGGED, world_size=2, rank=1, grad_dtype="f16", param_dtype="f16",
                steps=10, dynamic=True, init_scale=512.0, window=2,
                inject={2: 5, 3: 100000, 7: 1})
    assert _offload_run(case, lag, f"ragged lag={lag}") == 3


def test_offload_bf16_padding_rank_and_no_param_write():
    case = Case(numels=RAGGED, world_size=3, rank=2, grad_dtype="bf16", param_dtype="bf16",
                steps=4, grad_sigma=1e-2, adamw=False, weight_decay=0.1)
    _offload_run(case, 1, "bf16 adam-l2")
    _offload_run(case, 1, "bf16 no param write", write_params=False)


@pytest.mark.parametrize("lag", [1, 0])
def test_offload_fp32_gradients(lag):
    case = Case(numels=RAGGED, world_size=2, rank=0, grad_dtype="f32", param_dtype="bf16",
                steps=6, dynamic=True, init_scale=512.0, window=2, grad_sigma=1e-2,
                inject={3: 4097})
    assert _offload_run(case, lag, f"fp32 grads lag={lag}") == 1


@pytest.mark.parametrize("lag", [1, 0])
def test_offload_in_many_pieces(lag, monkeypatch):
    """Copies and update in 16 pieces (the piece size lowered for the test):
    a short last piece, pieces past the real range (padding rank), parameter
    copies sent piece by piece (lag 0) or after the update (lag 1), and a
    skipped step in between."""
    monkeypatch.setenv("ZERO_OFFLOAD_MIN_CHUNK", "4096")
    case = Case(numels=RAGGED, world_size=3, rank=2, grad_dtype="f16", param_dtype="f16",
                steps=7, dynamic=True, init_scale=1024.0, window=2, grad_sigma=1e-2,
                inject={4: 99999})
    assert _offload_run(case, lag, f"pieces lag={lag}", timeline=True) == 1
    case = Case(numels=RAGGED, world_size=2, rank=1, grad_dtype="f32", param_dtype="bf16",
                steps=4, grad_sigma=1e-2)
    assert _offload_run(case, lag, f"pieces fp32 lag={lag}", timeline=True) == 0


def test_offload_gpt2_small():
    case = Case.from_workload(get("gpt2_small"), steps=6)
    _offload_run(case, 1, "gpt2_small", n_threads=8, timeline=True)


@pytest.mark.parametrize("seed", range(60))
def test_offload_random_configuration(seed, monkeypatch):
    """The seeded random configurations of the device parity sweep, through
    the offload pipeline, with a random lag, parameter write-back or not,
    1-6 host threads and a random piece size (so 1 to 16 pieces)."""
    import random

    from test_gpu_random_parity import random_case
    rnd = random.Random(10_000 + seed)
    case = random_case(seed)
    lag = rnd.choice([0, 1])
    write_params = rnd.random() < 0.8
    threads = rnd.randint(1, 6)
    piece = rnd.choice([64, 256, 4096, None])
    if piece is not None:
        monkeypatch.setenv("ZERO_OFFLOAD_MIN_CHUNK", str(piece))
    timeline = rnd.random() < 0.5
    label = (f"offload random seed={seed} numels={case.numels} R={case.world_size} "
             f"r={case.rank} A={case.align} grads={case.grad_dtype} params={case.param_dtype} "
             f"adamw={case.adamw} inject_p={case.inject_p} lag={lag} write={write_params} "
             f"threads={threads} piece={piece} timeline={timeline}")
    _offload_run(case, lag, label, write_params=write_params, n_threads=threads,
                 timeline=timeline)
