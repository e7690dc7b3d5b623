"""Elastic re-planning: a run that changes its data-parallel degree.

Every rank's state is a contiguous shard [begin, begin + S) of the flat
model, so a checkpoint consolidates by concatenating the shards in rank
order and truncating at P, and a new plan for another degree (or another
alignment) scatters the consolidated state again.  Because the update is
elementwise, the run continued at the new degree must equal, bit for bit,
the same number of steps of the unpartitioned update ("ZeRO Optimization",
inferensys genomic MLOps page, checkpoint consolidation and elastic-training
bullets; ZeRO-1 paragraph of the instruction-tuning page for the partition).

Schedule: 3 steps at R = 8 (align 64), consolidate, 3 steps at R = 4
(align 64), consolidate, 2 steps at R = 3 (align 8); the step count t
carries over.  The CPU test steps each rank's shard with the oracle and
uses the library's planner for every offset; the GPU test steps each rank
through the HIP path into one shared parameter buffer.
"""
import numpy as np
import pytest

import oracle
import synth
import zero_partitioned_mixed_plan_amd as z

NUMELS = [3000, 1, 7, 100003, 65, 2048, 511, 30000, 13, 0, 4099]
P = sum(NUMELS)
SCHEDULE = [(8, 64, 3), (4, 64, 3), (3, 8, 2)]   # (R, align, steps)
HP = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, adamw=True)


def _inputs():
    rng = np.random.default_rng(7)
    steps = sum(s for _, _, s in SCHEDULE)
    grads = [[synth.half_bits(rng.normal(0, 1e-2, n).astype(np.float32), "bf16") for n in NUMELS]
             for _ in range(steps)]
    return rng.normal(0, 0.02, P).astype(np.float32), grads


def _unpartitioned(master0, grads):
    op = oracle.plan(NUMELS, 1, 0, 1)
    m = np.zeros(op.S, np.float32)
    m[:P] = master0
    mo, v = np.zeros_like(m), np.zeros_like(m)
    for t, g in enumerate(grads, 1):
        assert oracle.adam_step(t, 1.0, oracle.flatten(op, g), "bf16", m, mo, v, **HP) == 0
    param = np.zeros(P, np.uint16)
    oracle.write_param(m, P, 0, 0, param, "bf16")
    return m[:P], mo[:P], v[:P], param


def _consolidate(plans, shards):
    """Rank order, truncated at P: the checkpoint's consolidated state."""
    whole = np.concatenate(shards)
    assert whole.size == plans[0].P_pad
    out = whole[:P].copy()
    for plan, sh in zip(plans, shards):   # the same, by each plan's own range
        assert np.array_equal(out[plan.begin:plan.begin + plan.real].view(np.uint32),
                              sh[:plan.real].view(np.uint32))
        assert not sh[plan.real:].any(), "padding must stay zero"
    return out


def _scatter(plan, full):
    sh = np.zeros(plan.S, np.float32)
    sh[:plan.real] = full[plan.begin:plan.begin + plan.real]
    return sh


def test_replan_on_the_cpu_equals_the_unpartitioned_update():
    master0, grads = _inputs()
    want = _unpartitioned(master0, grads)
    full = [master0.copy(), np.zeros(P, np.float32), np.zeros(P, np.float32)]
    param = np.zeros(P, np.uint16)
    t = 0
    for R, A, steps in SCHEDULE:
        plans = [z.zero_partition_plan(NUMELS, R, r, A) for r in range(R)]
        oplans = [oracle.plan(NUMELS, R, r, A) for r in range(R)]
        state = [[_scatter(p, f) for f in full] for p in plans]
        for k in range(steps):
            for p, op, (m, mo, v) in zip(plans, oplans, state):
                assert (op.S, op.begin, op.real) == (p.S, p.begin, p.real)
                flat = oracle.flatten(op, grads[t + k])
                assert oracle.adam_step(t + k + 1, 1.0, flat, "bf16", m, mo, v, **HP) == 0
                oracle.write_param(m, p.real, p.begin, 0, param, "bf16")
        t += steps
        full = [_consolidate(plans, [st[i] for st in state]) for i in range(3)]
    for name, got, exp in zip(("master", "m", "v"), full, want[:3]):
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), name
    assert np.array_equal(param, want[3])


@pytest.mark.gpu
def test_replan_on_the_gpu_equals_the_unpartitioned_update():
    import torch
    dev = torch.device("cuda:0")
    master0, grads = _inputs()
    want = _unpartitioned(master0, grads)
    full = [master0.copy(), np.zeros(P, np.float32), np.zeros(P, np.float32)]
    param = torch.zeros(P, dtype=torch.bfloat16, device=dev)
    hp = z.AdamHParams(HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], HP["adamw"])
    t = 0
    for R, A, steps in SCHEDULE:
        plans = [z.zero_partition_plan(NUMELS, R, r, A) for r in range(R)]
        shards = []
        for p in plans:
            st = [torch.from_numpy(_scatter(p, f)).to(dev) for f in full]
            flat = torch.empty(p.S, dtype=torch.bfloat16, device=dev)
            for k in range(steps):
                g = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
                     for x in grads[t + k]]
                z.zero_flatten_grads(p, -1, g, flat)
                assert z.zero_adam_step(p, hp, t + k + 1, 1.0, flat, *st, param, 0) == 0
            shards.append([x.cpu().numpy() for x in st])
        t += steps
        full = [_consolidate(plans, [sh[i] for sh in shards]) for i in range(3)]
    for name, got, exp in zip(("master", "m", "v"), full, want[:3]):
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), name
    got_param = param.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_param, want[3])
