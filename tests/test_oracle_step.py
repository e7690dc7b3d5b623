"""Pins of the oracle's flatten, loss-scale policy and whole step (CPU only).

Checked against: element-by-element brute force of the flatten, loss-scale
trajectories worked by hand, and the data-parallel equivalence of the
partitioned step: R shards updated separately and written back at their
offsets give exactly the unpartitioned (R = 1) step over the whole model.
"""
import random

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import get


def _model_grads(numels, rng, dt="bf16"):
    out = []
    for n in numels:
        x = rng.normal(0, 1e-2, n).astype(np.float32)
        out.append(synth.half_bits(x, dt))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_flatten_brute_force(seed):
    rng = np.random.default_rng(seed)
    pr = random.Random(seed)
    numels = [pr.choice([0, 1, 5, 16, 33, 100]) for _ in range(pr.randint(1, 8))]
    grads = _model_grads(numels, rng)
    R = pr.randint(1, 4)
    A = pr.choice([1, 8])
    for r in range(R):
        p = oracle.plan(numels, R, r, A)
        flat = oracle.flatten(p, grads)
        exp = np.full(p.S, 0xAAAA, np.uint16)
        x = 0
        for g in grads:
            for j in range(g.size):
                if p.begin <= x < p.begin + p.S:
                    exp[x - p.begin] = g[j]
                x += 1
        exp[p.real:] = 0
        assert np.array_equal(flat, exp)


@pytest.mark.parametrize("seed", range(6))
def test_flatten_brute_force_f32(seed):
    rng = np.random.default_rng(100 + seed)
    pr = random.Random(seed)
    numels = [pr.choice([0, 1, 5, 16, 33, 100]) for _ in range(pr.randint(1, 8))]
    grads = [rng.normal(0, 1e-2, n).astype(np.float32).view(np.uint32) for n in numels]
    R = pr.randint(1, 4)
    A = pr.choice([1, 8])
    for r in range(R):
        p = oracle.plan(numels, R, r, A)
        flat = oracle.flatten(p, grads)
        assert flat.dtype == np.uint32
        exp = np.full(p.S, 0xAAAAAAAA, np.uint32)
        x = 0
        for g in grads:
            for j in range(g.size):
                if p.begin <= x < p.begin + p.S:
                    exp[x - p.begin] = g[j]
                x += 1
        exp[p.real:] = 0
        assert np.array_equal(flat, exp)
        # a rank of padding only: zeros of the right width with no arrays to tell it
        pad = oracle.plan(numels, R, r, A)
        if pad.real == 0:
            assert np.array_equal(oracle.flatten(pad, [None] * len(numels), "f32"),
                                  np.zeros(pad.S, np.uint32))


def test_scale_trajectory_of_the_tiny_workload():
    # iterations 1..10, an overflow at iteration 4: the scale halves once and
    # the step counter skips it
    s = oracle.Scaler(1024.0, dynamic=True)
    scales, ts, t = [], [], 0
    for it in range(1, 11):
        scales.append(s.value)
        ovf = 1 if it == 4 else 0
        if not ovf:
            t += 1
            ts.append(t)
        else:
            ts.append(None)
        s.update(ovf)
    assert scales == [1024.0] * 4 + [512.0] * 6
    assert ts == [1, 2, 3, None, 4, 5, 6, 7, 8, 9]


def test_scale_growth_backoff_and_floor():
    s = oracle.Scaler(8.0, dynamic=True, window=2)
    seq = [(0, 8.0), (0, 16.0), (1, 8.0), (0, 8.0), (1, 4.0), (0, 4.0), (0, 8.0)]
    for ovf, after in seq:
        s.update(ovf)
        assert s.value == after
    s = oracle.Scaler(2.0, dynamic=True, min_scale=1.0)
    for _ in range(3):
        s.update(1)
    assert s.value == 1.0
    st = oracle.Scaler(1.0, dynamic=False, window=1)
    for ovf in (1, 0, 0, 1):
        st.update(ovf)
        assert st.value == 1.0
    # growth restarts the clean-step count: with a window of 2, six clean
    # steps double the scale after the 2nd, 4th and 6th, not after every step
    # from the 2nd on
    s = oracle.Scaler(8.0, dynamic=True, window=2)
    trail = []
    for _ in range(6):
        s.update(0)
        trail.append((s.value, s.good.value))
    assert trail == [(8.0, 1), (16.0, 0), (16.0, 1), (32.0, 0), (32.0, 1), (64.0, 0)]


def test_dna_scale_trajectory_halves_per_injection():
    w = get("dna_20b")
    s = oracle.Scaler(w.init_scale, dynamic=True)
    n_before = 0
    real = 2_498_481_408
    for it in range(1, w.steps + 1):
        assert s.value == w.init_scale * 2.0 ** -n_before
        hit = synth.inject(w.seed, it, real, w.inject_p) is not None
        s.update(1 if hit else 0)
        n_before += hit
    assert 1 <= n_before <= 15


def _run_partitioned(numels, R, grads_per_step, pdt, gdt, scale, steps, A=8):
    P = sum(numels)
    param = np.zeros(P, np.uint16)
    masters = []
    full_master = np.random.default_rng(1000).normal(0, 0.02, P).astype(np.float32)
    for r in range(R):
        p = oracle.plan(numels, R, r, A)
        master = np.zeros(p.S, np.float32)
        master[:p.real] = full_master[p.begin:p.begin + p.real]
        m = np.zeros(p.S, np.float32)
        v = np.zeros(p.S, np.float32)
        for t in range(1, steps + 1):
            flat = oracle.flatten(p, grads_per_step[t - 1])
            assert oracle.adam_step(t, scale, flat, gdt, master, m, v) == 0
        oracle.write_param(master, p.real, p.begin, 0, param, pdt)
        masters.append(master[:p.real])
    return param, np.concatenate(masters)


@pytest.mark.parametrize("R", [2, 3, 4])
def test_partitioned_step_equals_unpartitioned(R):
    # ZeRO is data parallelism without the redundancy: the assembled shards
    # must equal the single-rank step over the whole model, bit for bit
    w = get("tiny")
    numels = w.numels
    rng = np.random.default_rng(5)
    steps = 3
    grads = [_model_grads(numels, rng, "f16") for _ in range(steps)]
    part_param, part_master = _run_partitioned(numels, R, grads, "f16", "f16", 1.0, steps)
    full_param, full_master = _run_partitioned(numels, 1, grads, "f16", "f16", 1.0, steps)
    assert np.array_equal(part_param, full_param)
    assert np.array_equal(part_master.view(np.uint32), full_master.view(np.uint32))
    assert part_master.size == sum(numels)


def test_partitioned_gpt2_small_equals_unpartitioned():
    # the same invariant at GPT-2-small's 148 tensors over 8 ranks (A = 64,
    # bf16): rank 0's shard lies inside the token embedding, the others cut
    # through the layers.  One step (the tiny case above takes three): the
    # invariant is about where each element lives, not about t.
    w = get("gpt2_small")
    rng = np.random.default_rng(6)
    steps = 1
    grads = [_model_grads(w.numels, rng, "bf16") for _ in range(steps)]
    part_param, part_master = _run_partitioned(w.numels, 8, grads, "bf16", "bf16", 1.0, steps,
                                               A=64)
    full_param, full_master = _run_partitioned(w.numels, 1, grads, "bf16", "bf16", 1.0, steps,
                                               A=64)
    assert part_master.size == sum(w.numels) == 124_439_808
    assert np.array_equal(part_param, full_param)
    assert np.array_equal(part_master.view(np.uint32), full_master.view(np.uint32))


@pytest.mark.parametrize("pdt", ["f16", "bf16"])
def test_write_param_casts_like_the_library_conversion(pdt):
    # the written parameters are the IEEE round-to-nearest-even cast of the
    # master (numpy float16 / torch bfloat16), in the parameter dtype asked for
    import torch
    rng = np.random.default_rng(11)
    master = np.concatenate([rng.normal(0, 0.02, 3000), rng.normal(0, 300.0, 1000),
                             rng.normal(0, 1e-6, 1000)]).astype(np.float32)
    param = np.zeros(master.size, np.uint16)
    oracle.write_param(master, master.size, 0, 0, param, pdt)
    if pdt == "f16":
        want = master.astype(np.float16).view(np.uint16)
    else:
        want = torch.from_numpy(master).to(torch.bfloat16).view(torch.int16).numpy().view(
            np.uint16)
    assert np.array_equal(param, want)


def test_write_param_lands_at_offset_and_skips_padding():
    master = np.array([0.5, -1.25, 3.0, 7.0], np.float32)
    param = np.full(10, 0xBEEF, np.uint16)
    oracle.write_param(master, 3, 6, 2, param, "bf16")   # flat [6, 9) into a window from 2
    assert param[4:7].tolist() == [0x3F00, 0xBFA0, 0x4040]
    assert param[:4].tolist() == [0xBEEF] * 4 and param[7:].tolist() == [0xBEEF] * 3
