"""Pins of the oracle's partition / bucket plan (CPU only).

Checked against: brute force over every element of small models, the tiling
invariants over every rank of every workload, and the byte accounting the
pages print (tests/golden/memory_accounting.txt).
"""
import os
import random

import numpy as np
import pytest

import oracle
from synth.workloads import WORKLOADS, get

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_accounting.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (s.strip() for s in line.split("="))
            vals[k] = float(v)
    return vals


def _brute_segments(numels, R, r, S):
    """Walk every element; group consecutive owned elements of one tensor."""
    begin, end = r * S, (r + 1) * S
    segs = []
    flat = 0
    for i, n in enumerate(numels):
        cur = None
        for j in range(n):
            x = flat + j
            if begin <= x < end:
                if cur is None:
                    cur = [i, j, x - begin, 0]
                cur[3] += 1
        if cur is not None:
            segs.append(tuple(cur))
        flat += n
    return segs


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_brute_force(seed):
    rng = random.Random(seed)
    n = rng.randint(0, 7)
    numels = [rng.choice([0, 1, 2, 3, 5, 8, 13, 40, 97]) for _ in range(n)]
    R = rng.randint(1, 5)
    A = rng.choice([1, 2, 3, 8])
    P = sum(numels)
    for r in range(R):
        p = oracle.plan(numels, R, r, A, bucket_elems=7)
        # padding: the smallest multiple of R*A not below P
        assert p.P == P and p.P_pad % (R * A) == 0 and p.P_pad >= P and p.P_pad - R * A < P or (
            P == 0 and p.P_pad == 0)
        assert p.S * R == p.P_pad and p.begin == r * p.S
        got = list(zip(p.seg_tensor.tolist(), p.seg_tensor_off.tolist(),
                       p.seg_shard_off.tolist(), p.seg_numel.tolist()))
        assert got == _brute_segments(numels, R, r, p.S)
        owned = sum(1 for x in range(P) if r * p.S <= x < (r + 1) * p.S)
        assert p.real == owned


def test_bucket_rule_by_hand():
    # last tensor first, whole tensors, close at >= B: {t3, t2} then {t1, t0}
    p = oracle.plan([5, 3, 7, 2], 1, 0, 1, bucket_elems=6)
    assert p.tensor_bucket.tolist() == [1, 1, 0, 0] and p.n_buckets == 2
    # an open bucket at the front stays a bucket of its own
    p = oracle.plan([1, 9, 2], 1, 0, 1, bucket_elems=5)
    assert p.tensor_bucket.tolist() == [1, 0, 0] and p.n_buckets == 2
    # B = 1 closes a bucket after every non-empty tensor; an empty tensor rides
    # along with the next one
    p = oracle.plan([4, 0, 4], 1, 0, 1, bucket_elems=1)
    assert p.tensor_bucket.tolist() == [1, 1, 0] and p.n_buckets == 2


@pytest.mark.parametrize("seed", range(20))
def test_bucket_invariants(seed):
    rng = random.Random(seed)
    numels = [rng.randint(0, 50) for _ in range(rng.randint(1, 30))]
    B = rng.randint(1, 120)
    p = oracle.plan(numels, 1, 0, 1, bucket_elems=B)
    tb = p.tensor_bucket.tolist()
    # buckets are contiguous descending runs starting at the last tensor
    assert tb[-1] == 0 and all(tb[i] >= tb[i + 1] >= tb[i] - 1 for i in range(len(tb) - 1))
    for b in range(p.n_buckets):
        members = [i for i, x in enumerate(tb) if x == b]
        size = sum(numels[i] for i in members)
        if b < p.n_buckets - 1:
            # closed buckets hold >= B, and would not without their last-added tensor
            assert size >= B and size - numels[min(members)] < B
        else:
            assert size >= B or min(members) == 0


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_shards_tile_the_flat_space(name):
    w = get(name)
    numels = w.numels
    offs = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    R = w.world_size
    covered = []
    total_real = 0
    for r in range(R):
        p = oracle.plan(numels, R, r, w.align, w.bucket_elems)
        assert p.begin == r * p.S and p.S * R == p.P_pad and p.P == w.total
        # segments are in shard order and tile [0, real) of the shard
        pos = 0
        for s in range(p.n_segments):
            assert p.seg_shard_off[s] == pos
            flat0 = offs[p.seg_tensor[s]] + p.seg_tensor_off[s]
            assert flat0 == p.begin + pos
            assert 0 < p.seg_numel[s] and p.seg_tensor_off[s] + p.seg_numel[s] <= numels[p.seg_tensor[s]]
            covered.append((int(flat0), int(p.seg_numel[s])))
            pos += int(p.seg_numel[s])
        assert pos == p.real
        total_real += p.real
    # every element of [0, P) exactly once, over all ranks
    covered.sort()
    x = 0
    for a, n in covered:
        assert a == x
        x += n
    assert x == w.total == total_real


def test_workload_shard_sizes():
    # shard sizes at A = 64
    expect = {"tiny": 2624, "gpt2_small": 15_555_008, "llama3_8b": 1_003_782_656,
              "llama2_70b": 8_622_081_024, "dna_20b": 2_498_481_408}
    nseg = {"tiny": 1, "gpt2_small": 1, "llama3_8b": 40, "llama2_70b": 86, "dna_20b": 300}
    for name, S in expect.items():
        w = get(name)
        p = oracle.plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
        assert p.S == S, name
        assert p.n_segments == nseg[name], name


def test_memory_accounting_matches_pages():
    g = _golden()
    per_param = g["param_bytes_fp16"] + g["grad_bytes_fp16"] + g["state_bytes_fp32"]
    assert per_param == 16
    assert g["optimizer_state_bytes_approx"] == g["state_bytes_fp32"]
    w = get("dna_20b")
    R = int(g["example_gpus"])
    p = oracle.plan(w.numels, R, w.rank, w.align, w.bucket_elems)
    # the workload is a 20B model: its total model state is ~320 GB ...
    assert abs(w.total / g["example_params"] - 1) < 0.01
    total_gb = per_param * p.P / 1e9
    assert abs(total_gb / g["example_total_GB_approx"] - 1) < 0.01
    # ... and stage 3 on 8 GPUs leaves ~40 GB per GPU
    assert abs(p.bytes_stage3 / 1e9 / g["example_stage3_per_gpu_GB_approx"] - 1) < 0.01
    assert p.bytes_stage3 == per_param * p.S
    # optimizer states: 12 B/param, divided by the data-parallel degree
    red = (g["state_bytes_fp32"] * p.P) / (g["state_bytes_fp32"] * p.S)
    assert abs(red / g["optimizer_state_reduction_at_8"] - 1) < 1e-6


def test_stage_bytes_from_the_pages_components():
    # per-rank model-state bytes built from the pages' per-parameter bytes
    # (half parameters, half gradients, fp32 master + momentum + variance)
    # and from what each stage partitions (stage 1 the optimizer states,
    # stage 2 also the gradients, stage 3 also the parameters); partitioned
    # parts are held for the S elements of the shard, replicated ones for P
    g = _golden()
    pb, gb, sb = (int(g["param_bytes_fp16"]), int(g["grad_bytes_fp16"]),
                  int(g["state_bytes_fp32"]))
    rng = np.random.default_rng(4)
    for _ in range(20):
        numels = rng.integers(0, 5000, int(rng.integers(1, 30))).tolist()
        R = int(rng.integers(1, 9))
        p = oracle.plan(numels, R, int(rng.integers(0, R)), int(rng.integers(1, 65)))
        assert p.bytes_stage1 == pb * p.P + gb * p.P + sb * p.S
        assert p.bytes_stage2 == pb * p.P + gb * p.S + sb * p.S
        assert p.bytes_stage3 == pb * p.S + gb * p.S + sb * p.S


def test_stage_factors_match_pages():
    g = _golden()
    numels = [1 << 30] * 8
    for R in (1, 2, 8, 64):
        p = oracle.plan(numels, R, 0, 64)
        full = 16 * p.P
        # stage 3 reduces by the GPU count
        assert full / p.bytes_stage3 == pytest.approx(R * g["stage3_reduction_is_gpu_count"],
                                                      rel=1e-6)
    # the "up to" factors of stages 1 and 2 are the limits for many GPUs
    p = oracle.plan(numels, 1 << 20, 0, 1)
    assert 16 * p.P / p.bytes_stage1 == pytest.approx(g["stage1_reduction_up_to"], rel=1e-4)
    assert 16 * p.P / p.bytes_stage2 == pytest.approx(g["stage2_reduction_up_to"], rel=1e-4)
    # and are smaller at finite R
    p = oracle.plan(numels, 8, 0, 64)
    assert 16 * p.P / p.bytes_stage1 < 4 and 16 * p.P / p.bytes_stage2 < 8


def test_invalid_plans_rejected():
    for args in [([4], 0, 0, 1), ([4], 2, 2, 1), ([4], 2, -1, 1), ([4], 1, 0, 0), ([-1], 1, 0, 1)]:
        with pytest.raises(ValueError):
            oracle.plan(*args)


def test_rank_past_the_end_has_only_padding():
    p = oracle.plan([3], 4, 3, 1)      # P=3 < R=4: rank 3 owns nothing real
    assert p.S == 1 and p.real == 0 and p.n_segments == 0
    p = oracle.plan([], 2, 1, 8)       # empty model
    assert p.P == 0 and p.S == 0 and p.real == 0
