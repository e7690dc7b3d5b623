"""GPU vs oracle parity over whole shards on seeded random configurations.

Each seed draws a model (1-16 tensors, sizes from a list that includes 0,
1, tile edges and large primes), a data-parallel degree and rank, an
alignment, a bucket size, gradient and parameter dtypes, Adam-L2 or AdamW, a
weight decay, a flatten mode (all buckets, one bucket at a time in order or
shuffled, or a buffer filled elsewhere that the step must scan), a parameter
mode (the full buffer, a window, none), a static or dynamic loss scale and,
for half the seeds, overflows injected with probability 0.3 per step.  A
quarter of the seeds run the asynchronous (device-resident) step.  The bar
is the other parity tests': identical flags, scale and applied-step count,
and bit-identical flat shard, master, moments and parameters.
"""
import random

import pytest

from harness import Case, compare_full, log

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 2, 7, 8, 63, 64, 65, 1000, 4095, 4096, 4097, 30011, 100003, 262147]


def random_case(seed):
    rnd = random.Random(seed)
    numels = [rnd.choice(SIZES) for _ in range(rnd.randint(1, 16))]
    R = rnd.randint(1, 8)
    gdt = rnd.choice(["f16", "bf16", "f32"])
    dynamic = gdt == "f16" or rnd.random() < 0.25
    return Case(numels=numels, world_size=R, rank=rnd.randrange(R), grad_dtype=gdt,
                param_dtype=rnd.choice(["f16", "bf16"]), steps=rnd.randint(2, 4),
                align=rnd.choice([1, 2, 8, 64, 128]),
                bucket_elems=rnd.choice([1, 100, 5000, 1 << 25]), grad_sigma=1e-2,
                dynamic=dynamic, init_scale=1024.0 if dynamic else 1.0, window=2,
                inject_p=0.3 if rnd.random() < 0.5 else 0.0, adamw=rnd.random() < 0.7,
                weight_decay=rnd.choice([0.0, 0.01, 0.1]), seed=seed,
                flatten_mode=rnd.choice(["all", "buckets", "buckets_shuffled", "scan"]),
                param_mode=rnd.choice(["full", "window", "none"]))


@pytest.mark.parametrize("seed", range(200))
def test_random_configuration(seed):
    case = random_case(seed)
    mode = "async" if seed % 4 == 3 else "sync"
    label = f"random seed={seed}"
    log(f"[random] {label}: numels={case.numels} R={case.world_size} r={case.rank} "
        f"A={case.align} B={case.bucket_elems} grads={case.grad_dtype} "
        f"params={case.param_dtype} adamw={case.adamw} wd={case.weight_decay} "
        f"dynamic={case.dynamic} inject_p={case.inject_p} flatten={case.flatten_mode} "
        f"param={case.param_mode} steps={case.steps} mode={mode}")
    worst = compare_full(case, label=label, mode=mode)
    assert worst["bit_exact"], worst
