"""bench.py's host-side bookkeeping, on the CPU: the algorithmic byte counts
it prices the kernels at, the kernel-source digest that gates the counted
HBM traffic, and that the committed counter summaries were taken with the
kernel source as it stands (so a GPU run reports `traffic` rather than
null)."""
import os
import re
import subprocess
import sys

import bench
import zero_partitioned_mixed_plan_amd as z
from synth.workloads import get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_algorithmic_bytes_per_element():
    # update: read the gradient and 3 fp32 state words, write the 3 state
    # words and one half parameter; flatten: read and write the gradient
    for gdt, g in (("f16", 2), ("bf16", 2), ("f32", 4)):
        assert bench.adam_bytes(gdt) == g + 3 * 4 + 3 * 4 + 2
        assert bench.flatten_bytes(gdt) == 2 * g
    assert bench.adam_bytes("bf16") == 28


def test_digest_ignores_comments_and_blank_lines(tmp_path):
    src = open(bench.KERNELS_SRC).read()
    base = bench.kernels_digest()
    commented = tmp_path / "a.hip"
    commented.write_text("// a new comment\n\n" + src.replace("\n", "  // trailing note\n", 3))
    assert bench.kernels_digest(str(commented)) == base
    changed = tmp_path / "b.hip"
    changed.write_text(src.replace("kAdamThreads = 128", "kAdamThreads = 256", 1))
    assert "kAdamThreads = 128" in src
    assert bench.kernels_digest(str(changed)) != base


def test_counter_summary_matches_the_kernel_source():
    # the committed FETCH_SIZE / WRITE_SIZE summary is for this kernel source
    # and the default workload, and its bytes are the update's 28 B x S
    traffic = bench.counted_traffic("llama2_70b", "bf16")
    assert traffic is not None, "kernels.hip changed since profiles/ counters were taken"
    w = get("llama2_70b")
    plan = z.zero_partition_plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
    alg = bench.adam_bytes("bf16") * plan.S
    assert abs(traffic / alg - 1) < 1e-3
    assert bench.counted_traffic("llama3_8b", "bf16") is None
    assert bench.counted_traffic("llama2_70b", "f32") is None


def test_every_profile_names_the_current_kernel_source():
    digest = bench.kernels_digest()
    named = 0
    for name in sorted(os.listdir(PROFILES)):
        text = open(os.path.join(PROFILES, name)).read()
        for h in re.findall(r"SHA-256 ([0-9a-f]{16,64})", text):
            assert digest.startswith(h), f"{name} was taken with another kernel source"
            named += 1
    assert named >= 5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
