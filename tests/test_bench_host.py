"""bench.py's host-side bookkeeping, on the CPU: the algorithmic byte counts
it prices the kernels at, the kernel-source digest that gates the counted
HBM traffic, the pricing of raw memory-request counts, and that the
committed counter summaries were taken with the kernel source as it stands
(so a GPU run reports `traffic` rather than null), the offload timeline's
summary, and the host streaming rate the host update is priced against."""
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
    changed.write_text(src.replace("kAdamSpan = 256", "kAdamSpan = 512", 1))
    assert "kAdamSpan = 256" in src
    assert bench.kernels_digest(str(changed)) != base


def test_counter_summaries_match_the_kernel_source():
    # the committed raw request counts are for this kernel source; priced at
    # the request sizes (128-byte read lines, 64-byte writes) they give the
    # update's 28 B x S on every large workload and the flatten's 4 B x S
    # (its write requests run up to ~0.05% over 2 B x S in some launches;
    # the 20B shard's misaligned pieces re-read ~0.09% of their lines)
    for name, flat_tol in (("llama2_70b", 1e-3), ("llama3_8b", 1e-3), ("dna_20b", 2e-3)):
        w = get(name)
        plan = z.zero_partition_plan(w.numels, w.world_size, w.rank, w.align, w.bucket_elems)
        adam = bench.counted_traffic(name, w.grad_dtype)
        assert adam is not None, f"{name}: kernels.hip changed since profiles/ counters were taken"
        assert abs(adam / (bench.adam_bytes(w.grad_dtype) * plan.S) - 1) < 1e-5, name
        flat = bench.counted_traffic(name, w.grad_dtype, "flatten")
        assert 0 <= flat / (bench.flatten_bytes(w.grad_dtype) * plan.S) - 1 < flat_tol, name
    assert bench.counted_traffic("llama2_70b", "f32") is None
    assert bench.counted_traffic("gpt2_small", "bf16") is None


def test_request_bytes():
    # reads priced at a 128-byte line (32 for 32-byte requests), writes at 64
    # (32 for the rest): a 4 GiB copy's counts give its 4 GiB each way
    assert bench.request_bytes(1 << 25, 0, 1 << 26, 1 << 26) == 2 * (4 << 30)
    assert bench.request_bytes(10, 4, 10, 6) == 6 * 128 + 4 * 32 + 6 * 64 + 4 * 32


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


def test_timeline_summary_by_hand():
    # two steps of two pieces: gradient copies [0,2) [2,4), updates [2,5)
    # [5,8), parameter copies [5,6) [8,9); the second step 10 ms later.
    # Copying 4 + 2 ms, updating 6 ms; the second gradient piece (2 ms) and
    # the first parameter piece (1 ms) run during the update; span 9 ms.
    tl = []
    for j, t in ((0, 0.0), (1, 10.0)):
        for kind, ivs in (("gradient copy", [(0, 2), (2, 4)]), ("host update", [(2, 5), (5, 8)]),
                          ("parameter copy", [(5, 6), (8, 9)])):
            for c, (a, b) in enumerate(ivs):
                tl.append({"step": j, "piece": c, "kind": kind, "start_ms": a + t,
                           "end_ms": b + t})
    s = bench.timeline_summary(tl)
    assert s == {"gradient_copy_ms": 4.0, "host_update_ms": 6.0, "parameter_copy_ms": 2.0,
                 "copies_during_update_ms": 3.0, "span_ms": 9.0, "pieces": 2, "steps": 1}
    assert bench._overlap([(0, 3), (5, 9)], [(2, 6), (8, 10)]) == 1 + 1 + 1
    assert bench._length([(0, 2), (1, 3), (5, 6)]) == 4


def test_host_stream_ceiling_counts_a_read_and_a_write_per_byte():
    nbytes = (32 << 20) + 12
    r = bench.host_stream_ceiling(nbytes, 3, reps=2)
    assert r["bytes"] == nbytes // 4 // 3 * 3 * 4 == 33_554_436   # whole floats, split evenly
    assert r["ms"] > 0
    assert abs(r["gbps"] - 2 * r["bytes"] / (r["ms"] * 1e-3) / 1e9) < 1e-9 * r["gbps"]
    assert "3 threads" in r["what"] and "2 passes" in r["what"]
