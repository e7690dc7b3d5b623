"""The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer
and under ThreadSanitizer (CPU only).

tests/sanitize_check.cpp drives the planner (every rank of every workload,
and 300 random small plans with zero-size tensors), the ABI's argument
checks, the loss-scale policy and the host update (ragged sizes, padding
ranks, fp16 / bf16, Adam-L2 / AdamW, injected NaN) against the C oracle, bit
for bit.  It is built with g++ from the library's host sources, the kernel
launchers replaced by stand-ins (tests/host_only_stubs.cpp), so nothing
here needs or touches a GPU.  Any out-of-bounds access, use after free,
leak, signed overflow, misaligned access or other undefined behaviour
aborts the AddressSanitizer + UBSan build; a data race between the host
update's threads aborts the ThreadSanitizer build.  Each runs once per
instruction-set path.
"""
import os
import shutil
import subprocess

import pytest

from synth.workloads import WORKLOADS, get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_plan_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("plan.cpp", "abi.cpp", "cpu_adam.cpp",
                                                "offload.cpp")]


SANITIZERS = {
    # -D_GLIBCXX_SANITIZE_VECTOR: std::vector annotations, so a write past
    # size() but inside capacity() is reported too
    "asan+ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-D_GLIBCXX_SANITIZE_VECTOR"],
    "tsan": ["-fsanitize=thread"],
}
RUNTIME_MARKERS = {"asan+ubsan": ("__asan_report", "__ubsan_handle"), "tsan": ("__tsan_",)}
RUN_ENV = {
    "asan+ubsan": {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1",
                   "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"},
    "tsan": {"TSAN_OPTIONS": "halt_on_error=1"},
}


@pytest.fixture(scope="module")
def workload_file(tmp_path_factory):
    path = tmp_path_factory.mktemp("workloads") / "workloads.txt"
    with open(path, "w") as f:
        for name in WORKLOADS:
            w = get(name)
            f.write(f"{name} {w.world_size} {w.align} {w.bucket_elems} {len(w.numels)} "
                    + " ".join(str(n) for n in w.numels) + "\n")
    return str(path)


_built = {}


def _build(kind, tmp_path_factory):
    if kind in _built:
        return _built[kind]
    if shutil.which("g++") is None or not os.path.exists(
            os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path_factory.mktemp("sanitize") / f"sanitize_check_{kind.replace('+', '_')}")
    # host code only: g++, no .hip source on this line
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *SANITIZERS[kind],
           "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *HOST_SOURCES, os.path.join(ROOT, "tests", "host_only_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize_check.cpp"),
           "-x", "c", os.path.join(ROOT, "oracle", "zero_oracle.c"), "-x", "none",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-lpthread", "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert all(m in syms for m in RUNTIME_MARKERS[kind]), f"{kind} runtime not linked in"
    _built[kind] = exe
    return exe


@pytest.mark.parametrize("kind", list(SANITIZERS))
@pytest.mark.parametrize("isa", ["avx512", "avx2", "scalar"])
def test_host_paths_clean_under_sanitizers(tmp_path_factory, workload_file, kind, isa):
    exe = _build(kind, tmp_path_factory)
    env = dict(os.environ, ZERO_CPU_ISA=isa, **RUN_ENV[kind])
    r = subprocess.run([exe, workload_file], capture_output=True, text=True, env=env,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "sanitize ok" in r.stdout, out[-2000:]
    got = r.stdout.strip().rsplit("isa ", 1)[-1]
    if got != isa:
        pytest.skip(f"this host has no {isa}")
