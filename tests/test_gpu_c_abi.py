"""The C ABI without Python: tests/c_abi_check (C++, hipMalloc'ed buffers,
built by __graft_entry__.build()) runs five cases through include/zero_mi355x.h
-- three through zero_adam_step, two through zero_adam_step_noalloc -- and
compares every step with the C oracle bit for bit, then compares the update
scalars zero_adam_scalars forms on the device with the host's, then runs the
ZeRO-Offload pipeline three times (lag 1 and 0; fp16, bf16 and fp32
gradients) through its calls alone, timeline included (see its header)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_program_matches_the_oracle():
    assert os.path.exists(BIN), "tests/c_abi_check is not built (python __graft_entry__.py)"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0 and "c-abi ok" in r.stdout, r.stdout + r.stderr
    assert r.stdout.count("(allocation-free step)") == 2 and "device = host" in r.stdout
