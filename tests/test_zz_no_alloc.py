"""zero_adam_step_noalloc against zero_adam_step, through the C ABI.

The allocation-free step keeps its overflow accumulator in the library's
device scratch array, shared by every call on the device and left holding
the last call's value.  Calls in a row must therefore each start from a
clear accumulator: a large clean step, then a smaller step with an inf
(skipped), then a smaller clean step.  Each call runs on a twin of the state
that zero_adam_step updates from the same inputs; flags, master, moments and
parameters must be identical bit for bit (and equal the oracle's).  The
call is also captured once into a HIP graph and replayed with new gradients
between replays, each replay checked the same way.
"""
import numpy as np
import pytest

import oracle
import synth
import zero_partitioned_mixed_plan_amd as z
from harness import to_device_grad, torch_dtype

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
INF = {"f16": 0x7C00, "bf16": 0x7F80, "f32": 0x7F800000}


def _bits(t):
    import torch
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Twin:
    """One shard's state twice on the device (a: zero_adam_step, b: the
    allocation-free step) and once on the host (the oracle)."""

    def __init__(self, numels, R, r, A, gdt, pdt, seed):
        import torch
        self.plan = z.zero_partition_plan(numels, R, r, A)
        self.op = oracle.plan(numels, R, r, A)
        self.gdt, self.pdt = gdt, pdt
        S, P = self.op.S, self.op.P
        rng = np.random.default_rng(seed)
        self.rng = rng
        m0 = np.zeros(S, np.float32)
        m0[:self.op.real] = rng.normal(0, 0.02, self.op.real).astype(np.float32)
        p0 = rng.integers(0, 1 << 15, P).astype(np.uint16)
        self.host = {"master": m0.copy(), "m": np.zeros(S, np.float32),
                     "v": np.zeros(S, np.float32), "param": p0.copy()}
        self.dev = []
        for _ in range(2):
            self.dev.append({
                "master": torch.from_numpy(m0.copy()).to(DEV),
                "m": torch.zeros(S, device=DEV), "v": torch.zeros(S, device=DEV),
                "param": torch.from_numpy(p0.view(np.int16).copy()).to(DEV).view(
                    torch_dtype(pdt))})
        self.flat = torch.empty(S, dtype=torch_dtype(gdt), device=DEV)
        self.out = torch.full((1,), -7, dtype=torch.int32, device=DEV)

    def grads(self, scale, inject):
        S, real = self.op.S, self.op.real
        bits = synth.grad_bits(self.rng.normal(0, 1e-2, S).astype(np.float32) * scale, self.gdt)
        bits[real:] = 0
        if inject is not None:
            bits[inject] = INF[self.gdt]
        self.flat.copy_(to_device_grad(bits, self.gdt, DEV))
        return bits

    def step_a(self, t, scale):
        d = self.dev[0]
        return z.zero_adam_step(self.plan, z.AdamHParams(), t, scale, self.flat, d["master"],
                                d["m"], d["v"], d["param"], 0)

    def step_b(self, t, scale):
        d = self.dev[1]
        z.zero_adam_step_noalloc(self.plan, z.AdamHParams(), t, scale, self.flat, d["master"],
                                 d["m"], d["v"], self.out, d["param"], 0)

    def oracle_step(self, t, scale, bits):
        h = self.host
        flag = oracle.adam_step(t, scale, bits, self.gdt, h["master"], h["m"], h["v"])
        if not flag:
            oracle.write_param(h["master"], self.op.real, self.op.begin, 0, h["param"], self.pdt)
        return flag

    def compare(self, label):
        for name in ("master", "m", "v", "param"):
            a, b = _bits(self.dev[0][name]), _bits(self.dev[1][name])
            assert np.array_equal(a, b), f"{label}: {name} differs from zero_adam_step's"
            h = self.host[name]
            assert np.array_equal(a, h.view(a.dtype)), f"{label}: {name} differs from the oracle"


def test_calls_in_a_row_match_zero_adam_step():
    import torch
    large = Twin([300000, 7, 123457, 64, 99999], 3, 2, 64, "bf16", "bf16", seed=11)
    small = Twin([1000, 37, 5], 4, 3, 64, "f16", "f16", seed=12)
    assert small.op.S < large.op.S and 0 < small.op.real < small.op.S
    for label, tw, t, scale, inject in (("large clean", large, 1, 1.0, None),
                                        ("small with inf", small, 1, 1024.0, small.op.real // 2),
                                        ("small clean", small, 1, 512.0, None),
                                        ("large clean again", large, 2, 1.0, None)):
        bits = tw.grads(scale, inject)
        fa = tw.step_a(t, scale)
        tw.step_b(t, scale)
        torch.cuda.synchronize()
        fb = int(tw.out.item())
        fo = tw.oracle_step(t, scale, bits)
        assert fa == fb == fo == (1 if inject is not None else 0), (label, fa, fb, fo)
        tw.compare(label)


def test_captured_in_a_graph_and_replayed():
    import torch
    tw = Twin([5000, 300, 17, 70000], 2, 1, 64, "bf16", "bf16", seed=13)
    bits = tw.grads(1.0, None)
    tw.step_b(1, 1.0)                       # first call outside the capture
    fa = tw.step_a(1, 1.0)
    torch.cuda.synchronize()
    assert fa == int(tw.out.item()) == tw.oracle_step(1, 1.0, bits) == 0
    tw.compare("eager step 1")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tw.step_b(2, 1.0)                   # recorded, not run
    torch.cuda.synchronize()
    tw.compare("after the capture")
    for it, inject in enumerate((None, tw.op.real - 1, None)):
        bits = tw.grads(1.0, inject)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        fb = int(tw.out.item())
        fa = tw.step_a(2, 1.0)
        fo = tw.oracle_step(2, 1.0, bits)
        assert fa == fb == fo == (1 if inject is not None else 0), (it, fa, fb, fo)
        tw.compare(f"replay {it}")
