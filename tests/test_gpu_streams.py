"""Plans are independent: two ranks of one model step concurrently on two HIP
streams (asynchronous step, each plan with its own device flag and state)
and write their parameter slices into ONE shared full parameter buffer.
Each rank is compared with its own oracle run after every iteration; an
overflow injected into rank 0 only must skip rank 0 only."""
import numpy as np
import pytest

import zero_partitioned_mixed_plan_amd as z
from harness import Case, OracleRun, compare_state, init_master_host, init_param_host, log, \
    torch_dtype

pytestmark = pytest.mark.gpu

RAGGED = [3000, 1, 7, 100003, 65, 2048, 511, 300000, 13, 0, 4099, 77777]


class _Rank:
    """Device state of one rank, on its own stream (param buffer shared)."""

    def __init__(self, case, param_full, stream):
        import torch
        self.case, self.stream = case, stream
        self.dev = torch.device("cuda:0")
        self.plan = z.zero_partition_plan(case.numels, case.world_size, case.rank, case.align,
                                          case.bucket_elems)
        p = self.plan
        self.hp = z.AdamHParams(case.lr, case.beta1, case.beta2, case.eps, case.weight_decay,
                                case.adamw)
        self.master = torch.from_numpy(init_master_host(case, p.begin, p.real, p.S)).to(self.dev)
        self.m = torch.zeros(p.S, dtype=torch.float32, device=self.dev)
        self.v = torch.zeros(p.S, dtype=torch.float32, device=self.dev)
        self.flat = torch.empty(p.S, dtype=torch_dtype(case.grad_dtype), device=self.dev)
        self.param_full = param_full
        self.scaler = z.LossScaler(case.init_scale, dynamic=case.dynamic, window=case.window)
        z.zero_state_upload(p, 0, self.scaler, stream=stream)
        self.mode = "async"

    def enqueue(self, grads_host):
        import torch
        gdt = torch_dtype(self.case.grad_dtype)
        with torch.cuda.stream(self.stream):
            grads = [None if g is None else
                     torch.from_numpy(g.view(np.int16)).to(self.dev, non_blocking=False).view(gdt)
                     for g in grads_host]
            z.zero_flatten_grads(self.plan, -1, grads, self.flat)
            z.zero_adam_step_async(self.plan, self.hp, self.flat, self.master, self.m, self.v,
                                   self.param_full, 0)
        self._keep = grads          # alive until the stream has consumed them

    def state_host(self):
        import torch
        torch.cuda.synchronize()
        return (self.master.cpu().numpy(), self.m.cpu().numpy(), self.v.cpu().numpy(),
                self.param_full.view(torch.int16).cpu().numpy().view(np.uint16),
                self.flat.view(torch.int16).cpu().numpy().view(np.uint16))


def test_two_ranks_concurrently_on_two_streams():
    import torch
    # param_mode "none": compare_state skips parameters; the shared buffer is
    # checked below against both ranks' oracle slices
    cases = [Case(numels=RAGGED, world_size=2, rank=r, grad_dtype="f16", param_dtype="f16",
                  steps=6, dynamic=True, init_scale=1024.0, window=3, param_mode="none",
                  inject={3: 100} if r == 0 else {}) for r in range(2)]
    orcs = [OracleRun(c) for c in cases]
    P = sum(RAGGED)
    param_full = torch.from_numpy(init_param_host(cases[0], P).view(np.int16)).to("cuda:0").view(
        torch.float16)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ranks = [_Rank(c, param_full, s) for c, s in zip(cases, streams)]
    worst = [dict(master=0.0, m=0.0, v=0.0, param_ulp=0, bit_exact=True, skipped=0)
             for _ in range(2)]
    for it in range(1, 7):
        steps = [orc.step(it) for orc in orcs]
        for rank, (_, grads, _) in zip(ranks, steps):
            rank.enqueue(grads)
        torch.cuda.synchronize()
        for r in range(2):
            st = z.zero_state_download(ranks[r].plan, stream=streams[r])
            assert st.last_flag == steps[r][0], (it, r)
            assert st.applied_steps == orcs[r].t and st.scale == orcs[r].scaler.value, (it, r)
            worst[r]["skipped"] += steps[r][0]
        for r in range(2):
            compare_state(ranks[r], orcs[r], worst[r], f"rank {r} it={it}")
        # the shared parameter buffer holds both ranks' slices
        merged = orcs[0].params().copy()
        b1 = orcs[1].plan.begin
        merged[b1:] = orcs[1].params()[b1:]
        got = ranks[0].state_host()[3]
        assert np.array_equal(got, merged), f"it={it}: shared parameter buffer differs"
    log(f"[streams] {worst}")
    assert worst[0]["skipped"] == 1 and worst[1]["skipped"] == 0
    assert worst[0]["bit_exact"] and worst[1]["bit_exact"]
