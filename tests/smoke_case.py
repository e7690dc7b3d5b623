"""One small invocation of the hot path on cuda:0, checked against the oracle:
the tiny workload (3 tensors, R=4 rank 1, fp16 grads, dynamic loss scale),
10 steps with +inf injected at step 4 (skipped step, scale halved)."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
for p in (HERE, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)


def run_smoke() -> None:
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU (cuda:0)")
    from harness import Case, compare_full, log
    from synth.workloads import get
    case = Case.from_workload(get("tiny"), inject={4: 2624 // 2})
    worst = compare_full(case, label="smoke")
    assert worst["skipped"] == 1, worst
    log(f"smoke ok: {worst}")


if __name__ == "__main__":
    run_smoke()
