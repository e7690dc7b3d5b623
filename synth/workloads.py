"""Synthetic workloads: parameter-shape lists and the optimizer setting of each.

Shapes are row-major [out, in] and listed in flat (registration) order.  No
weights or data are involved: the gradient and master values are drawn by
the seeded generator of this package.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15


def _mix64(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def small_sizes(count: int, lo: int = 64, hi: int = 6144) -> List[int]:
    """size_j = lo + (first SplitMix64 output from state j) mod (hi - lo + 1)."""
    span = hi - lo + 1
    return [lo + _mix64(j + _GOLDEN) % span for j in range(count)]


@dataclass
class Workload:
    name: str
    description: str
    shapes: List[Tuple[int, ...]]
    world_size: int
    rank: int
    grad_dtype: str            # "f16" | "bf16" ("f32": gradients kept in fp32)
    param_dtype: str           # "f16" | "bf16"
    grad_sigma: float
    steps: int
    master_sigma: float = 0.02
    dynamic_scale: bool = False
    init_scale: float = 1.0
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    inject_p: float = 0.0                 # per-iteration Bernoulli +inf injection
    inject_fixed: Optional[Tuple[int, str]] = None   # (iteration, "mid") fixed injection
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    adamw: bool = True
    seed: int = 0
    align: int = 64
    bucket_elems: int = 1 << 25
    extra: dict = field(default_factory=dict)

    @property
    def numels(self) -> List[int]:
        out = []
        for s in self.shapes:
            n = 1
            for d in s:
                n *= d
            out.append(n)
        return out

    @property
    def total(self) -> int:
        return sum(self.numels)


def _tiny() -> Workload:
    return Workload(
        name="tiny",
        description="3 fp32 params [64,32],[32],[128,64] (10272 elems), R=4 rank 1, fp16 grads "
                    "N(0,1e-3) x loss scale 1024 (dynamic), AdamW, 10 steps, +inf at step 4",
        shapes=[(64, 32), (32,), (128, 64)],
        world_size=4, rank=1, grad_dtype="f16", param_dtype="f16", grad_sigma=1e-3,
        steps=10, dynamic_scale=True, init_scale=1024.0, inject_fixed=(4, "mid"))


def _gpt2_small() -> Workload:
    d, ffn, vocab, ctx, layers = 768, 3072, 50257, 1024, 12
    shapes: List[Tuple[int, ...]] = [(vocab, d), (ctx, d)]
    for _ in range(layers):
        shapes += [(d,), (d,), (d, 3 * d), (3 * d,), (d, d), (d,), (d,), (d,),
                   (d, ffn), (ffn,), (ffn, d), (d,)]
    shapes += [(d,), (d,)]
    return Workload(
        name="gpt2_small",
        description="GPT-2-small shaped params (12 layers, d=768, ffn 3072, vocab 50257, tied "
                    "head, 124,439,808 elems), R=8 rank 0, bf16 grads N(0,1e-2), AdamW 100 steps",
        shapes=shapes, world_size=8, rank=0, grad_dtype="bf16", param_dtype="bf16",
        grad_sigma=1e-2, steps=100)


def _llama(d, kv, ffn, vocab, layers):
    shapes: List[Tuple[int, ...]] = [(vocab, d)]
    for _ in range(layers):
        shapes += [(d,), (d, d), (kv, d), (kv, d), (d, d), (d,), (ffn, d), (ffn, d), (d, ffn)]
    shapes += [(d,), (vocab, d)]
    return shapes


def _llama3_8b() -> Workload:
    return Workload(
        name="llama3_8b",
        description="Llama-3-8B shaped params (32 layers, d=4096, ffn 14336, 8 kv heads x 128, "
                    "vocab 128256, untied head), R=8 rank 3, bf16 grads N(0,1e-3) with 1% x100 "
                    "outliers, AdamW 20 steps",
        shapes=_llama(4096, 1024, 14336, 128256, 32), world_size=8, rank=3,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=20,
        outlier_p=0.01, outlier_mult=100.0)


def _llama2_70b() -> Workload:
    return Workload(
        name="llama2_70b",
        description="Llama-2-70B shaped params (80 layers, d=8192, ffn 28672, 8 kv heads x 128, "
                    "vocab 32000, untied head), R=8 rank 7, bf16 grads N(0,1e-3), AdamW 5 steps",
        shapes=_llama(8192, 1024, 28672, 32000, 80), world_size=8, rank=7,
        grad_dtype="bf16", param_dtype="bf16", grad_sigma=1e-3, steps=5)


def _dna_20b() -> Workload:
    d, ffn, vocab, layers = 6144, 24576, 4096, 44
    tiny = small_sizes(2000)
    shapes: List[Tuple[int, ...]] = [(vocab, d)]
    t = 0
    for layer in range(layers):
        shapes += [(3 * d, d), (d, d), (ffn, d), (d, ffn)]
        count = 46 if layer < 20 else 45
        shapes += [(s,) for s in tiny[t:t + count]]
        t += count
    assert t == 2000
    shapes += [(vocab, d)]
    return Workload(
        name="dna_20b",
        description="20B DNA-LM shaped params (44 layers, d=6144, ffn 24576, vocab 4096, untied "
                    "head, plus 2000 small tensors of 64-6144 elems), R=8 rank 2, fp16 grads, "
                    "dynamic loss scale 65536, +inf injected with p=0.1 per step, 50 steps",
        shapes=shapes, world_size=8, rank=2, grad_dtype="f16", param_dtype="f16",
        grad_sigma=1e-3, steps=50, dynamic_scale=True, init_scale=65536.0, inject_p=0.1)


WORKLOADS = {
    "tiny": _tiny,
    "gpt2_small": _gpt2_small,
    "llama3_8b": _llama3_8b,
    "llama2_70b": _llama2_70b,
    "dna_20b": _dna_20b,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()
