"""Seeded synthetic inputs for the sparse-attention workloads.

This module only draws random tensors and names the workloads. It holds none of the attention
arithmetic: base offsets and alpha schedules are named by kind here and computed by each side on
its own (the HIP library and the float64 oracle).

The shapes follow the paper's models ("Depth-Staggered Fibonacci Spacing for Sparse Attention",
§3 "Models and training"): 16 layers, 8 query heads sharing 2 key-value heads, head dim 64,
sequence length 1024 and 32 768 tokens per step (B = 32), plus the 4x length extrapolation shape
(B = 8, L = 4096). The paper trains on text datasets that are not available here; i.i.d. N(0, 1)
activations of the same shapes stand in for the attention inputs.

Seeds: the tiny workload draws q, k, v from seed 0. Layer l of workload number c >= 2 draws q, k,
v (and the upstream gradient do for the learned workload) in that order from seed 100 c + l.
The learned workload's per-layer theta ~ N(0, 0.5^2) comes from its own generator, seed 0.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    number: int        # 1..5, fixes the seeds
    B: int
    L: int
    Hq: int
    Hkv: int
    D: int
    dtype: str         # "f32" or "bf16": storage type of q, k, v, o and the gradients
    W: int             # window: distances 0..W
    base: str          # "fib", or "pow2_<max>": the power-of-two control base up to <max>
    schedule: str      # "fixed", "linear", "coprime" or "learned"
    n_layers: int
    backward: bool

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def seed(self, layer: int) -> int:
        return 0 if self.number == 1 else 100 * self.number + layer


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fixed_f32", 1, 1, 64, 8, 2, 64, "f32", 6, "fib", "fixed", 1, True),
        Workload("l1024_linear_bf16", 2, 32, 1024, 8, 2, 64, "bf16", 12, "fib", "linear", 16, False),
        Workload("l4096_coprime_bf16", 3, 8, 4096, 8, 2, 64, "bf16", 12, "fib", "coprime", 16, False),
        Workload("l1024_pow2_fixed_bf16", 4, 32, 1024, 8, 2, 64, "bf16", 8, "pow2_1024", "fixed", 16,
                 False),
        Workload("l1024_pow2_linear_bf16", 4, 32, 1024, 8, 2, 64, "bf16", 8, "pow2_1024", "linear", 16,
                 False),
        Workload("l1024_learned_bf16", 5, 32, 1024, 8, 2, 64, "bf16", 10, "fib", "learned", 16, True),
        # long-L variants at the 4x extrapolation shape: a power-of-two base grown with L (rung
        # 2048), and the window sweep of the paper's run matrix (W = 12 is l4096_coprime_bf16)
        Workload("l4096_pow2_2048_linear_bf16", 6, 8, 4096, 8, 2, 64, "bf16", 8, "pow2_2048", "linear", 16,
                 False),
        Workload("l4096_w6_coprime_bf16", 7, 8, 4096, 8, 2, 64, "bf16", 6, "fib", "coprime", 16, False),
        Workload("l4096_w8_coprime_bf16", 8, 8, 4096, 8, 2, 64, "bf16", 8, "fib", "coprime", 16, False),
        Workload("l4096_w10_coprime_bf16", 9, 8, 4096, 8, 2, 64, "bf16", 10, "fib", "coprime", 16, False),
    ]
}


def pow2_max(w: Workload) -> int:
    """The largest rung of a power-of-two base workload (from its name), e.g. 1024 for "pow2_1024"."""
    return int(w.base.split("_")[1])


def draw(w: Workload, layer: int, B: Optional[int] = None, L: Optional[int] = None,
         with_grad: Optional[bool] = None):
    """q [B,Hq,L,D], k, v [B,Hkv,L,D] (and do [B,Hq,L,D]) on the CPU in the workload's dtype.

    N(0, 1) draws in float32, rounded to bfloat16 (round-to-nearest-even) for bf16 workloads.
    B and L may be reduced for small parity cases; the stream then starts the same way.
    """
    B = w.B if B is None else B
    L = w.L if L is None else L
    with_grad = w.backward if with_grad is None else with_grad
    g = torch.Generator(device="cpu").manual_seed(w.seed(layer))
    q = torch.randn(B, w.Hq, L, w.D, generator=g, dtype=torch.float32)
    k = torch.randn(B, w.Hkv, L, w.D, generator=g, dtype=torch.float32)
    v = torch.randn(B, w.Hkv, L, w.D, generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_grad:
        out.append(torch.randn(B, w.Hq, L, w.D, generator=g, dtype=torch.float32))
    return tuple(x.to(w.torch_dtype) for x in out)


def draw_theta(n_layers: int = 16, seed: int = 0) -> torch.Tensor:
    """Per-layer theta ~ N(0, 0.5^2) (float64) for the learned-alpha workload."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return 0.5 * torch.randn(n_layers, generator=g, dtype=torch.float64)


def randn_like_seeded(shape, seed: int, dtype=torch.float32) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)
