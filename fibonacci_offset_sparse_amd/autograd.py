"""torch.autograd wrapper over fibattn_fwd / fibattn_bwd.

Argument marshalling only, like the rest of the binding: the forward and backward passes, the
alpha of a learned layer and the chain factor d(alpha)/d(theta) are all computed by the library
(alpha = 0.5 + sigmoid(theta), §2 "Per-layer scalar" of "Depth-Staggered Fibonacci Spacing for
Sparse Attention"; d(theta) comes out of fibattn_bwd). Python only moves tensors and host scalars.

    o = fib_attention(q, k, v, W, offsets, alpha=0.8)          # static schedule
    o = fib_attention(q, k, v, W, offsets, theta=theta)        # learned: theta a 0-dim tensor

theta is read on the host (alpha selects the slot plan, which the library builds on the host), so a
theta on the GPU costs one device-to-host copy per call; its gradient comes back on theta's device.
The forward runs in a workspace large enough for the backward and keeps it for the backward, which
then skips its own key prep where the library reports the forward's is the same
(fibattn_bwd_reuses_fwd_prep).
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (BF16, F32, STAGE_ALL, STAGE_KEY, STAGE_QUERY, fibattn_alpha_from_theta,
               fibattn_bwd_reuses_fwd_prep, fibattn_bwd_stages, fibattn_bwd_workspace_bytes, fibattn_fwd,
               fibattn_fwd_workspace_bytes)


class FibAttnFn(torch.autograd.Function):
    """Autograd node of one sparse-attention call: inputs (q, k, v, theta or None), output o."""

    @staticmethod
    def forward(ctx, q, k, v, theta, alpha: Optional[float], W: int, offsets: Sequence[int], rope_theta: float):
        dadt = 0.0
        if theta is not None:
            alpha, dadt = fibattn_alpha_from_theta(float(theta.detach().to("cpu", torch.float64).item()))
        B, Hq, L, D = q.shape
        Hkv = k.shape[1]
        dt = BF16 if q.dtype == torch.bfloat16 else F32
        nbytes = max(fibattn_fwd_workspace_bytes(B, L, Hkv, D, dt),
                     fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, W, len(offsets), dt))
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        o, _ = fibattn_fwd(q, k, v, alpha, W, offsets, rope_theta=rope_theta, need_lse=False, workspace=ws)
        ctx.save_for_backward(q, k, v)
        ctx.ws, ctx.alpha, ctx.dadt, ctx.W, ctx.offsets, ctx.rope_theta = ws, alpha, dadt, W, tuple(offsets), rope_theta
        ctx.theta_device = theta.device if theta is not None else None
        ctx.theta_dtype = theta.dtype if theta is not None else None
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        do = do.contiguous()
        B, Hq, L, D = q.shape
        Hkv = k.shape[1]
        dt = BF16 if q.dtype == torch.bfloat16 else F32
        want_theta = ctx.needs_input_grad[3]
        stages = STAGE_ALL
        if fibattn_bwd_reuses_fwd_prep(ctx.alpha, ctx.W, ctx.offsets, B, L, Hq, Hkv, D, dt):
            stages = STAGE_QUERY | STAGE_KEY            # the forward's prep is in ctx.ws
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dth = torch.empty(1, dtype=torch.float32, device=q.device) if want_theta else None
        fibattn_bwd_stages(stages, q, k, v, do, ctx.alpha, ctx.W, ctx.offsets, dq, dk, dv, ctx.ws,
                           rope_theta=ctx.rope_theta, dalpha_dtheta=ctx.dadt, dtheta=dth)
        ctx.ws = None
        dtheta = dth.reshape(()).to(ctx.theta_device, ctx.theta_dtype) if want_theta else None
        return dq, dk, dv, dtheta, None, None, None, None


def fib_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, W: int, offsets: Sequence[int],
                  alpha: Optional[float] = None, theta: Optional[torch.Tensor] = None,
                  rope_theta: float = 1e4) -> torch.Tensor:
    """Sparse attention output o [B, Hq, L, D], differentiable in q, k, v and (learned layers) theta.

    Give exactly one of alpha (a static schedule's float) or theta (a 0-dim tensor; alpha =
    0.5 + sigmoid(theta)). d(theta) needs every rung interpolated at that alpha (the library returns
    UNSUPPORTED otherwise)."""
    if (alpha is None) == (theta is None):
        raise ValueError("give exactly one of alpha and theta")
    if theta is not None and theta.dim() != 0:
        raise ValueError("theta must be a 0-dim tensor")
    return FibAttnFn.apply(q, k, v, theta, alpha, int(W), tuple(int(f) for f in offsets), float(rope_theta))


__all__ = ["FibAttnFn", "fib_attention"]
