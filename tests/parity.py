"""Tolerances of the GPU path against the float64 oracle.

float32 storage (float32 arithmetic): per tensor, max|gpu - ref| / max|ref| <= 1e-5.

bfloat16 storage: every output (o, lse, dq, dk, dv) must be within 1e-2 of the exact value, plus
half a bfloat16 ulp of the exact value for tensors stored as bfloat16 (whose rounding alone
exceeds 1e-2 once |ref| >= 4): |gpu - ref| <= 1e-2 + half_ulp_bf16(ref). The forward kernel for
bf16 storage multiplies fp16-rounded operands (relative error <= 2^-11 each) with float32
accumulation, so the result is not the exact value rounded to bf16; the number of bf16 ulps
between the two is reported, not asserted.
"""

import numpy as np
import torch

F32_RTOL = 1e-5
BF16_ATOL = 1e-2
ABS_FLOOR = 1e-5     # below this, a value and the rounded exact value count as equal (reporting)


def to64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_f32(gpu, ref, rtol: float = F32_RTOL, what: str = ""):
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    scale = max(np.max(np.abs(r)), 1e-30)
    err = np.max(np.abs(g - r)) / scale
    assert err <= rtol, f"{what}: relative inf-norm error {err:.3e} > {rtol:.0e}"
    return err


def check_bf16(gpu, ref, atol: float = BF16_ATOL, what: str = "", stored_bf16: bool = True):
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = atol + (0.5 * bf16_ulp(r) if stored_bf16 else 0.0)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (f"{what}: |gpu - ref| = {err.flat[worst]:.4e} at ref = {r.flat[worst]:.4f} "
                                  f"exceeds {np.broadcast_to(bound, err.shape).flat[worst]:.4e}")
    rounded = torch.from_numpy(r).to(torch.float32).to(torch.bfloat16).double().numpy()
    diff = np.abs(g - rounded)
    ulps = np.where(diff > ABS_FLOOR, diff / bf16_ulp(np.maximum(np.abs(g), np.abs(rounded))), 0.0)
    return float(np.max(err)), float(np.max(ulps))


def check(gpu, ref, dtype: torch.dtype, what: str = "", stored_bf16: bool = True):
    """Tolerance of the storage type `dtype`; stored_bf16=False for float32 outputs (lse) of a
    bf16 call."""
    if dtype == torch.float32:
        return check_f32(gpu, ref, what=what)
    return check_bf16(gpu, ref, what=what, stored_bf16=stored_bf16)
