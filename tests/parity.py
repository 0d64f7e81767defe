"""Tolerances of the GPU path against the float64 oracle.

float32 storage: per tensor, max|gpu - ref| / max|ref| <= 1e-5.

bfloat16 storage (float32 arithmetic): the outputs are rounded to bfloat16, whose half-ulp
alone exceeds 1e-2 once |ref| >= 4. The reading used: the computation must be within 1e-2 of
the exact value and the final rounding to bfloat16 may add at most half an ulp of the exact
value, so |gpu - ref| <= 1e-2 + half_ulp_bf16(ref). A second, stronger check: the GPU's bf16
value is the exact value rounded to bf16, give or take one bf16 ulp (or within 1e-5 of it, for
values that are float32 noise around an exact zero).
"""

import numpy as np
import torch

F32_RTOL = 1e-5
BF16_ATOL = 1e-2
ABS_FLOOR = 1e-5     # below this, a bf16 value and the rounded exact value count as equal


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


def check_bf16(gpu, ref, atol: float = BF16_ATOL, what: str = ""):
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = atol + 0.5 * bf16_ulp(r)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (f"{what}: |gpu - ref| = {err.flat[worst]:.4e} at ref = {r.flat[worst]:.4f} "
                                  f"exceeds {bound.flat[worst]:.4e}")
    rounded = torch.from_numpy(r).to(torch.float32).to(torch.bfloat16).double().numpy()
    diff = np.abs(g - rounded)
    off = diff > ABS_FLOOR               # near exact zeros both sides hold float32 noise
    ulps = diff / bf16_ulp(np.maximum(np.abs(g), np.abs(rounded)))
    assert np.all(ulps[off] <= 1.0 + 1e-9), f"{what}: {np.max(ulps[off])} bf16 ulps from the rounded exact value"
    # fraction of elements one ulp off: reported, not asserted (sums of a few bf16 values often
    # sit exactly on a rounding tie, which any float32 perturbation breaks one way or the other)
    frac = np.mean(off)
    return float(np.max(err)), float(frac)


def check(gpu, ref, dtype: torch.dtype, what: str = ""):
    if dtype == torch.float32:
        return check_f32(gpu, ref, what=what)
    return check_bf16(gpu, ref, what=what)
