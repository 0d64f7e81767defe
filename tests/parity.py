"""Tolerances of the GPU path against the float64 oracle.

float32 storage (float32 arithmetic): per tensor, max|gpu - ref| / max|ref| <= 1e-5.

bfloat16 storage: every output is within 1e-2 of the exact value (the oracle on the same bf16
inputs upcast exactly). A bf16 value rounds with at most half a bf16 ulp, 2^-9 |ref|, which stays
below 1e-2 for |ref| < 4 (7.8e-3 at the top of [2, 4)): there the bare 1e-2 is asserted. From
|ref| = 4 on, rounding alone can exceed 1e-2 (half an ulp is 1.56e-2 in [4, 8)), so no bf16 output
could meet a bare 1e-2; there the bound is 1e-2 plus half a bf16 ulp of ref. Float32 outputs of a
bf16 call (lse) take the bare 1e-2 at every magnitude.

Each check also reports the largest error per |ref| band ([0,1), [1,2), [2,4), [4,inf)) and the
largest distance, in bf16 ulps, between the GPU value and the correctly rounded exact value.
"""

import numpy as np
import torch

F32_RTOL = 1e-5
BF16_ATOL = 1e-2
BARE_BELOW = 4.0     # |ref| under which the bare 1e-2 holds for bf16-stored outputs
ABS_FLOOR = 1e-5     # below this, a value and the rounded exact value count as equal (ulp report)
BANDS = ((0.0, 1.0), (1.0, 2.0), (2.0, 4.0), (4.0, np.inf))


def to64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def bf16_bound(ref: np.ndarray, atol: float = BF16_ATOL, stored_bf16: bool = True) -> np.ndarray:
    """The bf16 bar per element: atol where |ref| < 4 (or for float32 outputs), else atol plus half
    a bf16 ulp of ref."""
    if not stored_bf16:
        return np.full(ref.shape, atol)
    return np.where(np.abs(ref) < BARE_BELOW, atol, atol + 0.5 * bf16_ulp(ref))


def band_errors(err: np.ndarray, ref: np.ndarray) -> dict:
    """Largest |gpu - ref| in each |ref| band (bands with no element are left out)."""
    a = np.abs(ref)
    out = {}
    for lo, hi in BANDS:
        m = (a >= lo) & (a < hi)
        if m.any():
            out[f"[{lo:g},{hi:g})"] = float(err[m].max())
    return out


def check_f32(gpu, ref, rtol: float = F32_RTOL, what: str = ""):
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    scale = max(np.max(np.abs(r)), 1e-30)
    err = np.max(np.abs(g - r)) / scale
    assert err <= rtol, f"{what}: relative inf-norm error {err:.3e} > {rtol:.0e}"
    return err


def check_bf16(gpu, ref, atol: float = BF16_ATOL, what: str = "", stored_bf16: bool = True):
    """Asserts the bf16 bar; returns (max error, max bf16 ulps from the rounded exact value,
    max error per |ref| band)."""
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = bf16_bound(r, atol, stored_bf16)
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), (f"{what}: |gpu - ref| = {err.flat[worst]:.4e} at ref = {r.flat[worst]:.4f} "
                                  f"exceeds {bound.flat[worst]:.4e}; per |ref| band {band_errors(err, r)}")
    rounded = torch.from_numpy(r).to(torch.float32).to(torch.bfloat16).double().numpy()
    diff = np.abs(g - rounded)
    ulps = np.where(diff > ABS_FLOOR, diff / bf16_ulp(np.maximum(np.abs(g), np.abs(rounded))), 0.0)
    return float(np.max(err)), float(np.max(ulps)), band_errors(err, r)


def check_relative(gpu, ref, rtol: float, what: str = ""):
    """max|gpu - ref| <= rtol * max|ref| (inputs far from the unit scale)."""
    g, r = to64(gpu), to64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    scale = np.max(np.abs(r))
    err = np.max(np.abs(g - r))
    assert err <= rtol * scale, f"{what}: max error {err:.4e} > {rtol:g} x max|ref| = {rtol * scale:.4e}"
    return err / scale if scale > 0 else err


def check(gpu, ref, dtype: torch.dtype, what: str = "", stored_bf16: bool = True):
    """Tolerance of the storage type `dtype`; stored_bf16=False for float32 outputs (lse) of a
    bf16 call."""
    if dtype == torch.float32:
        return check_f32(gpu, ref, what=what)
    return check_bf16(gpu, ref, what=what, stored_bf16=stored_bf16)
