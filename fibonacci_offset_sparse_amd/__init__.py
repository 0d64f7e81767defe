"""Python binding of libfibattn.so: Fibonacci-offset sparse attention on MI355X (gfx950).

Argument marshalling only. Every step of the forward and backward pass runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream. The functions carry the
names of the C entry points in include/fibattn.h. Importing this package fails if the library
has not been built (python fibonacci_offset_sparse_amd/build.py).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfibattn.so")
# the same library with the forward attention kernel's phase trace compiled in (measurement only)
TRACE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfibattn_trace.so")

F32, BF16 = 0, 1
DUP, INT, INTERP = 0, 1, 2
BASE_FIB, BASE_POW2 = 0, 1
SCHEDULE_FIXED, SCHEDULE_LINEAR, SCHEDULE_COPRIME = 0, 1, 2
MAX_W, MAX_K = 31, 32
STAGE_PREP, STAGE_QUERY, STAGE_KEY, STAGE_ALL = 1, 2, 4, 7

_c_i32, _c_u8, _c_f32, _c_f64 = ctypes.c_int32, ctypes.c_uint8, ctypes.c_float, ctypes.c_double
_c_ptr, _c_size = ctypes.c_void_p, ctypes.c_size_t
_P = ctypes.POINTER


def _load() -> ctypes.CDLL:
    return _load_from(LIB_PATH)


def _load_from(path: str) -> ctypes.CDLL:
    """The library at path with every entry point's signature set (the usual build or the trace build)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python fibonacci_offset_sparse_amd/build.py`")
    lib = ctypes.CDLL(path)
    sig = {
        "fibattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "fibattn_last_error": (ctypes.c_char_p, []),
        "fibattn_base_offsets": (ctypes.c_int, [_c_i32, _c_i32, _P(_c_i32), _c_i32, _P(_c_i32)]),
        "fibattn_alpha_schedule": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _P(_c_f64)]),
        "fibattn_alpha_from_theta": (ctypes.c_int, [_c_f64, _P(_c_f64), _P(_c_f64)]),
        "fibattn_round_offsets": (ctypes.c_int, [_c_f64, _P(_c_i32), _c_i32, _P(_c_i32), _c_i32, _P(_c_i32)]),
        "fibattn_plan": (ctypes.c_int, [_c_f64, _c_i32, _P(_c_i32), _c_i32, _P(_c_u8), _P(_c_i32),
                                         _P(_c_f32), _P(_c_i32)]),
        "fibattn_fwd_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
        "fibattn_fwd": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32, _P(_c_i32), _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f64,
                                        _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
        "fibattn_fwd_prep": (ctypes.c_int, [_c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                             _c_f64, _c_ptr, _c_size, _c_ptr]),
        "fibattn_fwd_attend": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32, _P(_c_i32), _c_i32,
                                               _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f64,
                                               _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
        "fibattn_fwd_noalloc": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32, _P(_c_i32), _c_i32,
                                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f64,
                                                _c_ptr, _c_ptr, _c_ptr]),
        "fibattn_fwd_noalloc_max_bytes": (_c_size, []),
        "fibattn_decode": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32, _P(_c_i32), _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f64, _c_ptr,
                                           _c_ptr, _c_ptr]),
        "fibattn_bwd_workspace_bytes": (_c_size, [_c_i32] * 8),
        "fibattn_bwd": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32,
                                        _P(_c_i32), _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_i32, _c_f64, _c_f64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                        _c_ptr, _c_ptr, _c_size, _c_ptr]),
        "fibattn_bwd_reuses_fwd_prep": (_c_i32, [_c_f64, _c_i32, _P(_c_i32), _c_i32, _c_i32, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i32]),
        "fibattn_bwd_stages": (ctypes.c_int, [_c_i32, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_f64, _c_i32,
                                               _P(_c_i32), _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                               _c_i32, _c_f64, _c_f64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                               _c_ptr, _c_ptr, _c_size, _c_ptr]),
        "fibattn_phase_trace_read": (ctypes.c_int, [_P(ctypes.c_uint64), _c_i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class FibAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def fibattn_status_string(status: int) -> str:
    return lib.fibattn_status_string(status).decode()


def fibattn_last_error() -> str:
    return lib.fibattn_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise FibAttnError(status, f"{fibattn_status_string(status)}: {fibattn_last_error()}")


def _i32_array(values: Sequence[int]):
    values = [int(x) for x in values]
    return (_c_i32 * max(1, len(values)))(*values), len(values)


# ------------------------------------------------------------------------------------------------
# Host-only entry points (no GPU needed)
# ------------------------------------------------------------------------------------------------

def fibattn_base_offsets(base: int = BASE_FIB, pow2_max: int = 1024) -> Tuple[int, ...]:
    out = (_c_i32 * MAX_K)()
    n = _c_i32()
    _check(lib.fibattn_base_offsets(base, pow2_max, out, MAX_K, ctypes.byref(n)))
    return tuple(out[: n.value])


def fibattn_alpha_schedule(schedule: int, layer: int, n_layers: int) -> float:
    a = _c_f64()
    _check(lib.fibattn_alpha_schedule(schedule, layer, n_layers, ctypes.byref(a)))
    return a.value


def fibattn_alpha_from_theta(theta: float) -> Tuple[float, float]:
    a, d = _c_f64(), _c_f64()
    _check(lib.fibattn_alpha_from_theta(float(theta), ctypes.byref(a), ctypes.byref(d)))
    return a.value, d.value


def fibattn_round_offsets(alpha: float, offsets: Sequence[int]) -> Tuple[int, ...]:
    """Rounded-integer stagger: the distinct round-half-even(alpha f_k) >= 1, increasing; run them with
    alpha = 1."""
    offs, K = _i32_array(offsets)
    out = (_c_i32 * max(K, 1))()
    n = _c_i32()
    _check(lib.fibattn_round_offsets(float(alpha), offs, K, out, max(K, 1), ctypes.byref(n)))
    return tuple(int(out[i]) for i in range(n.value))


def fibattn_plan(alpha: float, W: int, offsets: Sequence[int]):
    """(kind uint8[K], floor int32[K], t float32[K], reach int32[K]) of the offset plan."""
    offs, K = _i32_array(offsets)
    kind = np.zeros(max(K, 1), np.uint8)
    fl = np.zeros(max(K, 1), np.int32)
    t = np.zeros(max(K, 1), np.float32)
    reach = np.zeros(max(K, 1), np.int32)
    _check(lib.fibattn_plan(float(alpha), int(W), offs, K,
                            kind.ctypes.data_as(_P(_c_u8)), fl.ctypes.data_as(_P(_c_i32)),
                            t.ctypes.data_as(_P(_c_f32)), reach.ctypes.data_as(_P(_c_i32))))
    return kind[:K], fl[:K], t[:K], reach[:K]


def fibattn_fwd_workspace_bytes(B: int, L: int, Hkv: int, D: int = 64, dtype: int = BF16) -> int:
    return int(lib.fibattn_fwd_workspace_bytes(B, L, Hkv, D, dtype))


def fibattn_bwd_workspace_bytes(B: int, L: int, Hq: int, Hkv: int, D: int, W: int, K: int,
                                dtype: int = BF16) -> int:
    return int(lib.fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, W, K, dtype))


# ------------------------------------------------------------------------------------------------
# Device entry points
# ------------------------------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, shape, dtype) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, L, D]")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return int(s.cuda_stream)


def _shapes(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, L, D]")
    B, Hq, L, D = q.shape
    return B, Hq, L, D, k.shape[1]


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not ws.is_cuda or ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
    return ws


def fibattn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: float, W: int,
                offsets: Sequence[int], rope_theta: float = 1e4, o: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, need_lse: bool = True,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """o [B, Hq, L, D] (and lse [B, Hq, L] float32 when need_lse) of the sparse attention."""
    B, Hq, L, D, Hkv = _shapes(q, k)
    dt = _dtype_code(q)
    args = [_dev(q, "q", (B, Hq, L, D), q.dtype), _dev(k, "k", (B, Hkv, L, D), q.dtype),
            _dev(v, "v", (B, Hkv, L, D), q.dtype)]
    o = torch.empty_like(q) if o is None else o
    if need_lse and lse is None:
        lse = torch.empty(B, Hq, L, dtype=torch.float32, device=q.device)
    optr = _dev(o, "o", (B, Hq, L, D), q.dtype)
    lptr = _dev(lse, "lse", (B, Hq, L), torch.float32) if lse is not None else None
    nbytes = fibattn_fwd_workspace_bytes(B, L, Hkv, D, dt)
    ws = _workspace(workspace, nbytes, q.device)
    offs, K = _i32_array(offsets)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_fwd(*args, float(alpha), int(W), offs, K, B, L, Hq, Hkv, D, dt,
                               float(rope_theta), optr, lptr, ws.data_ptr(), ws.numel(),
                               _stream(q.device, stream)))
    return o, lse


def fibattn_phase_trace_read(n_wg: int) -> np.ndarray:
    """The forward attention kernel's phase records of its last launch, uint64 [n_wg, 8] (the trace
    build only: load TRACE_LIB_PATH; other builds raise FibAttnError UNSUPPORTED)."""
    out = np.zeros((int(n_wg), 8), dtype=np.uint64)
    _check(lib.fibattn_phase_trace_read(out.ctypes.data_as(_P(ctypes.c_uint64)), int(n_wg)))
    return out


def fibattn_fwd_noalloc_max_bytes() -> int:
    return int(lib.fibattn_fwd_noalloc_max_bytes())


def fibattn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: float, W: int,
                        offsets: Sequence[int], o: torch.Tensor, lse: Optional[torch.Tensor] = None,
                        rope_theta: float = 1e4, stream=None) -> None:
    """The allocation-free forward: o (and lse if given) written in place, no workspace (the library
    holds fibattn_fwd_noalloc_max_bytes() of device scratch per GPU). Calls that overlap on one GPU
    race on that scratch."""
    B, Hq, L, D, Hkv = _shapes(q, k)
    dt = _dtype_code(q)
    args = [_dev(q, "q", (B, Hq, L, D), q.dtype), _dev(k, "k", (B, Hkv, L, D), q.dtype),
            _dev(v, "v", (B, Hkv, L, D), q.dtype)]
    optr = _dev(o, "o", (B, Hq, L, D), q.dtype)
    lptr = _dev(lse, "lse", (B, Hq, L), torch.float32) if lse is not None else None
    offs, K = _i32_array(offsets)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_fwd_noalloc(*args, float(alpha), int(W), offs, K, B, L, Hq, Hkv, D, dt, float(rope_theta),
                                       optr, lptr, _stream(q.device, stream)))


def fibattn_fwd_prep(k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor, rope_theta: float = 1e4,
                     stream=None):
    """First forward stage: rotated keys (and fp16 values for bf16) into `workspace`."""
    B, Hkv, L, D = k.shape
    dt = _dtype_code(k)
    _dev(k, "k", (B, Hkv, L, D), k.dtype)
    _dev(v, "v", (B, Hkv, L, D), k.dtype)
    with torch.cuda.device(k.device):
        _check(lib.fibattn_fwd_prep(k.data_ptr(), v.data_ptr(), B, L, Hkv, D, dt, float(rope_theta),
                                    workspace.data_ptr(), workspace.numel(), _stream(k.device, stream)))


def fibattn_fwd_attend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: float, W: int,
                       offsets: Sequence[int], workspace: torch.Tensor, o: torch.Tensor,
                       lse: Optional[torch.Tensor] = None, rope_theta: float = 1e4, stream=None):
    """Second forward stage; reads what fibattn_fwd_prep left in `workspace`."""
    B, Hq, L, D, Hkv = _shapes(q, k)
    dt = _dtype_code(q)
    _dev(q, "q", (B, Hq, L, D), q.dtype)
    _dev(k, "k", (B, Hkv, L, D), q.dtype)
    _dev(v, "v", (B, Hkv, L, D), q.dtype)
    _dev(o, "o", (B, Hq, L, D), q.dtype)
    lptr = _dev(lse, "lse", (B, Hq, L), torch.float32) if lse is not None else None
    offs, K = _i32_array(offsets)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_fwd_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(alpha), int(W), offs, K, B, L,
                                      Hq, Hkv, D, dt, float(rope_theta), o.data_ptr(), lptr,
                                      workspace.data_ptr(), workspace.numel(), _stream(q.device, stream)))


def fibattn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
                   alpha: float, W: int, offsets: Sequence[int], rope_theta: float = 1e4,
                   o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, need_lse: bool = True,
                   stream=None):
    """(o [B, Hq, D], lse [B, Hq] or None): each sequence's new query q[b] at position positions[b]
    (int32 on the device) against its cache rows k_cache[b], v_cache[b] ([B, Hkv, Lmax, D])."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches [B, Hkv, Lmax, D]")
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    args = [_dev(q, "q", (B, Hq, D), q.dtype), _dev(k_cache, "k_cache", (B, Hkv, Lmax, D), q.dtype),
            _dev(v_cache, "v_cache", (B, Hkv, Lmax, D), q.dtype), _dev(positions, "positions", (B,), torch.int32)]
    o = torch.empty_like(q) if o is None else o
    if need_lse and lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    optr = _dev(o, "o", (B, Hq, D), q.dtype)
    lptr = _dev(lse, "lse", (B, Hq), torch.float32) if lse is not None else None
    offs, K = _i32_array(offsets)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_decode(*args, float(alpha), int(W), offs, K, B, Lmax, Hq, Hkv, D, dt, float(rope_theta),
                                  optr, lptr, _stream(q.device, stream)))
    return o, lse


def fibattn_bwd_reuses_fwd_prep(alpha: float, W: int, offsets: Sequence[int], B: int, L: int, Hq: int,
                                Hkv: int, D: int = 64, dtype: int = BF16) -> bool:
    """Whether the backward's STAGE_PREP writes what fibattn_fwd_prep writes (then a backward whose
    workspace holds the forward's prep of the same k, v may run STAGE_QUERY | STAGE_KEY only)."""
    offs, K = _i32_array(offsets)
    return bool(lib.fibattn_bwd_reuses_fwd_prep(float(alpha), int(W), offs, K, B, L, Hq, Hkv, D, dtype))


def fibattn_bwd_stages(stages: int, q, k, v, dout, alpha: float, W: int, offsets: Sequence[int],
                       dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, workspace: torch.Tensor,
                       rope_theta: float = 1e4, dalpha_dtheta: float = 0.0,
                       dalpha: Optional[torch.Tensor] = None, dtheta: Optional[torch.Tensor] = None,
                       stream=None):
    """Backward stages selected by the mask `stages` (STAGE_PREP | STAGE_QUERY | STAGE_KEY) into
    the given outputs; a subset must follow the calls that ran the earlier stages on the same
    workspace and stream."""
    B, Hq, L, D, Hkv = _shapes(q, k)
    dt = _dtype_code(q)
    ptrs = [_dev(q, "q", (B, Hq, L, D), q.dtype), _dev(k, "k", (B, Hkv, L, D), q.dtype),
            _dev(v, "v", (B, Hkv, L, D), q.dtype), _dev(dout, "dout", (B, Hq, L, D), q.dtype)]
    outs = [_dev(dq, "dq", (B, Hq, L, D), q.dtype), _dev(dk, "dk", (B, Hkv, L, D), q.dtype),
            _dev(dv, "dv", (B, Hkv, L, D), q.dtype),
            _dev(dalpha, "dalpha", (1,), torch.float32) if dalpha is not None else None,
            _dev(dtheta, "dtheta", (1,), torch.float32) if dtheta is not None else None]
    offs, K = _i32_array(offsets)
    nbytes = fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, W, K, dt)
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_bwd_stages(int(stages), *ptrs, float(alpha), int(W), offs, K, B, L, Hq, Hkv, D, dt,
                                      float(rope_theta), float(dalpha_dtheta), *outs, ws.data_ptr(), ws.numel(),
                                      _stream(q.device, stream)))


def fibattn_bwd(q, k, v, o, lse, dout, alpha: float, W: int, offsets: Sequence[int],
                rope_theta: float = 1e4, dalpha_dtheta: float = 0.0, want_dalpha: bool = False,
                workspace: Optional[torch.Tensor] = None, stream=None, dq: Optional[torch.Tensor] = None,
                dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None):
    """(dq, dk, dv, dalpha, dtheta); dalpha and dtheta are float32[1] GPU tensors or None.

    o and lse may be None (the library does not read them). dq, dk, dv are allocated unless given."""
    B, Hq, L, D, Hkv = _shapes(q, k)
    dt = _dtype_code(q)
    # o and lse are part of the usual signature; the library recomputes what it needs from them
    ptrs = [_dev(q, "q", (B, Hq, L, D), q.dtype), _dev(k, "k", (B, Hkv, L, D), q.dtype),
            _dev(v, "v", (B, Hkv, L, D), q.dtype),
            _dev(o, "o", (B, Hq, L, D), q.dtype) if o is not None else None,
            _dev(lse, "lse", (B, Hq, L), torch.float32) if lse is not None else None,
            _dev(dout, "dout", (B, Hq, L, D), q.dtype)]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    outs = [_dev(dq, "dq", (B, Hq, L, D), q.dtype), _dev(dk, "dk", (B, Hkv, L, D), q.dtype),
            _dev(dv, "dv", (B, Hkv, L, D), q.dtype)]
    da = torch.empty(1, dtype=torch.float32, device=q.device) if want_dalpha else None
    dth = torch.empty(1, dtype=torch.float32, device=q.device) if want_dalpha else None
    offs, K = _i32_array(offsets)
    nbytes = fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, W, K, dt)
    ws = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        _check(lib.fibattn_bwd(*ptrs, float(alpha), int(W), offs, K, B, L, Hq, Hkv, D, dt,
                               float(rope_theta), float(dalpha_dtheta), *outs,
                               da.data_ptr() if da is not None else None,
                               dth.data_ptr() if dth is not None else None, ws.data_ptr(), ws.numel(),
                               _stream(q.device, stream)))
    return dq, dk, dv, da, dth


__all__ = [
    "fibattn_status_string", "fibattn_last_error", "fibattn_base_offsets", "fibattn_alpha_schedule",
    "fibattn_alpha_from_theta", "fibattn_round_offsets", "fibattn_plan", "fibattn_fwd_workspace_bytes", "fibattn_fwd",
    "fibattn_fwd_prep", "fibattn_fwd_attend", "fibattn_fwd_noalloc", "fibattn_fwd_noalloc_max_bytes", "fibattn_bwd_workspace_bytes", "fibattn_bwd",
    "fibattn_bwd_stages", "fibattn_bwd_reuses_fwd_prep", "fibattn_decode", "STAGE_PREP", "STAGE_QUERY", "STAGE_KEY", "STAGE_ALL",
    "fibattn_phase_trace_read", "FibAttnError", "lib", "LIB_PATH", "TRACE_LIB_PATH",
]
