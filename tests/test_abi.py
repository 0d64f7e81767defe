"""Host-side tests of libfibattn.so: no GPU needed.

* the library loads and exports every function include/fibattn.h declares;
* the offset plan is bit-exact against the oracle's planner (kind, floor, float32 t, reach);
* base lists and schedules equal the oracle's;
* every argument check returns its status (and never launches: all are caught on the host).
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import fibonacci_offset_sparse_amd as fa
from oracle import fibattn_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KIND = {O.DUP: fa.DUP, O.INT: fa.INT, O.INTERP: fa.INTERP}


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fibattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fibattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) <= set(fa.__all__)


def _plan_equal(alpha, W, offsets):
    kind, fl, t, reach = fa.fibattn_plan(alpha, W, offsets)
    ref = O.plan_offsets(alpha, W, offsets)
    assert [KIND[r.kind] for r in ref] == kind.tolist()
    assert [r.a for r in ref] == fl.tolist()
    assert [r.reach for r in ref] == reach.tolist()
    assert np.array_equal(np.array([r.t for r in ref], dtype=np.float32).view(np.uint32), t.view(np.uint32))


@pytest.mark.parametrize("schedule", ["fixed", "linear", "coprime"])
@pytest.mark.parametrize("W,base", [(6, "fib"), (10, "fib"), (12, "fib"), (8, "pow2")])
def test_plan_bit_exact_against_the_oracle_on_every_schedule(schedule, W, base):
    offsets = O.FIB_BASE if base == "fib" else O.POW2_BASE_1024
    code = {"fixed": fa.SCHEDULE_FIXED, "linear": fa.SCHEDULE_LINEAR, "coprime": fa.SCHEDULE_COPRIME}[schedule]
    ref_fn = {"fixed": O.alpha_fixed, "linear": O.alpha_linear, "coprime": O.alpha_coprime}[schedule]
    for layer in range(16):
        alpha = fa.fibattn_alpha_schedule(code, layer, 16)
        assert alpha == ref_fn(layer, 16)
        _plan_equal(alpha, W, offsets)


def test_coprime_schedule_is_the_printed_permutation():
    from golden import loader
    perm = loader.int_list("coprime_permutation.txt")
    for layer in range(16):
        assert fa.fibattn_alpha_schedule(fa.SCHEDULE_COPRIME, layer, 16) == \
            fa.fibattn_alpha_schedule(fa.SCHEDULE_LINEAR, perm[layer], 16)


def test_plan_bit_exact_on_random_and_learned_alphas():
    rng = np.random.default_rng(7)
    for alpha in rng.uniform(0.5, 1.5, 10000):
        _plan_equal(float(alpha), int(rng.integers(0, 32)), O.FIB_BASE)
    import workloads
    for th in workloads.draw_theta(16).tolist():
        a, d = fa.fibattn_alpha_from_theta(th)
        assert abs(a - O.alpha_from_theta(th)) <= 2 ** -52
        assert abs(d - O.dalpha_dtheta(th)) <= 1e-15
        _plan_equal(a, 10, O.FIB_BASE)


def test_kept_rungs_floors_and_reach_never_decrease():
    # the matrix-core kernels count the rungs a tile reaches, and those its near block holds, from
    # the kept rungs' floors and reach as counts under a bound: equal to the prefix lengths only
    # because both sequences are non-decreasing (the distances alpha f increase with the rung)
    rng = np.random.default_rng(11)
    bases = [O.FIB_BASE, fa.fibattn_base_offsets(fa.BASE_POW2, 1024), fa.fibattn_base_offsets(fa.BASE_POW2, 2048)]
    alphas = list(rng.uniform(0.05, 4.0, 3000)) + [0.5 + l / 15 for l in range(16)] + [1.0, 2.0, 1.5, 0.5]
    for base in bases:
        for alpha in alphas:
            kind, fl, t, reach = fa.fibattn_plan(float(alpha), 12, base)
            kept = kind != fa.DUP
            assert (np.diff(fl[kept]) >= 0).all() and (np.diff(reach[kept]) >= 0).all(), (alpha, fl, reach)


def test_plan_snaps_the_float64_traps():
    kind, fl, t, reach = fa.fibattn_plan(O.alpha_linear(5, 16), 12, [144])
    assert kind[0] == fa.INT and fl[0] == 120 and t[0] == 0.0
    kind, fl, t, reach = fa.fibattn_plan(O.alpha_linear(10, 16), 12, [144])
    assert kind[0] == fa.INT and fl[0] == 168


def test_base_offsets_match_the_oracle():
    assert fa.fibattn_base_offsets(fa.BASE_FIB) == O.FIB_BASE
    assert fa.fibattn_base_offsets(fa.BASE_POW2, 1024) == O.POW2_BASE_1024
    assert fa.fibattn_base_offsets(fa.BASE_POW2, 2048) == O.POW2_BASE_2048
    assert fa.fibattn_base_offsets(fa.BASE_POW2, 1000)[-1] == 512


def test_workspace_sizes():
    assert fa.fibattn_fwd_workspace_bytes(32, 1024, 2) >= 32 * 2 * 1024 * 64 * 4
    assert fa.fibattn_bwd_workspace_bytes(32, 1024, 8, 2, 64, 10, 15) > fa.fibattn_fwd_workspace_bytes(32, 1024, 2)
    assert fa.fibattn_fwd_workspace_bytes(0, 1024, 2) == 0


# ------------------------------------------------------------------------------------------------
# Argument checks. Pointers are fake non-null integers: every call must fail on the host.
# ------------------------------------------------------------------------------------------------

FAKE = 0x1000


def fwd_call(q=FAKE, k=FAKE, v=FAKE, alpha=1.0, W=6, offsets=O.FIB_BASE, K=None, B=1, L=64, Hq=8, Hkv=2,
             D=64, dtype=0, theta=1e4, o=FAKE, lse=FAKE, ws=FAKE, ws_bytes=None):
    offs, n = fa._i32_array(offsets)
    K = n if K is None else K
    if ws_bytes is None:
        ws_bytes = 0
    return fa.lib.fibattn_fwd(q, k, v, alpha, W, offs if offsets is not None else None, K, B, L, Hq, Hkv, D,
                              dtype, theta, o, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), fa.FibAttnError and 1),
    (dict(k=None), 1),
    (dict(v=None), 1),
    (dict(o=None), 1),
    (dict(B=0), 1),
    (dict(L=0), 1),
    (dict(Hq=0), 1),
    (dict(Hkv=0), 1),
    (dict(Hq=8, Hkv=3), 1),
    (dict(W=-1), 1),
    (dict(K=33), 1),
    (dict(K=-1), 1),
    (dict(alpha=0.0), 1),
    (dict(alpha=-1.0), 1),
    (dict(alpha=float("nan")), 1),
    (dict(alpha=float("inf")), 1),
    (dict(offsets=[1, 3, 2]), 1),
    (dict(offsets=[0, 1, 2]), 1),
    (dict(offsets=[5, 5]), 1),
    (dict(dtype=7), 1),
    (dict(theta=0.0), 1),
    (dict(theta=float("nan")), 1),
    (dict(D=32), 2),
    (dict(D=128), 2),
    (dict(W=32), 2),
    (dict(L=(1 << 20) + 1), 2),
    (dict(ws=None), 3),
    (dict(ws_bytes=10), 3),
])
def test_fwd_argument_checks(kwargs, status):
    st = fwd_call(**kwargs)
    assert st == status, (kwargs, st, fa.fibattn_last_error())
    assert fa.fibattn_last_error() != ""
    assert fa.fibattn_status_string(st) != "unknown status"


def test_fwd_null_offsets_with_positive_k():
    st = fa.lib.fibattn_fwd(FAKE, FAKE, FAKE, 1.0, 6, None, 3, 1, 64, 8, 2, 64, 0, 1e4, FAKE, FAKE, FAKE, 1 << 30,
                            None)
    assert st == 1


def bwd_call(alpha=0.73, offsets=O.FIB_BASE, want_dalpha=True, ws_bytes=1 << 40, dq=FAKE, lse=FAKE, D=64,
             dadt=0.25):
    offs, n = fa._i32_array(offsets)
    return fa.lib.fibattn_bwd(FAKE, FAKE, FAKE, FAKE, lse, FAKE, alpha, 6, offs, n, 1, 64, 8, 2, D, 1, 1e4, dadt,
                              dq, FAKE, FAKE, FAKE if want_dalpha else None, None, FAKE, ws_bytes, None)


def test_bwd_argument_checks():
    assert bwd_call(dq=None) == 1
    assert bwd_call(D=48) == 2
    assert bwd_call(ws_bytes=100) == 3
    assert bwd_call(dadt=float("nan")) == 1
    # d(alpha) at an integral rung has no two-sided slope: refused
    assert bwd_call(alpha=1.0) == 2
    assert "integral" in fa.fibattn_last_error()


def test_bwd_stage_mask_checks():
    offs, n = fa._i32_array(O.FIB_BASE)

    def staged(mask, dq=FAKE):
        return fa.lib.fibattn_bwd_stages(mask, FAKE, FAKE, FAKE, FAKE, 0.73, 6, offs, n, 1, 64, 8, 2, 64, 1, 1e4,
                                         0.0, dq, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    for bad in (0, 8, -1):
        assert staged(bad) == 1
        assert "stage mask" in fa.fibattn_last_error()
    # every argument is checked whatever the mask
    assert staged(fa.STAGE_PREP, dq=None) == 1


def test_bwd_reuses_fwd_prep():
    # bf16 on the matrix-core backward (query heads per kv head a multiple of 4, W <= 15, at most
    # 16 kept rungs) reads the forward's staged arrays; float32 runs the same key rotation in both
    assert fa.fibattn_bwd_reuses_fwd_prep(0.5 + 3 / 15, 12, O.FIB_BASE, 32, 1024, 8, 2)
    assert fa.fibattn_bwd_reuses_fwd_prep(1.0, 12, O.FIB_BASE, 1, 64, 8, 2, dtype=fa.F32)
    assert fa.fibattn_bwd_reuses_fwd_prep(1.0, 31, O.FIB_BASE, 1, 64, 6, 2, dtype=fa.F32)
    # general bf16 backward (float32 keys of its own): GQA group of 2, a window past 15
    assert not fa.fibattn_bwd_reuses_fwd_prep(0.7, 12, O.FIB_BASE, 1, 64, 4, 2)
    assert not fa.fibattn_bwd_reuses_fwd_prep(0.7, 20, O.FIB_BASE, 1, 64, 8, 2)
    # arguments the backward rejects
    assert not fa.fibattn_bwd_reuses_fwd_prep(0.7, 12, O.FIB_BASE, 1, 64, 8, 3)
    assert not fa.fibattn_bwd_reuses_fwd_prep(-1.0, 12, O.FIB_BASE, 1, 64, 8, 2)
    assert not fa.fibattn_bwd_reuses_fwd_prep(0.7, 12, O.FIB_BASE, 1, 64, 8, 2, D=48)


def test_round_offsets_match_the_oracle():
    # every linear and coprime ramp value, both bases, and a few hand-picked alphas with ties
    alphas = [O.alpha_linear(l, 16) for l in range(16)] + [O.alpha_coprime(l, 16) for l in range(16)]
    alphas += [1.0, 0.5, 1.5, 2.5, 0.37, 0.5 + 5 / 15]
    for base in (O.FIB_BASE, O.POW2_BASE_1024):
        for a in alphas:
            assert fa.fibattn_round_offsets(a, base) == O.rounded_offsets(a, base), (a, base)
    # the integer path reads them at alpha = 1: every kept rung integral
    kind, fl, t, _ = fa.fibattn_plan(1.0, 12, fa.fibattn_round_offsets(0.5 + 7 / 15, O.FIB_BASE))
    assert set(kind.tolist()) <= {fa.INT, fa.DUP} and not t.any()


def test_round_offsets_argument_checks():
    offs, n = fa._i32_array(O.FIB_BASE)
    out = (ctypes.c_int32 * 15)()
    cnt = ctypes.c_int32()
    assert fa.lib.fibattn_round_offsets(-1.0, offs, n, out, 15, ctypes.byref(cnt)) == 1
    assert fa.lib.fibattn_round_offsets(1.0, offs, n, None, 15, ctypes.byref(cnt)) == 1
    assert fa.lib.fibattn_round_offsets(1.0, offs, n, out, 14, ctypes.byref(cnt)) == 1     # 15 distinct at alpha = 1
    bad, m = fa._i32_array([1, 3, 2])
    assert fa.lib.fibattn_round_offsets(1.0, bad, m, out, 15, ctypes.byref(cnt)) == 1
    assert fa.lib.fibattn_round_offsets(2e9, offs, n, out, 15, ctypes.byref(cnt)) == 2
    assert fa.lib.fibattn_round_offsets(0.5, offs, 0, out, 0, ctypes.byref(cnt)) == 0 and cnt.value == 0


def test_host_helpers_argument_checks():
    out = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32()
    assert fa.lib.fibattn_base_offsets(fa.BASE_FIB, 0, out, 4, ctypes.byref(n)) == 1     # capacity < 15
    assert fa.lib.fibattn_base_offsets(9, 0, out, 4, ctypes.byref(n)) == 1
    assert fa.lib.fibattn_base_offsets(fa.BASE_POW2, 0, out, 4, ctypes.byref(n)) == 1
    a = ctypes.c_double()
    assert fa.lib.fibattn_alpha_schedule(fa.SCHEDULE_LINEAR, 16, 16, ctypes.byref(a)) == 1
    assert fa.lib.fibattn_alpha_schedule(fa.SCHEDULE_COPRIME, 0, 14, ctypes.byref(a)) == 1
    assert fa.lib.fibattn_alpha_schedule(5, 0, 16, ctypes.byref(a)) == 1
    assert fa.lib.fibattn_alpha_from_theta(float("inf"), ctypes.byref(a), None) == 1
    with pytest.raises(fa.FibAttnError):
        fa.fibattn_plan(1.0, -1, O.FIB_BASE)
    with pytest.raises(fa.FibAttnError):
        fa.fibattn_plan(2e9, 4, [1])
    assert fa.fibattn_status_string(99) == "unknown status"
    assert math.isfinite(fa.fibattn_alpha_schedule(fa.SCHEDULE_COPRIME, 3, 16))


def test_phase_trace_reader_in_both_builds():
    # the usual library has no trace and says so; the trace build exports the same functions and
    # checks its arguments before touching the GPU
    buf = (ctypes.c_uint64 * 8)()
    lib = ctypes.CDLL(fa.LIB_PATH)
    f = lib.fibattn_phase_trace_read
    f.restype, f.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]
    assert f(buf, 1) == 2
    tlib = ctypes.CDLL(fa.TRACE_LIB_PATH)
    for name in declared_functions():
        assert hasattr(tlib, name), name
    g = tlib.fibattn_phase_trace_read
    g.restype, g.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]
    assert g(None, 1) == 1
    assert g(buf, -1) == 1
    assert g(buf, 65537) == 1
