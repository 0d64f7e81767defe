"""Pins of the float64 oracle to what the paper and the mathematics fix.

None of these tests re-types the oracle's formulas. Each check comes from somewhere else:
* the paper's printed constants (tests/golden, each with its citation);
* exact rational arithmetic (fractions.Fraction) for the offset plan;
* brute force with explicit per-query loops, RoPE written with complex numbers, and a library
  routine (torch scaled_dot_product_attention in float64 on the CPU) for masked dense attention;
* special cases that reduce to textbook attention, closed-form rows and invariants;
* central finite differences for every gradient.
Citations name sections of "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static
Schedules Beat Learned Dilation and Extrapolate Where Dense Attention Fails".
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from golden import loader
from oracle import fibattn_oracle as O

rng = np.random.default_rng(1234)


# ------------------------------------------------------------------------------------------------
# Independent helpers (brute force). They share nothing with the oracle's code.
# ------------------------------------------------------------------------------------------------

def rot_complex(x, p, theta=1e4):
    """Rotate one row at position p: pairs (x_j, x_{j+D/2}) as complex numbers times e^{i p w_j}."""
    D = x.shape[-1]
    w = np.array([theta ** (-(2.0 * j) / D) for j in range(D // 2)])
    z = (x[: D // 2] + 1j * x[D // 2:]) * np.exp(1j * p * w)
    return np.concatenate([z.real, z.imag])


def exact_offsets(alpha_frac, W, base):
    """Attended offsets from exact rationals: list of (rows, weights, min_query) per kept rung."""
    out = []
    for f in base:
        d = alpha_frac * f
        if d.denominator == 1:
            if d <= W:
                continue                        # already a window distance
            n = int(d)
            out.append(([n], [1.0], n))
        else:
            a = d.numerator // d.denominator
            t = float(d - a)
            out.append(([a, a + 1], [1.0 - t, t], a + 1))
    return out


def brute_force_forward(q, k, v, alpha_frac, W, base, theta=1e4):
    """Per query: list the (key, value) pairs of the attended set, then softmax over them."""
    B, Hq, L, D = q.shape
    G = Hq // k.shape[1]
    offs = exact_offsets(alpha_frac, W, base)
    o = np.zeros((B, Hq, L, D))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            krot = [rot_complex(k[b, g, j], j, theta) for j in range(L)]
            for i in range(L):
                qi = rot_complex(q[b, h, i], i, theta)
                keys, vals = [], []
                for dist in range(W + 1):
                    if i - dist >= 0:
                        keys.append(krot[i - dist])
                        vals.append(v[b, g, i - dist])
                for dists, wts, imin in offs:
                    if i >= imin:
                        keys.append(sum(w * krot[i - dd] for w, dd in zip(wts, dists)))
                        vals.append(sum(w * v[b, g, i - dd] for w, dd in zip(wts, dists)))
                s = np.array([qi @ kk for kk in keys]) / math.sqrt(D)
                m = s.max()
                e = np.exp(s - m)
                o[b, h, i] = (e[:, None] * np.array(vals)).sum(0) / e.sum()
                lse[b, h, i] = m + math.log(e.sum())
    return o, lse


def rope_all(x, theta=1e4):
    out = np.empty_like(x)
    for idx in np.ndindex(*x.shape[:-2]):
        for p in range(x.shape[-2]):
            out[idx + (p,)] = rot_complex(x[idx + (p,)], p, theta)
    return out


def sdpa_masked(q, k, v, mask, theta=1e4):
    """Dense attention with a boolean mask via torch's SDPA (CPU float64), keys/values per head."""
    G = q.shape[1] // k.shape[1]
    qr = torch.from_numpy(rope_all(q, theta))
    kr = torch.from_numpy(rope_all(k, theta)).repeat_interleave(G, dim=1)
    vv = torch.from_numpy(np.asarray(v, dtype=np.float64)).repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, attn_mask=torch.from_numpy(mask))
    return out.numpy()


def integer_mask(L, W, distances):
    """M[i, j] = True iff i - j is in {0..W} or in the integer distance set, and j >= 0."""
    M = np.zeros((L, L), dtype=bool)
    allowed = set(range(W + 1)) | set(distances)
    for i in range(L):
        for dd in allowed:
            if 0 <= i - dd:
                M[i, i - dd] = True
    return M


def randn(*shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------------------------------------
# Constants and schedules
# ------------------------------------------------------------------------------------------------

def test_fib_base_is_the_papers_list():
    assert list(O.FIB_BASE) == loader.int_list("fib_base.txt")
    assert len(O.FIB_BASE) == 15


def test_pow2_base_is_powers_of_two_to_1024():
    assert list(O.POW2_BASE_1024) == [1 << n for n in range(11)]


def test_model_shape_constants():
    shape = loader.table("model_shape.txt")
    assert O.ROPE_THETA == shape["rope_theta"]
    assert shape["n_heads"] * shape["head_dim"] == shape["d_model"]
    assert shape["tokens_per_step"] / shape["seq_len"] == 32


def test_linear_schedule_endpoints_and_exact_values():
    g = loader.table("schedules.txt")
    n = int(g["n_layers"])
    vals = [O.alpha_linear(l, n) for l in range(n)]
    assert vals[0] == g["alpha_min"] and vals[-1] == g["alpha_max"]
    for l, a in enumerate(vals):
        exact = Fraction(1, 2) + Fraction(l, n - 1)
        assert abs(Fraction(a) - exact) <= Fraction(1, 2 ** 52)


def test_coprime_schedule_is_a_permutation_with_the_same_multiset():
    g = loader.table("schedules.txt")
    n, stride = int(g["n_layers"]), int(g["stride"])
    assert math.gcd(stride, n) == 1
    idx = [O.coprime_index(l, n, stride) for l in range(n)]
    assert sorted(idx) == list(range(n))
    lin = sorted(O.alpha_linear(l, n) for l in range(n))
    cop = sorted(O.alpha_coprime(l, n, stride) for l in range(n))
    assert lin == cop
    # adjacent layers move stride/(n-1) apart on the ramp (mod the wrap), never one step
    steps = [abs(idx[l + 1] - idx[l]) for l in range(n - 1)]
    assert min(steps) >= min(stride, n - stride)


def test_coprime_schedule_is_the_printed_permutation():
    # the exact map, not only its properties: a shifted (1-indexed) or mirrored map keeps the
    # multiset and the step sizes but not this list
    perm = loader.int_list("coprime_permutation.txt")
    n = int(loader.table("schedules.txt")["n_layers"])
    assert [O.coprime_index(l, n) for l in range(n)] == perm
    for l in range(n):
        assert O.alpha_coprime(l, n) == O.alpha_linear(perm[l], n)


def test_learned_alpha_parameterisation():
    g = loader.table("schedules.txt")
    assert O.alpha_from_theta(0.0) == g["alpha_at_theta_zero"]
    for th in np.linspace(-30, 30, 61):
        a = O.alpha_from_theta(float(th))
        assert g["alpha_min"] <= a <= g["alpha_max"]
    for th in [-1.3, 0.0, 0.4, 2.2]:
        h = 1e-6
        fd = (O.alpha_from_theta(th + h) - O.alpha_from_theta(th - h)) / (2 * h)
        assert abs(fd - O.dalpha_dtheta(th)) < 1e-9


# ------------------------------------------------------------------------------------------------
# Offset plan against exact rationals
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("base_name,W", [("fib", 6), ("fib", 10), ("fib", 12), ("pow2", 8)])
def test_plan_matches_exact_rationals_on_the_linear_ramp(base_name, W):
    base = O.FIB_BASE if base_name == "fib" else O.POW2_BASE_1024
    for l in range(16):
        alpha_frac = Fraction(15 + 2 * l, 30)          # 0.5 + l/15 exactly
        plan = O.plan_offsets(O.alpha_linear(l, 16), W, base)
        for off, f in zip(plan, base):
            d = alpha_frac * f
            if d.denominator == 1:
                assert off.kind == (O.DUP if d <= W else O.INT), (l, f)
                assert off.a == int(d) and off.t == 0.0 and off.reach == int(d)
            else:
                a = d.numerator // d.denominator
                assert off.kind == O.INTERP, (l, f)
                assert off.a == a and off.reach == a + 1
                assert abs(Fraction(off.t) - (d - a)) <= Fraction(1, 2 ** 40)


def test_plan_integral_points_of_the_fib_ramp():
    # exact count: with alpha_l = (15 + 2l)/30, l*f is integral only at these 16 (l, f) pairs
    hits = []
    for l in range(16):
        for f in O.FIB_BASE:
            if (Fraction(15 + 2 * l, 30) * f).denominator == 1:
                hits.append((l, f))
    assert len(hits) == 16
    for l, f in hits:
        off = O.plan_offsets(O.alpha_linear(l, 16), 0, [f])[0]
        assert off.kind == O.INT and off.d == float(Fraction(15 + 2 * l, 30) * f)
    # the two float64 traps: 0.8333..*144 and 1.1666..*144 land a hair below 120 and 168
    assert O.alpha_linear(5, 16) * 144 != 120.0
    assert O.plan_offsets(O.alpha_linear(5, 16), 12, [144])[0].a == 120
    assert O.plan_offsets(O.alpha_linear(10, 16), 12, [144])[0].a == 168


def test_plan_dedupes_only_integral_window_distances():
    plan = O.plan_offsets(1.0, 6, O.FIB_BASE)
    assert [p.kind for p in plan[:4]] == [O.DUP] * 4          # 1, 2, 3, 5 <= 6
    assert all(p.kind == O.INT for p in plan[4:])
    plan = O.plan_offsets(0.5, 12, O.FIB_BASE)                  # 0.5, 1, 1.5, 2.5, 4, ...
    assert plan[0].kind == O.INTERP and plan[0].a == 0 and plan[0].t == 0.5
    assert plan[1].kind == O.DUP
    assert plan[2].kind == O.INTERP and plan[2].reach == 2


# ------------------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------------------

def test_rope_against_complex_rotation_and_its_adjoint():
    x = randn(2, 3, 40, 16)
    np.testing.assert_allclose(O.rope(x), rope_all(x), rtol=0, atol=1e-13)
    g = randn(2, 3, 40, 16)
    # <R x, g> = <x, R^T g>
    assert abs(np.sum(O.rope(x) * g) - np.sum(x * O.rope_transpose(g))) < 1e-10
    np.testing.assert_allclose(O.rope_transpose(O.rope(x)), x, atol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    qv, kv = randn(16), randn(16)
    L = 50
    qr = O.rope(np.tile(qv, (L, 1)))
    kr = O.rope(np.tile(kv, (L, 1)))
    for delta in [0, 3, 17]:
        s = [qr[i] @ kr[i - delta] for i in range(delta, L)]
        np.testing.assert_allclose(s, s[0], atol=1e-11)


# ------------------------------------------------------------------------------------------------
# Forward: brute force, library routine, special cases
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("alpha_frac,W,base_name,L", [
    (Fraction(1), 6, "fib", 64),          # tiny workload's plan: 1,2,3,5 dropped
    (Fraction(1), 8, "pow2", 64),         # power-of-two base, alpha = 1
    (Fraction(2), 3, "fib", 48),          # every d integral, some beyond the window
    (Fraction(3), 5, "pow2", 40),         # 3, 6, 12, ...: 3 dropped, the rest integral rungs
])
def test_forward_integer_offsets_equal_masked_dense_attention(alpha_frac, W, base_name, L):
    base = O.FIB_BASE if base_name == "fib" else O.POW2_BASE_1024
    offs = exact_offsets(alpha_frac, W, base)
    if any(len(rows) > 1 for rows, _, _ in offs):
        pytest.skip("plan has interpolated rungs")
    q, k, v = randn(1, 4, L, 16), randn(1, 2, L, 16), randn(1, 2, L, 16)
    dists = [rows[0] for rows, _, _ in offs]
    ref = sdpa_masked(q, k, v, integer_mask(L, W, dists))
    o, _ = O.forward(q, k, v, float(alpha_frac), W, base)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("alpha_frac,W,base_name", [
    (Fraction(11, 15), 2, "fib"),         # all rungs interpolated
    (Fraction(1, 2), 3, "fib"),           # d = 0.5 reads rows i and i-1; d = 1 dropped
    (Fraction(19, 15), 4, "pow2"),
    (Fraction(15 + 2 * 5, 30), 3, "fib"),  # ramp layer 5: 144 -> 120 integral, rest interpolated
])
def test_forward_interpolated_equals_per_query_brute_force(alpha_frac, W, base_name):
    base = O.FIB_BASE if base_name == "fib" else O.POW2_BASE_1024
    L = 36 if base_name == "fib" else 30
    if alpha_frac == Fraction(15 + 2 * 5, 30):
        L = 130                                           # reach the integral rung 120
    q, k, v = randn(1, 4, L, 8), randn(1, 2, L, 8), randn(1, 2, L, 8)
    o_ref, lse_ref = brute_force_forward(q, k, v, alpha_frac, W, base)
    o, lse = O.forward(q, k, v, float(alpha_frac), W, base)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_forward_full_window_is_causal_attention():
    L = 40
    q, k, v = randn(2, 4, L, 16), randn(2, 2, L, 16), randn(2, 2, L, 16)
    causal = np.tril(np.ones((L, L), dtype=bool))
    ref = sdpa_masked(q, k, v, causal)
    for base in (O.FIB_BASE, O.POW2_BASE_1024):
        o, _ = O.forward(q, k, v, 1.0, L - 1, base)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # non-integral alpha adds synthetic blended keys, so it is not causal attention
    o, _ = O.forward(q, k, v, 0.7, L - 1, O.FIB_BASE)
    assert np.max(np.abs(o - ref)) > 1e-3


def test_interpolated_gather_reduces_exactly_to_the_integer_gather():
    x = randn(2, 3, 30, 8)
    valid = np.ones(30, dtype=bool)
    for a in [0, 1, 7, 29]:
        interp = O.gather(x, O.Slot("interp", a, 0.0, 1, valid))
        integer = O.gather(x, O.Slot("int", a, 0.0, 1, valid))
        assert np.array_equal(interp, integer)


def test_forward_is_continuous_as_alpha_approaches_an_integer():
    L = 60
    q, k, v = randn(1, 4, L, 8), randn(1, 2, L, 8), randn(1, 2, L, 8)
    o1, _ = O.forward(q, k, v, 2.0, 1, [3, 7])               # d = 6, 14 integral
    o2, _ = O.forward(q, k, v, 2.0 + 1e-7, 1, [3, 7])        # just past: interpolated
    # rows where the interpolated slot is valid (i >= a + 1) agree to first order in eps
    rows = np.arange(L) >= 15
    assert np.max(np.abs(o1[:, :, rows] - o2[:, :, rows])) < 1e-5
    # at i = a the interpolated slot needs row -1 and is masked, the integer one is not
    assert np.max(np.abs(o1[:, :, 6] - o2[:, :, 6])) > 1e-3


def test_first_row_is_its_own_value_and_zero_query_is_a_mean():
    L = 40
    q, k, v = randn(1, 4, L, 8), randn(1, 2, L, 8), randn(1, 2, L, 8)
    o, lse = O.forward(q, k, v, 0.8, 3, O.FIB_BASE)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h, 0], v[0, h // 2, 0])
    q0 = np.zeros_like(q)
    o0, lse0 = O.forward(q0, k, v, 1.0, 3, O.FIB_BASE)      # alpha = 1: plain rows
    for i in [0, 1, 5, 39]:
        dists = sorted({dd for dd in range(4) if dd <= i} | {f for f in O.FIB_BASE if 3 < f <= i})
        mean = np.mean([v[0, 0, i - dd] for dd in dists], axis=0)
        np.testing.assert_allclose(o0[0, 0, i], mean, atol=1e-13)
        assert abs(lse0[0, 0, i] - math.log(len(dists))) < 1e-13


def test_gqa_equals_repeated_key_value_heads():
    L = 50
    q, k, v = randn(2, 8, L, 16), randn(2, 2, L, 16), randn(2, 2, L, 16)
    o_gqa, l_gqa = O.forward(q, k, v, 0.9, 4, O.FIB_BASE)
    o_mha, l_mha = O.forward(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.9, 4, O.FIB_BASE)
    np.testing.assert_array_equal(o_gqa, o_mha)
    np.testing.assert_array_equal(l_gqa, l_mha)


def test_softmax_weights_sum_to_one_and_masked_slots_are_zero():
    L = 70
    q, k, v = randn(1, 2, L, 8), randn(1, 1, L, 8), randn(1, 1, L, 8)
    o, lse, P, sl = O.forward(q, k, v, 1.3, 5, O.FIB_BASE, return_probs=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    for n, s in enumerate(sl):
        assert np.all(P[..., ~s.valid, n] == 0.0)


# ------------------------------------------------------------------------------------------------
# Backward: central finite differences in float64
# ------------------------------------------------------------------------------------------------

def _loss(q, k, v, do, alpha, W, base):
    o, _ = O.forward(q, k, v, alpha, W, base)
    return float(np.sum(o * do))


@pytest.mark.parametrize("alpha,W,base", [(0.73, 2, O.FIB_BASE), (1.0, 3, O.FIB_BASE),
                                          (1.37, 1, O.POW2_BASE_1024)])
def test_backward_matches_central_differences(alpha, W, base):
    L, D = 16, 8
    q, k, v, do = randn(1, 4, L, D), randn(1, 2, L, D), randn(1, 2, L, D), randn(1, 4, L, D)
    dq, dk, dv, da = O.backward(q, k, v, do, alpha, W, base)
    h = 1e-6
    for x, g in [(q, dq), (k, dk), (v, dv)]:
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, alpha, W, base)
            x[idx] = old - h
            lm = _loss(q, k, v, do, alpha, W, base)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))
    if alpha != 1.0:
        fd_a = (_loss(q, k, v, do, alpha + h, W, base) - _loss(q, k, v, do, alpha - h, W, base)) / (2 * h)
        assert abs(fd_a - da) <= 1e-6 * max(1.0, abs(da))
    else:
        assert da == 0.0


def test_dtheta_of_every_layer_on_the_learned_workload_slice():
    # B = 1, L = 64 slice, 8 query / 2 key-value heads, head dim 64, W = 10, fib base
    import workloads
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    theta = workloads.draw_theta(16).numpy()
    for layer in range(16):
        q, k, v, do = [x.double().numpy() for x in workloads.draw(w, layer, B=1, L=64)]
        th = float(theta[layer])
        alpha = O.alpha_from_theta(th)
        _, _, _, da = O.backward(q, k, v, do, alpha, w.W, O.FIB_BASE)
        dth = da * O.dalpha_dtheta(th)
        h = 1e-6
        lp = _loss(q, k, v, do, O.alpha_from_theta(th + h), w.W, O.FIB_BASE)
        lm = _loss(q, k, v, do, O.alpha_from_theta(th - h), w.W, O.FIB_BASE)
        fd = (lp - lm) / (2 * h)
        assert abs(fd - dth) <= 1e-6 * max(1.0, abs(dth)), (layer, fd, dth)


def test_no_learned_offset_lands_on_an_integer():
    import workloads
    theta = workloads.draw_theta(16).numpy()
    for th in theta:
        alpha = O.alpha_from_theta(float(th))
        for f in O.FIB_BASE:
            d = alpha * f
            assert abs(d - round(d)) > 1e-6


# ------------------------------------------------------------------------------------------------
# Rounded-integer stagger (§2 "Implementation note": the fixed and staggered variants have integer
# offsets and can run through a fused boolean-mask path, numerically identical to the gather)
# ------------------------------------------------------------------------------------------------

# Worked by hand from the definition: alpha f_k rounded to the nearest integer, ties to even, the
# distinct values >= 1. alpha = 1/2: 0.5, 1, 1.5, 2.5, 4, 6.5, 10.5, 17, 27.5, 44.5, 72, 116.5,
# 188.5, 305, 493.5 (0 is the window's self slot; 1.5 and 2.5 both round to 2).
ROUNDED_FIB = {
    Fraction(1, 2): (1, 2, 4, 6, 10, 17, 28, 44, 72, 116, 188, 305, 494),
    Fraction(3, 2): (2, 3, 4, 8, 12, 20, 32, 51, 82, 134, 216, 350, 566, 915, 1480),
    Fraction(5, 6): (1, 2, 4, 7, 11, 18, 28, 46, 74, 120, 194, 314, 508, 822),   # ramp layer 5
    Fraction(1): (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987),
}


def exact_rounded(alpha_frac, base):
    """Round half to even on exact rationals; the distinct values >= 1."""
    out = set()
    for f in base:
        d = alpha_frac * f
        n = d.numerator // d.denominator
        rem = d - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        if n >= 1:
            out.add(n)
    return tuple(sorted(out))


@pytest.mark.parametrize("alpha_frac", list(ROUNDED_FIB))
def test_rounded_offsets_worked_examples(alpha_frac):
    assert exact_rounded(alpha_frac, O.FIB_BASE) == ROUNDED_FIB[alpha_frac]
    assert O.rounded_offsets(float(alpha_frac), O.FIB_BASE) == ROUNDED_FIB[alpha_frac]


def test_rounded_offsets_match_exact_rationals_on_every_static_schedule():
    # the float64 ramp values carry rounding error; ties such as (0.5 + 5/15) * 3 = 2.5 must still
    # be recognised
    for layer in range(16):
        lin = Fraction(15 + 2 * layer, 30)                       # 0.5 + l / 15
        cop = Fraction(15 + 2 * O.coprime_index(layer, 16), 30)
        for base in (O.FIB_BASE, O.POW2_BASE_1024):
            assert O.rounded_offsets(O.alpha_linear(layer, 16), base) == exact_rounded(lin, base)
            assert O.rounded_offsets(O.alpha_coprime(layer, 16), base) == exact_rounded(cop, base)
    assert O.rounded_offsets(O.alpha_fixed(0, 16), O.FIB_BASE) == O.FIB_BASE


@pytest.mark.parametrize("alpha_frac,W,L", [
    (Fraction(1, 2), 3, 40),      # rungs 1, 2 inside the window; 4, 6, 10, 17, 28 beyond it
    (Fraction(5, 6), 6, 48),      # ties 2.5 -> 2 and 17.5 -> 18
    (Fraction(3, 2), 8, 64),      # 4.5 -> 4, 7.5 -> 8 (a window distance), 19.5 -> 20, ...
    (Fraction(23, 30), 12, 72),   # ramp layer 4
])
def test_rounded_forward_equals_masked_dense_attention(alpha_frac, W, L):
    dists = O.rounded_offsets(float(alpha_frac), O.FIB_BASE)
    q, k, v = randn(1, 4, L, 16), randn(1, 2, L, 16), randn(1, 2, L, 16)
    ref = sdpa_masked(q, k, v, integer_mask(L, W, dists))
    o, _ = O.forward(q, k, v, 1.0, W, dists)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_rounded_backward_matches_central_differences():
    L, D, W = 16, 8, 2
    dists = O.rounded_offsets(0.5, O.FIB_BASE)                # 1, 2 dropped; 4, 6, 10 read
    q, k, v, do = randn(1, 4, L, D), randn(1, 2, L, D), randn(1, 2, L, D), randn(1, 4, L, D)
    dq, dk, dv, da = O.backward(q, k, v, do, 1.0, W, dists)
    assert da == 0.0
    h = 1e-6
    for x, g in [(q, dq), (k, dk), (v, dv)]:
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, 1.0, W, dists)
            x[idx] = old - h
            lm = _loss(q, k, v, do, 1.0, W, dists)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - g)) <= 1e-6 * max(1.0, np.max(np.abs(g)))
