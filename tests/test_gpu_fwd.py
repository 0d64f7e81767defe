"""GPU parity of the forward pass against the float64 oracle (needs an MI355X).

Cases: every workload's layer calls at reduced sizes that span several tiles and a ragged tail,
every workload at full size (sampled batch elements, since rows of different batch elements never
mix), edge cases (tiny and ragged L, W = 0 and 31, no offsets, 32 offsets, GQA groups 1, 2, 8,
alphas that put every offset below one row or beyond L), NaN guard rows around K and V, bitwise
determinism and a non-default stream.
"""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import fibattn_oracle as O
from parity import check

pytestmark = pytest.mark.gpu

fa = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global fa
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fibonacci_offset_sparse_amd as m
    fa = m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def base_of(w):
    if w.base == "fib":
        return O.FIB_BASE
    return {1024: O.POW2_BASE_1024, 2048: O.POW2_BASE_2048}[workloads.pow2_max(w)]


def alphas_of(w):
    if w.schedule == "learned":
        return [O.alpha_from_theta(float(t)) for t in workloads.draw_theta(w.n_layers)]
    fn = {"fixed": O.alpha_fixed, "linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    return [fn(l, w.n_layers) for l in range(w.n_layers)]


def run_fwd(q, k, v, alpha, W, base, **kw):
    dev = torch.device("cuda:0")
    o, lse = fa.fibattn_fwd(q.to(dev), k.to(dev), v.to(dev), alpha, W, base, **kw)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare(q, k, v, alpha, W, base, what, bsel=None):
    o, lse = run_fwd(q, k, v, alpha, W, base)
    if bsel is not None:
        q, k, v, o, lse = q[bsel], k[bsel], v[bsel], o[bsel], lse[bsel]
    o_ref, lse_ref = O.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), alpha, W, base)
    check(o, o_ref, q.dtype, what=f"{what} o")
    check(lse, lse_ref, q.dtype, what=f"{what} lse", stored_bf16=False)


def test_tiny_workload():
    w = workloads.WORKLOADS["tiny_fixed_f32"]
    q, k, v, _ = workloads.draw(w, 0)
    say("tiny workload B=1 L=64 fp32 alpha=1 W=6")
    compare(q, k, v, 1.0, w.W, base_of(w), "tiny")


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_every_layer_at_reduced_size(name):
    w = workloads.WORKLOADS[name]
    base = base_of(w)
    for layer, alpha in enumerate(alphas_of(w)):
        B, L = (2, 200) if layer % 2 == 0 else (1, 1100)
        q, k, v = workloads.draw(w, layer, B=B, L=L, with_grad=False)
        say(f"{name} layer {layer} alpha={alpha!r} B={B} L={L}")
        compare(q, k, v, alpha, w.W, base, f"{name}/{layer}")


FULL = [n for n in workloads.WORKLOADS if n != "tiny_fixed_f32"]


@pytest.mark.parametrize("name,layer", [(n, l) for n in FULL for l in range(workloads.WORKLOADS[n].n_layers)])
def test_full_size_every_layer(name, layer):
    # every layer of every workload at its full shape, launched as the bench launches it (the whole
    # batch, so every far rung of the layer's alpha is staged at every length it reaches); one batch
    # element per layer is checked against the oracle (batch elements never mix), a different one
    # from layer to layer
    w = workloads.WORKLOADS[name]
    alpha = alphas_of(w)[layer]
    q, k, v = workloads.draw(w, layer, with_grad=False)
    b = (7 * layer + 3) % w.B
    say(f"{name} full size layer {layer} alpha={alpha!r} B={w.B} L={w.L}, checking batch {b}")
    compare(q, k, v, alpha, w.W, base_of(w), f"{name}/{layer}", bsel=[b])


@pytest.mark.parametrize("name", ["l1024_linear_bf16", "l4096_coprime_bf16", "l1024_pow2_linear_bf16"])
def test_rounded_stagger(name):
    # §2 "Implementation note": the static schedules with integer offsets (alpha f_k rounded, the
    # library's rounding checked against the oracle's), on the integer path at alpha = 1
    w = workloads.WORKLOADS[name]
    base = base_of(w)
    for layer, alpha in enumerate(alphas_of(w)):
        if layer % 3:
            continue
        dists = O.rounded_offsets(alpha, base)
        assert fa.fibattn_round_offsets(alpha, base) == dists
        B, L = (2, 300) if layer % 2 == 0 else (1, 1500)
        q, k, v = workloads.draw(w, layer, B=B, L=L, with_grad=False)
        say(f"rounded {name} layer {layer} alpha={alpha!r} B={B} L={L} offsets={dists}")
        compare(q, k, v, 1.0, w.W, dists, f"rounded {name}/{layer}")


def test_rounded_stagger_full_size_sampled_batches():
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    alpha = alphas_of(w)[7]
    dists = fa.fibattn_round_offsets(alpha, base_of(w))
    q, k, v = workloads.draw(w, 7, with_grad=False)
    say(f"rounded l1024_linear_bf16 layer 7 full size, offsets {dists}")
    compare(q, k, v, 1.0, w.W, dists, "rounded full size", bsel=[0, 15, 31])


def randn(shape, seed, dtype=torch.float32):
    return workloads.randn_like_seeded(shape, seed, dtype)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 129, 1000])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_lengths(L, dtype):
    q, k, v = randn((2, 8, L, 64), 1, dtype), randn((2, 2, L, 64), 2, dtype), randn((2, 2, L, 64), 3, dtype)
    say(f"ragged L={L} {dtype}")
    compare(q, k, v, 0.77, 5, O.FIB_BASE, f"L={L}")


@pytest.mark.parametrize("W,offsets,alpha", [
    (0, O.FIB_BASE, 1.0), (0, O.FIB_BASE, 0.61), (31, O.FIB_BASE, 1.0), (31, O.FIB_BASE, 1.13),
    (4, [], 1.0), (4, list(range(1, 33)), 1.0), (4, list(range(1, 33)), 0.93),
    (3, O.FIB_BASE, 0.001), (3, O.FIB_BASE, 10.5), (2, O.POW2_BASE_1024, 1.5),
])
def test_window_and_offset_extremes(W, offsets, alpha):
    L = 300
    q, k, v = randn((1, 8, L, 64), 4), randn((1, 2, L, 64), 5), randn((1, 2, L, 64), 6)
    say(f"W={W} K={len(offsets)} alpha={alpha}")
    compare(q, k, v, alpha, W, offsets, f"W={W} K={len(offsets)} a={alpha}")


# Integral plans (alpha = 1) in bf16, which the matrix-core kernels take on their integer-offset
# path: no rung within 64 rows, one, a group of four with rungs at 64 and 65 (the near block's
# last row and the first far one), two groups (the second partial), more than eight (the ninth
# goes to a far step), and a plan whose far steps do not fit that path (the interpolating kernels
# take it, with t = 0).
INT_PLANS = [
    (4, [70, 100, 150, 290]), (4, [10, 100, 150, 250, 290]), (2, [3, 5, 64, 65, 200]),
    (2, [3, 5, 8, 13, 21, 100, 200]), (0, list(range(1, 11)) + [64, 65, 66, 200]),
    (0, [1] + list(range(70, 85))),
]


@pytest.mark.parametrize("W,offsets", INT_PLANS)
@pytest.mark.parametrize("L", [300, 1100])
def test_integer_offset_plans(W, offsets, L):
    q, k, v = (randn((2, 8, L, 64), 61, torch.bfloat16), randn((2, 2, L, 64), 62, torch.bfloat16),
               randn((2, 2, L, 64), 63, torch.bfloat16))
    say(f"integral plan W={W} offsets={offsets} L={L}")
    compare(q, k, v, 1.0, W, offsets, f"int W={W} K={len(offsets)} L={L}")


@pytest.mark.parametrize("Hq,Hkv,L", [(16, 2, 300), (8, 2, 65), (4, 1, 130)])
def test_integer_offset_path_gqa_and_ragged(Hq, Hkv, L):
    # a group of 8 query heads (two workgroups per tile), a tail one row past a tile, one KV head
    q, k, v = (randn((1, Hq, L, 64), 64, torch.bfloat16), randn((1, Hkv, L, 64), 65, torch.bfloat16),
               randn((1, Hkv, L, 64), 66, torch.bfloat16))
    for W, offsets in ((2, [3, 5, 64, 65, 200]), (2, [3, 5, 8, 13, 21, 100, 200])):
        say(f"integral plan Hq={Hq} Hkv={Hkv} L={L} W={W} offsets={offsets}")
        compare(q, k, v, 1.0, W, offsets, f"int Hq={Hq} L={L} K={len(offsets)}")


def test_grid_order_covers_every_tile_once():
    # B = 20 at the paper's head counts: 40 (batch, KV head) units of 16 tiles, 80 workgroup slots
    # per XCD, so the grid order takes one row of 32 slots in launch order, the next in reverse and
    # leaves the last, partial row (16 slots) in order. Outputs start as NaN: a tile computed twice
    # or never shows in the comparison over every batch element.
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    q, k, v = workloads.draw(w, 6, B=20, L=1024, with_grad=False)
    dev = torch.device("cuda:0")
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    alpha = O.alpha_linear(6, 16)
    say("grid order: B=20 L=1024")
    fa.fibattn_fwd(q.to(dev), k.to(dev), v.to(dev), alpha, w.W, O.FIB_BASE, o=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), alpha, w.W, O.FIB_BASE)
    check(o.cpu(), o_ref, q.dtype, what="B=20 o")
    check(lse.cpu(), lse_ref, q.dtype, what="B=20 lse", stored_bf16=False)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (4, 2), (8, 1), (6, 2), (3, 3)])
def test_gqa_group_sizes(Hq, Hkv):
    L = 150
    q, k, v = randn((2, Hq, L, 64), 7), randn((2, Hkv, L, 64), 8), randn((2, Hkv, L, 64), 9)
    say(f"Hq={Hq} Hkv={Hkv}")
    compare(q, k, v, 0.88, 6, O.FIB_BASE, f"Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_nan_guard_rows_are_never_read(dtype):
    L, pad = 400, 4096
    dev = torch.device("cuda:0")
    q = randn((1, 8, L, 64), 10, dtype)
    k, v = randn((1, 1, L, 64), 11, dtype), randn((1, 1, L, 64), 12, dtype)
    q8 = q[:, :4].contiguous()
    guards = []
    for x in (k, v):
        buf = torch.full((2 * pad + L * 64,), float("nan"), dtype=dtype, device=dev)
        buf[pad:pad + L * 64] = x.reshape(-1).to(dev)
        guards.append(buf[pad:pad + L * 64].view(1, 1, L, 64))
    for alpha in (1.0, 0.71, 1.49):
        say(f"guard rows alpha={alpha} {dtype}")
        o, lse = fa.fibattn_fwd(q8.to(dev), guards[0], guards[1], alpha, 7, O.FIB_BASE)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        o_ref, _ = O.forward(q8.double().numpy(), k.double().numpy(), v.double().numpy(), alpha, 7, O.FIB_BASE)
        check(o.cpu(), o_ref, dtype, what=f"guard a={alpha}")


def test_bitwise_determinism_and_side_stream():
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    q, k, v = [x.to("cuda:0") for x in workloads.draw(w, 3, B=4, with_grad=False)]
    alpha = O.alpha_linear(3, 16)
    say("determinism B=4 L=1024 bf16")
    o1, l1 = fa.fibattn_fwd(q, k, v, alpha, w.W, O.FIB_BASE)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = fa.fibattn_fwd(q, k, v, alpha, w.W, O.FIB_BASE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_staged_entry_points_equal_the_combined_call():
    w = workloads.WORKLOADS["l4096_coprime_bf16"]
    q, k, v = [x.to("cuda:0") for x in workloads.draw(w, 5, B=1, with_grad=False)]
    alpha = O.alpha_coprime(5, 16)
    say("staged entry points B=1 L=4096")
    o1, l1 = fa.fibattn_fwd(q, k, v, alpha, w.W, O.FIB_BASE)
    ws = torch.empty(fa.fibattn_fwd_workspace_bytes(1, w.L, 2), dtype=torch.uint8, device="cuda:0")
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    fa.fibattn_fwd_prep(k, v, ws)
    fa.fibattn_fwd_attend(q, k, v, alpha, w.W, O.FIB_BASE, ws, o2, l2)
    fa.fibattn_fwd_attend(q, k, v, alpha, w.W, O.FIB_BASE, ws, o2, None)      # inference: no lse
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- inputs outside fp16's range: tiles whose rows fp16 cannot hold exactly enough are computed in
# float32 from the caller's bf16 rows (the prep's range flags, and each tile's own q rows) ----

def _scaled_case(scales, seed, L=300, W=7, alpha=0.83):
    q, k, v = (workloads.randn_like_seeded(sh, seed + i) * s for i, (sh, s) in
               enumerate(zip([(1, 8, L, 64), (1, 2, L, 64), (1, 2, L, 64)], scales)))
    return tuple(x.to(torch.bfloat16) for x in (q, k, v)) + (alpha, W)


@pytest.mark.parametrize("scales,W", [
    ((3e5, 3e-6, 3e5), 7),       # q and v far above fp16's range, scores of order 1
    ((3e-6, 3e5, 1.0), 7),       # k far above, q far below
    ((1e-6, 1e-6, 1e-6), 7),     # everything below fp16's normal range
    ((1.0, 1.0, 1e-6), 7),       # values only
    ((3e5, 3e-6, 3e5), 20),      # the general kernel (W > 15)
])
def test_inputs_outside_fp16_range(scales, W):
    q, k, v, alpha, W = _scaled_case(scales, 80, W=W)
    say(f"range q,k,v x {scales} W={W}")
    o, lse = run_fwd(q, k, v, alpha, W, O.FIB_BASE)
    o_ref, lse_ref = O.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), alpha, W, O.FIB_BASE)
    # bf16 outputs: each within 2^-8 of its own magnitude plus 1e-3 of the output's scale
    g, r = o.double().numpy(), o_ref
    assert np.all(np.isfinite(g))
    assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-3 * np.abs(r).max()), np.abs(g - r).max()
    # lse: the scores are of order 1 in every case; the log-normaliser shifts with log of the scale
    assert np.max(np.abs(lse.double().numpy() - lse_ref)) <= 1e-3 * max(1.0, np.abs(lse_ref).max())


def test_one_value_outside_fp16_range_in_a_row_few_queries_read():
    # one value element of 1e5 (fp16 would make it inf, and 0 * inf a NaN in every query whose
    # slots do not read that row but whose matrix products touch it): the tiles reading its block
    # compute in float32, the others on the matrix cores; every output is checked
    L = 300
    q, k, v = randn((1, 8, L, 64), 90, torch.bfloat16), randn((1, 2, L, 64), 91, torch.bfloat16), \
        randn((1, 2, L, 64), 92, torch.bfloat16)
    v[0, 1, 133, 17] = 1e5
    k[0, 0, 200:240] = 0                                  # zero rows (padding) stay on the matrix cores
    say("one value of 1e5 at row 133, zero key rows 200..239")
    o, lse = run_fwd(q, k, v, 0.91, 9, O.FIB_BASE)
    o_ref, lse_ref = O.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.91, 9, O.FIB_BASE)
    assert torch.isfinite(o.float()).all()
    check(o, o_ref, torch.bfloat16, what="one big value o")
    check(lse, lse_ref, torch.bfloat16, what="one big value lse", stored_bf16=False)
