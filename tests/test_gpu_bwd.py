"""GPU parity of the backward pass against the float64 oracle (needs an MI355X).

dq, dk, dv per element; d(alpha) and d(theta) per layer. Cases: the tiny workload (integral
offsets, no d(alpha)), float32 interpolated cases, every layer of the learned-alpha workload at a
reduced size, the learned workload at full size (sampled batch elements for dq/dk/dv, the full
batch for d(theta)), the bench's two shapes at full size, GQA group sizes, ragged lengths, and
bitwise determinism.
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


# d(alpha) and d(theta): relative error against the oracle, 1e-5 for float32 storage and 1e-3 for
# bfloat16 storage. The scalar sums every (position, head, rung) term with heavy cancellation; a
# call that asks for it takes its scores from split (high + low fp16) q and keys.
DALPHA_RTOL = {torch.float32: 1e-5, torch.bfloat16: 1e-3}


def run(q, k, v, do, alpha, W, base, want_dalpha, dadt=0.0):
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.fibattn_fwd(q, k, v, alpha, W, base)
    dq, dk, dv, da, dth = fa.fibattn_bwd(q, k, v, o, lse, do, alpha, W, base, dalpha_dtheta=dadt,
                                         want_dalpha=want_dalpha)
    torch.cuda.synchronize()
    out = [dq.cpu(), dk.cpu(), dv.cpu()]
    out += [float(da.item()) if da is not None else None, float(dth.item()) if dth is not None else None]
    return out


def compare(q, k, v, do, alpha, W, base, what, want_dalpha=True, bsel=None, dadt=0.0):
    dq, dk, dv, da, dth = run(q, k, v, do, alpha, W, base, want_dalpha, dadt)
    n64 = [x.double().numpy() for x in (q, k, v, do)]
    if bsel is not None:
        n64 = [x[bsel] for x in n64]
        dq, dk, dv = dq[bsel], dk[bsel], dv[bsel]
    rq, rk, rv, ra = O.backward(*n64, alpha, W, base)
    check(dq, rq, q.dtype, what=f"{what} dq")
    check(dk, rk, q.dtype, what=f"{what} dk")
    check(dv, rv, q.dtype, what=f"{what} dv")
    if want_dalpha and bsel is None:
        tol = DALPHA_RTOL[q.dtype]
        assert abs(da - ra) <= tol * max(abs(ra), 1e-3), f"{what} dalpha {da} vs {ra}"
        if dadt:
            assert abs(dth - ra * dadt) <= tol * max(abs(ra * dadt), 1e-3), f"{what} dtheta {dth} vs {ra * dadt}"
    return da


def randn(shape, seed, dtype=torch.float32):
    return workloads.randn_like_seeded(shape, seed, dtype)


def test_tiny_workload_integral_offsets():
    w = workloads.WORKLOADS["tiny_fixed_f32"]
    q, k, v, do = workloads.draw(w, 0)
    say("bwd tiny workload fp32 alpha=1")
    compare(q, k, v, do, 1.0, w.W, O.FIB_BASE, "tiny", want_dalpha=False)


@pytest.mark.parametrize("alpha,W,L", [(0.73, 6, 64), (1.21, 3, 200), (0.5 + 1e-3, 12, 130), (1.49, 10, 1100)])
def test_fp32_interpolated(alpha, W, L):
    q, k, v, do = randn((2, 8, L, 64), 21), randn((2, 2, L, 64), 22), randn((2, 2, L, 64), 23), randn((2, 8, L, 64), 24)
    say(f"bwd fp32 alpha={alpha} W={W} L={L}")
    compare(q, k, v, do, alpha, W, O.FIB_BASE, f"a={alpha}")


def test_learned_workload_every_layer_reduced():
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    theta = workloads.draw_theta(w.n_layers).tolist()
    for layer, th in enumerate(theta):
        alpha, dadt = O.alpha_from_theta(th), O.dalpha_dtheta(th)
        B, L = (2, 200) if layer % 2 == 0 else (1, 1100)
        q, k, v, do = workloads.draw(w, layer, B=B, L=L)
        say(f"bwd learned layer {layer} theta={th!r} B={B} L={L}")
        compare(q, k, v, do, alpha, w.W, O.FIB_BASE, f"learned/{layer}", dadt=dadt)


@pytest.mark.parametrize("layer", [0, 9])
def test_learned_workload_full_size(layer):
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    th = float(workloads.draw_theta(w.n_layers)[layer])
    alpha, dadt = O.alpha_from_theta(th), O.dalpha_dtheta(th)
    q, k, v, do = workloads.draw(w, layer)
    say(f"bwd learned full size layer {layer} B={w.B} L={w.L}")
    # dq, dk, dv on three batch elements (batch elements never mix)
    compare(q, k, v, do, alpha, w.W, O.FIB_BASE, f"full/{layer}", bsel=[0, w.B // 2, w.B - 1], dadt=dadt)
    # d(alpha) is a sum over the batch: the oracle's per-element sums added up
    dq, dk, dv, da, dth = run(q, k, v, do, alpha, w.W, O.FIB_BASE, True, dadt)
    ref = 0.0
    for b in range(w.B):
        ref += O.backward(*[x[b:b + 1].double().numpy() for x in (q, k, v, do)], alpha, w.W, O.FIB_BASE)[3]
    tol = DALPHA_RTOL[q.dtype]
    assert abs(da - ref) <= tol * abs(ref), (da, ref)
    assert abs(dth - ref * dadt) <= tol * abs(ref * dadt), (dth, ref * dadt)


ALPHA_FN = {"linear": O.alpha_linear, "coprime": O.alpha_coprime}


@pytest.mark.parametrize("name,layer", [(n, l) for n in ("l1024_learned_bf16", "l1024_linear_bf16", "l4096_coprime_bf16")
                                        for l in range(16)])
def test_full_size_every_layer(name, layer):
    # every layer of the learned workload and of the bench's two shapes at full size, in the
    # bench's launch configuration; dq, dk, dv on one batch element per layer (a different one
    # from layer to layer). d(alpha) is asked for on the learned layers (every rung interpolated),
    # so their backward runs the precise-score query side; its sum over the whole batch is checked
    # at full size in test_learned_workload_full_size.
    w = workloads.WORKLOADS[name]
    if w.schedule == "learned":
        th = float(workloads.draw_theta(w.n_layers)[layer])
        alpha, dadt, want = O.alpha_from_theta(th), O.dalpha_dtheta(th), True
    else:
        alpha, dadt, want = ALPHA_FN[w.schedule](layer, w.n_layers), 0.0, False
    q, k, v, do = workloads.draw(w, layer, with_grad=True)
    b = (5 * layer + 1) % w.B
    say(f"bwd {name} full size layer {layer} alpha={alpha!r} B={w.B} L={w.L}, checking batch {b}")
    compare(q, k, v, do, alpha, w.W, O.FIB_BASE, f"{name}/{layer}", want_dalpha=want, bsel=[b], dadt=dadt)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_guard_rows_are_never_read(dtype):
    # q, k, v and do each sit between NaN rows (4096 elements on either side): a read before the
    # first or past the last row of any of them shows as a non-finite gradient
    L, pad = 300, 4096
    dev = torch.device("cuda:0")
    shapes = {"q": (1, 4, L, 64), "k": (1, 1, L, 64), "v": (1, 1, L, 64), "do": (1, 4, L, 64)}
    host = {n: randn(sh, 60 + i, dtype) for i, (n, sh) in enumerate(shapes.items())}
    dev_t = {}
    for n, x in host.items():
        buf = torch.full((2 * pad + x.numel(),), float("nan"), dtype=dtype, device=dev)
        buf[pad:pad + x.numel()] = x.reshape(-1).to(dev)
        dev_t[n] = buf[pad:pad + x.numel()].view(x.shape)
    n64 = [host[n].double().numpy() for n in ("q", "k", "v", "do")]
    for alpha, want in ((1.0, False), (0.71, True), (1.49, True)):
        say(f"bwd guard rows alpha={alpha} {dtype}")
        dq, dk, dv, da, _ = fa.fibattn_bwd(dev_t["q"], dev_t["k"], dev_t["v"], None, None, dev_t["do"], alpha, 7,
                                           O.FIB_BASE, want_dalpha=want)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert torch.isfinite(t.float()).all()
        rq, rk, rv, ra = O.backward(*n64, alpha, 7, O.FIB_BASE)
        check(dq.cpu(), rq, dtype, what=f"guard a={alpha} dq")
        check(dk.cpu(), rk, dtype, what=f"guard a={alpha} dk")
        check(dv.cpu(), rv, dtype, what=f"guard a={alpha} dv")
        if want:
            assert abs(float(da.item()) - ra) <= DALPHA_RTOL[dtype] * abs(ra), (float(da.item()), ra)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (6, 2)])
def test_gqa_group_sizes(Hq, Hkv):
    L = 150
    q, k, v, do = randn((1, Hq, L, 64), 31), randn((1, Hkv, L, 64), 32), randn((1, Hkv, L, 64), 33), randn((1, Hq, L, 64), 34)
    say(f"bwd Hq={Hq} Hkv={Hkv}")
    compare(q, k, v, do, 0.83, 4, O.FIB_BASE, f"Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("L", [1, 65, 333])
def test_ragged_lengths_bf16(L):
    d = torch.bfloat16
    q, k, v, do = randn((2, 8, L, 64), 41, d), randn((2, 2, L, 64), 42, d), randn((2, 2, L, 64), 43, d), randn((2, 8, L, 64), 44, d)
    say(f"bwd ragged L={L}")
    compare(q, k, v, do, 0.67, 9, O.FIB_BASE, f"L={L}")


def test_integral_offsets_with_pow2_base_and_window_extremes():
    L = 260
    q, k, v, do = randn((1, 8, L, 64), 51), randn((1, 2, L, 64), 52), randn((1, 2, L, 64), 53), randn((1, 8, L, 64), 54)
    say("bwd pow2 alpha=1 W=0 / W=31 / no offsets")
    compare(q, k, v, do, 1.0, 0, O.POW2_BASE_1024, "pow2 W=0", want_dalpha=False)
    compare(q, k, v, do, 1.0, 31, O.FIB_BASE, "fib W=31", want_dalpha=False)
    compare(q, k, v, do, 1.0, 5, [], "no offsets", want_dalpha=False)


# Integral plans (alpha = 1) in bf16 on the matrix-core kernels' integer-offset path: no rung
# within 64 rows, one, rungs at 64 and 65 (the near block's last row and the first far one), two
# groups of four (the second partial), more than eight, and a plan whose far steps do not fit that
# path (the interpolating kernels take it, with t = 0).
INT_PLANS = [
    (4, [70, 100, 150, 290]), (4, [10, 100, 150, 250, 290]), (2, [3, 5, 64, 65, 200]),
    (2, [3, 5, 8, 13, 21, 100, 200]), (0, list(range(1, 11)) + [64, 65, 66, 200]),
    (0, [1] + list(range(70, 85))),
]


@pytest.mark.parametrize("W,offsets", INT_PLANS)
@pytest.mark.parametrize("L", [300, 1100])
def test_integer_offset_plans(W, offsets, L):
    B = 2 if L <= 300 else 1
    q, k, v, do = (randn((B, 8, L, 64), 71, torch.bfloat16), randn((B, 2, L, 64), 72, torch.bfloat16),
                   randn((B, 2, L, 64), 73, torch.bfloat16), randn((B, 8, L, 64), 74, torch.bfloat16))
    say(f"bwd integral plan W={W} offsets={offsets} L={L}")
    compare(q, k, v, do, 1.0, W, offsets, f"int W={W} K={len(offsets)} L={L}", want_dalpha=False)


@pytest.mark.parametrize("Hq,Hkv,L", [(16, 2, 300), (8, 2, 65), (4, 1, 130)])
def test_integer_offset_path_gqa_and_ragged(Hq, Hkv, L):
    q, k, v, do = (randn((1, Hq, L, 64), 75, torch.bfloat16), randn((1, Hkv, L, 64), 76, torch.bfloat16),
                   randn((1, Hkv, L, 64), 77, torch.bfloat16), randn((1, Hq, L, 64), 78, torch.bfloat16))
    for W, offsets in ((2, [3, 5, 64, 65, 200]), (2, [3, 5, 8, 13, 21, 100, 200])):
        say(f"bwd integral plan Hq={Hq} Hkv={Hkv} L={L} W={W} offsets={offsets}")
        compare(q, k, v, do, 1.0, W, offsets, f"int Hq={Hq} L={L} K={len(offsets)}", want_dalpha=False)


@pytest.mark.parametrize("name", ["l1024_linear_bf16", "l4096_coprime_bf16"])
def test_rounded_stagger(name):
    # the integer path at alpha = 1 with the rounded offsets of §2 "Implementation note"; d(alpha)
    # is not defined there (integral offsets)
    w = workloads.WORKLOADS[name]
    fn = {"linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    for layer in (0, 7, 15):
        dists = fa.fibattn_round_offsets(fn(layer, 16), O.FIB_BASE)
        B, L = (2, 300) if layer != 7 else (1, 1500)
        q, k, v, do = workloads.draw(w, layer, B=B, L=L, with_grad=True)
        say(f"bwd rounded {name} layer {layer} B={B} L={L} offsets={dists}")
        compare(q, k, v, do, 1.0, w.W, dists, f"rounded {name}/{layer}", want_dalpha=False)


@pytest.mark.parametrize("name,layer", [("l4096_pow2_2048_linear_bf16", 9), ("l4096_w6_coprime_bf16", 4)])
def test_long_workload_variants(name, layer):
    # the power-of-two base grown to 2048 and a narrower window at the 4x length shape; L reaches
    # the largest rungs
    w = workloads.WORKLOADS[name]
    base = O.POW2_BASE_2048 if w.base == "pow2_2048" else O.FIB_BASE
    fn = {"linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    q, k, v, do = workloads.draw(w, layer, B=1, L=2600, with_grad=True)
    say(f"bwd {name} layer {layer} B=1 L=2600")
    compare(q, k, v, do, fn(layer, 16), w.W, base, f"{name}/{layer}", want_dalpha=False)


def test_staged_calls_equal_the_combined_call():
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    q, k, v, do = [x.to("cuda:0") for x in workloads.draw(w, 3, B=2)]
    th = float(workloads.draw_theta(16)[3])
    alpha, dadt = O.alpha_from_theta(th), O.dalpha_dtheta(th)
    say("bwd staged calls B=2 L=1024")
    ref = fa.fibattn_bwd(q, k, v, None, None, do, alpha, w.W, O.FIB_BASE, dalpha_dtheta=dadt, want_dalpha=True)
    ws = torch.empty(fa.fibattn_bwd_workspace_bytes(2, w.L, 8, 2, 64, w.W, len(O.FIB_BASE)), dtype=torch.uint8,
                     device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    da, dth = torch.empty(1, device="cuda:0"), torch.empty(1, device="cuda:0")
    for st in (fa.STAGE_PREP, fa.STAGE_QUERY, fa.STAGE_KEY):
        fa.fibattn_bwd_stages(st, q, k, v, do, alpha, w.W, O.FIB_BASE, dq, dk, dv, ws, dalpha_dtheta=dadt,
                              dalpha=da, dtheta=dth)
    torch.cuda.synchronize()
    for x, y in zip(ref, (dq, dk, dv, da, dth)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_after_forward_skips_its_prep(dtype):
    # the forward's prep in the shared workspace stands in for the backward's own: same bits
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    q, k, v, do = [x.to("cuda:0", dtype) for x in workloads.draw(w, 5, B=2)]
    th = float(workloads.draw_theta(16)[5])
    alpha, dadt = O.alpha_from_theta(th), O.dalpha_dtheta(th)
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    dt = fa.BF16 if dtype == torch.bfloat16 else fa.F32
    assert fa.fibattn_bwd_reuses_fwd_prep(alpha, w.W, O.FIB_BASE, B, L, Hq, Hkv, D, dt)
    say(f"bwd after fwd without prep {dtype} B=2 L=1024")
    ref = fa.fibattn_bwd(q, k, v, None, None, do, alpha, w.W, O.FIB_BASE, dalpha_dtheta=dadt, want_dalpha=True)
    nbytes = max(fa.fibattn_fwd_workspace_bytes(B, L, Hkv, D, dt),
                 fa.fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, w.W, len(O.FIB_BASE), dt))
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda:0")
    fa.fibattn_fwd(q, k, v, alpha, w.W, O.FIB_BASE, workspace=ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    da, dth = torch.empty(1, device="cuda:0"), torch.empty(1, device="cuda:0")
    fa.fibattn_bwd_stages(fa.STAGE_QUERY | fa.STAGE_KEY, q, k, v, do, alpha, w.W, O.FIB_BASE, dq, dk, dv, ws,
                          dalpha_dtheta=dadt, dalpha=da, dtheta=dth)
    torch.cuda.synchronize()
    for x, y in zip(ref, (dq, dk, dv, da, dth)):
        assert torch.equal(x, y)


def test_bitwise_determinism():
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    q, k, v, do = workloads.draw(w, 2, B=4)
    alpha = O.alpha_from_theta(float(workloads.draw_theta(16)[2]))
    say("bwd determinism B=4 L=1024")
    a = run(q, k, v, do, alpha, w.W, O.FIB_BASE, True)
    b = run(q, k, v, do, alpha, w.W, O.FIB_BASE, True)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert a[3] == b[3]


def test_maximum_length_sampled_rows():
    # L = 2^20 (the largest the library takes), one sequence, 4 query heads on one key-value head:
    # every offset computation at its largest. Outputs at row c depend only on rows within the
    # reach (1382 here; under 1500 for any alpha <= 1.5), and RoPE scores only on relative
    # positions, so the oracle runs on a slice around c: dq at c needs keys c - 1382 .. c, dk and
    # dv at c need queries c .. c + 1382.
    L, B, Hq, Hkv, D = 1 << 20, 1, 4, 1, 64
    alpha, W = 1.4, 12
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(2024)
    q, k, v, do = (torch.randn(B, h, L, D, generator=g).to(torch.bfloat16) for h in (Hq, Hkv, Hkv, Hq))
    say(f"max length L={L}: forward + backward")
    dq, dk, dv, _, _ = fa.fibattn_bwd(q.to(dev), k.to(dev), v.to(dev), None, None, do.to(dev), alpha, W, O.FIB_BASE)
    o, _ = fa.fibattn_fwd(q.to(dev), k.to(dev), v.to(dev), alpha, W, O.FIB_BASE)
    torch.cuda.synchronize()
    dq, dk, dv, o = dq.cpu(), dk.cpu(), dv.cpu(), o.cpu()
    for c in (5000, L // 2 + 77, L - 1600):
        s0, s1 = c - 1500, min(L, c + 1500)
        n64 = [x[:, :, s0:s1].double().numpy() for x in (q, k, v, do)]
        o_ref, _ = O.forward(*n64[:3], alpha, W, O.FIB_BASE)
        rq, rk, rv, _ = O.backward(*n64, alpha, W, O.FIB_BASE)
        r = c - s0
        check(o[:, :, c], o_ref[:, :, r], q.dtype, what=f"L=2^20 row {c} o")
        check(dq[:, :, c], rq[:, :, r], q.dtype, what=f"L=2^20 row {c} dq")
        check(dk[:, :, c], rk[:, :, r], q.dtype, what=f"L=2^20 row {c} dk")
        check(dv[:, :, c], rv[:, :, r], q.dtype, what=f"L=2^20 row {c} dv")
    # decode of the last position against the same slice rule
    pos = torch.tensor([L - 1], dtype=torch.int32, device=dev)
    od, _ = fa.fibattn_decode(q[:, :, L - 1].contiguous().to(dev), k.to(dev), v.to(dev), pos, alpha, W, O.FIB_BASE)
    torch.cuda.synchronize()
    n64 = [x[:, :, L - 3000:].double().numpy() for x in (q, k, v)]
    o_ref, _ = O.forward(*n64, alpha, W, O.FIB_BASE)
    check(od.cpu(), o_ref[:, :, -1], q.dtype, what="L=2^20 decode")


# ---- inputs and gradients far from the unit scale: q and do are carried as row / 2^e in fp16
# (exact power-of-two scaling, undone in float32), the query side's hand-off to the key side per
# tile likewise; tiles that read key or value rows outside fp16's range are computed in float32 ----

def _close(gpu, ref, what):
    # bf16 outputs: within 2^-8 of their own magnitude plus 2e-3 of the tensor's scale
    g, r = gpu.double().numpy(), ref
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    bound = 2.0 ** -8 * np.abs(r) + 2e-3 * np.abs(r).max()
    assert np.all(np.abs(g - r) <= bound), f"{what}: max excess {np.max(np.abs(g - r) - bound):.3e} (scale {np.abs(r).max():.3e})"


@pytest.mark.parametrize("scales", [
    (1.0, 1.0, 1.0, 2.0 ** -20),     # gradients of a loss averaged over many tokens
    (1.0, 1.0, 1.0, 2.0 ** 20),
    (3e5, 3e-6, 1.0, 1.0),           # q far above fp16's range (k far below: the float32 tiles)
    (1.0, 1.0, 3e5, 2.0 ** -10),     # values far above
    (1e-6, 1e-6, 1e-6, 1e-6),        # everything far below
])
def test_inputs_and_gradients_far_from_unit_scale(scales):
    L = 300
    sh = [(1, 8, L, 64), (1, 2, L, 64), (1, 2, L, 64), (1, 8, L, 64)]
    q, k, v, do = ((workloads.randn_like_seeded(s_, 110 + i) * f).to(torch.bfloat16) for i, (s_, f) in
                   enumerate(zip(sh, scales)))
    th = 0.37
    alpha, dadt = O.alpha_from_theta(th), O.dalpha_dtheta(th)
    say(f"bwd scales q,k,v,do x {scales}")
    dq, dk, dv, da, dth = run(q, k, v, do, alpha, 9, O.FIB_BASE, True, dadt)
    n64 = [x.double().numpy() for x in (q, k, v, do)]
    rq, rk, rv, ra = O.backward(*n64, alpha, 9, O.FIB_BASE)
    _close(dq, rq, "dq")
    _close(dk, rk, "dk")
    _close(dv, rv, "dv")
    assert abs(da - ra) <= 1e-3 * abs(ra), (da, ra)
    assert abs(dth - ra * dadt) <= 1e-3 * abs(ra * dadt), (dth, ra * dadt)


def test_one_value_outside_fp16_range_backward():
    # one value element of 1e5 at row 211 of KV head 1: the query tiles that read its block take the
    # float32 tile, the others the matrix cores; their hand-offs to the key side (scaled per tile)
    # meet in the key rows both reach
    L = 400
    q, k, v, do = (randn(s_, 120 + i, torch.bfloat16) for i, s_ in
                   enumerate([(2, 8, L, 64), (2, 2, L, 64), (2, 2, L, 64), (2, 8, L, 64)]))
    v[1, 1, 211, 5] = 1e5
    say("bwd one value of 1e5")
    compare(q, k, v, do, 0.77, 8, O.FIB_BASE, "one big value", want_dalpha=False)
