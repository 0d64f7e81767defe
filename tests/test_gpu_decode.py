"""GPU parity of single-token decode against the float64 oracle (needs an MI355X).

The decode output of a sequence at position p is the forward pass's output row p over that
sequence's first p + 1 rows (§2 "Attended set"), so the oracle is its forward pass, read at that
row. Cases: every schedule's layers with ragged positions per sequence (cache rows past each
position hold NaN, so a stray read would show), the rounded-integer offsets, float32 storage at
1e-5, a position outside the cache, the paper's shape at full size on sampled sequences, and the
4x length shape with ragged positions.
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


def decode_case(q_full, k, v, positions, alpha, W, base, what, Lmax=None):
    """q_full, k, v: [B, H, L, D] CPU tensors; sequence b decodes its row positions[b]."""
    B, Hq, L, D = q_full.shape
    Lmax = L if Lmax is None else Lmax
    dev = torch.device("cuda:0")
    qd = torch.stack([q_full[b, :, positions[b]] for b in range(B)]).contiguous()
    kc = torch.full((B, k.shape[1], Lmax, D), float("nan"), dtype=k.dtype)
    vc = torch.full_like(kc, float("nan"))
    for b in range(B):
        kc[b, :, : positions[b] + 1] = k[b, :, : positions[b] + 1]
        vc[b, :, : positions[b] + 1] = v[b, :, : positions[b] + 1]
    pos = torch.tensor(positions, dtype=torch.int32)
    o, lse = fa.fibattn_decode(qd.to(dev), kc.to(dev), vc.to(dev), pos.to(dev), alpha, W, base)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b in range(B):
        p = positions[b]
        n64 = [x[b:b + 1, :, : p + 1].double().numpy() for x in (q_full, k, v)]
        o_ref, lse_ref = O.forward(*n64, alpha, W, base)
        check(o[b:b + 1], o_ref[:, :, p], q_full.dtype, what=f"{what} b={b} pos={p} o")
        check(lse[b:b + 1], lse_ref[:, :, p], q_full.dtype, what=f"{what} b={b} pos={p} lse", stored_bf16=False)
    return o, lse


def alphas_of(w):
    if w.schedule == "learned":
        return [O.alpha_from_theta(float(t)) for t in workloads.draw_theta(w.n_layers)]
    fn = {"fixed": O.alpha_fixed, "linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    return [fn(l, w.n_layers) for l in range(w.n_layers)]


@pytest.mark.parametrize("name", ["l1024_linear_bf16", "l1024_learned_bf16", "l1024_pow2_fixed_bf16",
                                  "l4096_coprime_bf16"])
def test_ragged_positions(name):
    w = workloads.WORKLOADS[name]
    base = O.FIB_BASE if w.base == "fib" else {1024: O.POW2_BASE_1024, 2048: O.POW2_BASE_2048}[workloads.pow2_max(w)]
    L = min(w.L, 1600)
    positions = [L - 1, 0, 517, 64, 13]
    for layer in (0, 7, 15):
        alpha = alphas_of(w)[layer]
        q, k, v = workloads.draw(w, layer, B=len(positions), L=L, with_grad=False)
        say(f"decode {name} layer {layer} alpha={alpha!r} positions={positions}")
        decode_case(q, k, v, positions, alpha, w.W, base, f"{name}/{layer}")


def test_rounded_integer_offsets():
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    for layer in (0, 5, 15):
        dists = O.rounded_offsets(O.alpha_linear(layer, 16), O.FIB_BASE)
        q, k, v = workloads.draw(w, layer, B=3, L=1024, with_grad=False)
        say(f"decode rounded layer {layer} offsets {dists}")
        decode_case(q, k, v, [1023, 700, 31], 1.0, w.W, dists, f"rounded/{layer}")


def test_float32_storage():
    w = workloads.WORKLOADS["tiny_fixed_f32"]
    q, k, v, _ = workloads.draw(w, 0)
    say("decode tiny fp32")
    decode_case(q, k, v, [63], 1.0, w.W, O.FIB_BASE, "tiny f32")
    qf, kf, vf = (workloads.randn_like_seeded((2, 8, 300, 64), s, torch.float32) for s in (71, 72, 73))
    qf, kf, vf = qf, kf[:, :2].contiguous(), vf[:, :2].contiguous()
    decode_case(qf, kf, vf, [299, 150], 0.73, 9, O.FIB_BASE, "f32 interpolated")


def test_window_and_offset_extremes():
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    q, k, v = workloads.draw(w, 3, B=2, L=400, with_grad=False)
    say("decode W=0 / W=31 / 32 offsets / none")
    decode_case(q, k, v, [399, 200], 1.21, 0, O.FIB_BASE, "W=0")
    decode_case(q, k, v, [399, 30], 0.9, 31, O.FIB_BASE, "W=31")
    decode_case(q, k, v, [399, 5], 1.0, 4, list(range(1, 33)), "32 offsets")
    decode_case(q, k, v, [399, 0], 1.0, 7, [], "no offsets")


def test_position_outside_the_cache_gives_nan():
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    q, k, v = workloads.draw(w, 1, B=2, L=128, with_grad=False)
    dev = torch.device("cuda:0")
    qd = q[:, :, 100].contiguous().to(dev)
    pos = torch.tensor([100, 128], dtype=torch.int32, device=dev)     # 128 = Lmax: outside
    o, lse = fa.fibattn_decode(qd, k.to(dev), v.to(dev), pos, 0.8, w.W, O.FIB_BASE)
    torch.cuda.synchronize()
    assert torch.isnan(o[1].float()).all() and torch.isnan(lse[1]).all()
    assert torch.isfinite(o[0].float()).all() and torch.isfinite(lse[0]).all()


def test_full_size_paper_shape_sampled_sequences():
    # B = 32 sequences of a 1024-row cache, every sequence at the last position; sampled check
    w = workloads.WORKLOADS["l1024_linear_bf16"]
    q, k, v = workloads.draw(w, 11, with_grad=False)
    B = q.shape[0]
    dev = torch.device("cuda:0")
    pos = torch.full((B,), w.L - 1, dtype=torch.int32, device=dev)
    qd = q[:, :, w.L - 1].contiguous()
    alpha = O.alpha_linear(11, 16)
    say(f"decode full size B={B} pos={w.L - 1}")
    o, lse = fa.fibattn_decode(qd.to(dev), k.to(dev), v.to(dev), pos, alpha, w.W, O.FIB_BASE)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b in (0, 17, 31):
        n64 = [x[b:b + 1].double().numpy() for x in (q, k, v)]
        o_ref, lse_ref = O.forward(*n64, alpha, w.W, O.FIB_BASE)
        check(o[b:b + 1], o_ref[:, :, -1], q.dtype, what=f"full b={b} o")
        check(lse[b:b + 1], lse_ref[:, :, -1], q.dtype, what=f"full b={b} lse", stored_bf16=False)


def test_long_shape_ragged_positions():
    # the 4x length shape: B = 8 sequences of a 4096-row cache, each at its own position (the
    # coprime stagger's layer with the largest alpha, whose rungs reach 1481 rows back)
    w = workloads.WORKLOADS["l4096_coprime_bf16"]
    layer = max(range(w.n_layers), key=lambda l: O.alpha_coprime(l, w.n_layers))
    alpha = O.alpha_coprime(layer, w.n_layers)
    q, k, v = workloads.draw(w, layer, with_grad=False)
    positions = [w.L - 1, 3000, 1481, 1480, 700, 64, 1, 0]
    say(f"decode l4096_coprime_bf16 layer {layer} alpha={alpha!r} positions={positions}")
    decode_case(q, k, v, positions, alpha, w.W, O.FIB_BASE, "l4096 decode")
