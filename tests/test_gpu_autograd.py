"""GPU test of the torch.autograd wrapper (fibonacci_offset_sparse_amd.autograd) against the oracle.

loss = sum(o * do) through the wrapper gives q.grad, k.grad, v.grad and, for a learned layer,
theta.grad; they must equal the oracle's backward (d(theta) = d(alpha) * sigmoid'(theta)) at the
same bars as the direct calls.
"""

import sys

import pytest
import torch

import workloads
from oracle import fibattn_oracle as O
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ag():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fibonacci_offset_sparse_amd import autograd
    return autograd


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _leaves(tensors, dev):
    return [x.to(dev).requires_grad_(True) for x in tensors]


@pytest.mark.parametrize("layer", [2, 11])
def test_learned_layer_gradients(ag, layer):
    w = workloads.WORKLOADS["l1024_learned_bf16"]
    th = float(workloads.draw_theta(w.n_layers)[layer])
    q, k, v, do = workloads.draw(w, layer, B=2, L=400)
    dev = torch.device("cuda:0")
    qd, kd, vd = _leaves((q, k, v), dev)
    theta = torch.tensor(th, dtype=torch.float64, requires_grad=True)
    say(f"autograd learned layer {layer} theta={th!r}")
    o = ag.fib_attention(qd, kd, vd, w.W, O.FIB_BASE, theta=theta)
    (o.float() * do.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    n64 = [x.double().numpy() for x in (q, k, v, do)]
    alpha = O.alpha_from_theta(th)
    o_ref, _ = O.forward(*n64[:3], alpha, w.W, O.FIB_BASE)
    rq, rk, rv, ra = O.backward(*n64, alpha, w.W, O.FIB_BASE)
    check(o.detach().cpu(), o_ref, q.dtype, what="autograd o")
    check(qd.grad.cpu(), rq, q.dtype, what="autograd dq")
    check(kd.grad.cpu(), rk, q.dtype, what="autograd dk")
    check(vd.grad.cpu(), rv, q.dtype, what="autograd dv")
    ref_dth = ra * O.dalpha_dtheta(th)
    assert theta.grad is not None and theta.grad.device.type == "cpu"
    assert abs(float(theta.grad) - ref_dth) <= 1e-3 * abs(ref_dth), (float(theta.grad), ref_dth)


def test_static_layer_gradients_float32(ag):
    q, k, v, do = (workloads.randn_like_seeded(sh, 70 + i) for i, sh in
                   enumerate([(1, 8, 150, 64), (1, 2, 150, 64), (1, 2, 150, 64), (1, 8, 150, 64)]))
    dev = torch.device("cuda:0")
    qd, kd, vd = _leaves((q, k, v), dev)
    alpha = O.alpha_linear(4, 16)
    say("autograd static layer float32")
    o = ag.fib_attention(qd, kd, vd, 9, O.FIB_BASE, alpha=alpha)
    (o * do.to(dev)).sum().backward()
    torch.cuda.synchronize()
    n64 = [x.double().numpy() for x in (q, k, v, do)]
    rq, rk, rv, _ = O.backward(*n64, alpha, 9, O.FIB_BASE)
    check(qd.grad.cpu(), rq, torch.float32, what="autograd f32 dq")
    check(kd.grad.cpu(), rk, torch.float32, what="autograd f32 dk")
    check(vd.grad.cpu(), rv, torch.float32, what="autograd f32 dv")
