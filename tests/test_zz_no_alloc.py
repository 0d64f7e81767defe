"""GPU test of the allocation-free forward (fibattn_fwd_noalloc) against fibattn_fwd.

The entry point runs the same kernels with its workspace in the library's device array: two calls
in a row (the second smaller, so the array holds the first call's rows beyond what the second
writes) must each equal fibattn_fwd on the same inputs bit for bit, and meet the oracle's bar; a
call needing more than the array holds is refused before anything is queued.
"""

import sys

import pytest
import torch

import workloads
from oracle import fibattn_oracle as O
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fibonacci_offset_sparse_amd as m
    return m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(fa, name, layer, B, L, check_oracle_batch):
    w = workloads.WORKLOADS[name]
    fn = {"linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    alpha = fn(layer, w.n_layers)
    q, k, v = workloads.draw(w, layer, B=B, L=L, with_grad=False)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    need = fa.fibattn_fwd_workspace_bytes(B, L, w.Hkv)
    assert need <= fa.fibattn_fwd_noalloc_max_bytes()
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    say(f"allocation-free forward {name} layer {layer} B={B} L={L} ({need} bytes of scratch)")
    fa.fibattn_fwd_noalloc(qd, kd, vd, alpha, w.W, O.FIB_BASE, o, lse)
    o_ref, lse_ref = fa.fibattn_fwd(qd, kd, vd, alpha, w.W, O.FIB_BASE)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    b = check_oracle_batch
    r_o, r_lse = O.forward(q[b:b + 1].double().numpy(), k[b:b + 1].double().numpy(), v[b:b + 1].double().numpy(),
                           alpha, w.W, O.FIB_BASE)
    check(o[b:b + 1].cpu(), r_o, q.dtype, what="noalloc o")
    check(lse[b:b + 1].cpu(), r_lse, q.dtype, what="noalloc lse", stored_bf16=False)


def test_noalloc_forward_equals_fibattn_fwd_on_two_calls(fa):
    # the paper's shape (16.25 MiB of scratch), then a smaller, ragged call
    _case(fa, "l1024_linear_bf16", 5, 32, 1024, check_oracle_batch=17)
    _case(fa, "l4096_coprime_bf16", 9, 1, 777, check_oracle_batch=0)


def test_noalloc_forward_refuses_a_call_beyond_its_array(fa):
    dev = torch.device("cuda:0")
    B, L = 4, 16384                                      # 32 MiB + the table: over the array
    assert fa.fibattn_fwd_workspace_bytes(B, L, 2) > fa.fibattn_fwd_noalloc_max_bytes()
    q = torch.zeros(B, 8, L, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, 2, L, 64, dtype=torch.bfloat16, device=dev)
    o = torch.full_like(q, float("nan"))
    with pytest.raises(fa.FibAttnError) as ei:
        fa.fibattn_fwd_noalloc(q, k, k, 1.0, 4, O.FIB_BASE, o)
    assert ei.value.status == 3 and "allocation-free" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()                 # nothing was queued
    # an argument error is reported as fibattn_fwd reports it
    with pytest.raises(fa.FibAttnError) as ei:
        fa.fibattn_fwd_noalloc(q, k, k, -1.0, 4, O.FIB_BASE, o)
    assert ei.value.status == 1
