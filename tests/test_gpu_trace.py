"""GPU checks of the phase-trace build (libfibattn_trace.so, needs an MI355X): its forward computes
bit for bit what the usual library computes, and its records are whole (one per workgroup, stamps in
order, every tile of every (batch, head group) once)."""

import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import fibattn_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fibonacci_offset_sparse_amd as m
    return m


@pytest.mark.parametrize("L,alpha,offsets", [(1100, 0.77, O.FIB_BASE), (300, 1.0, O.POW2_BASE_1024)])
def test_trace_build_matches_and_records_every_workgroup(fa, L, alpha, offsets):
    dev = torch.device("cuda:0")
    B, Hq, Hkv, W = 2, 8, 2, 12
    q = workloads.randn_like_seeded((B, Hq, L, 64), 81, torch.bfloat16).to(dev)
    k = workloads.randn_like_seeded((B, Hkv, L, 64), 82, torch.bfloat16).to(dev)
    v = workloads.randn_like_seeded((B, Hkv, L, 64), 83, torch.bfloat16).to(dev)
    say(f"phase trace L={L} alpha={alpha} K={len(offsets)}")
    o_ref, lse_ref = fa.fibattn_fwd(q, k, v, alpha, W, offsets)
    torch.cuda.synchronize()
    usual = fa.lib
    try:
        fa.lib = fa._load_from(fa.TRACE_LIB_PATH)
        o, lse = fa.fibattn_fwd(q, k, v, alpha, W, offsets)
        torch.cuda.synchronize()
        n_tiles = (L + 63) // 64
        n_wg = B * Hkv * (Hq // Hkv // 4) * n_tiles
        rec = fa.fibattn_phase_trace_read(n_wg)
    finally:
        fa.lib = usual
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    t = rec[:, :6].astype(np.int64)
    assert (np.diff(t, axis=1) >= 0).all(), "stamps out of order"
    assert (t[:, 5] - t[:, 0] < 10 ** 7).all(), "a workgroup spanned more than 0.1 s"
    tiles = (rec[:, 6] & np.uint64(0xffff)).astype(np.int64)
    counts = np.bincount(tiles, minlength=n_tiles)
    assert (counts == B * Hkv * (Hq // Hkv // 4)).all(), counts
