"""The bench's arithmetic accounting (valid slots per forward call) against the oracle's attended set.

The bench counts valid (query-head, slot) pairs from the library's offset plan in closed form; the
oracle builds the attended set of every query explicitly (window distances 0..W and the kept rungs,
each valid from its reach on, per "Depth-Staggered Fibonacci Spacing for Sparse Attention", §2
"Attended set"). The two must agree exactly for every layer of every workload.
"""

import numpy as np
import pytest

import bench
import fibonacci_offset_sparse_amd as fa
import workloads
from oracle import fibattn_oracle as O


def _alphas(w):
    if w.schedule == "learned":
        return [O.alpha_from_theta(t) for t in workloads.draw_theta(w.n_layers).tolist()]
    fn = {"fixed": O.alpha_fixed, "linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    return [fn(layer, w.n_layers) for layer in range(w.n_layers)]


def _base(w):
    if w.base == "fib":
        return O.FIB_BASE
    return {1024: O.POW2_BASE_1024, 2048: O.POW2_BASE_2048}[workloads.pow2_max(w)]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_valid_slot_counts_match_the_attended_set(name):
    w = workloads.WORKLOADS[name]
    base = _base(w)
    for alpha in _alphas(w):
        n_valid, n_interp = bench.fwd_slot_counts(fa, w, alpha, base)
        plan = O.plan_offsets(alpha, w.W, base)
        per_query = O.valid_slot_count(w.L, w.W, plan)
        assert n_valid == w.B * w.Hq * int(per_query.sum()), (name, alpha)
        interp_rows = sum(int(s.valid.sum()) for s in O.slots(w.L, w.W, plan) if s.label == "interp")
        assert n_interp == w.B * w.Hkv * interp_rows, (name, alpha)


def test_full_causal_window_counts_every_pair():
    # W >= L - 1 and no rungs: every query attends to all earlier positions and itself
    w = workloads.WORKLOADS["tiny_fixed_f32"]
    class Full:
        B, Hq, Hkv, L = w.B, w.Hq, w.Hkv, w.L
        W = w.L - 1
    n_valid, n_interp = bench.fwd_slot_counts(fa, Full, 1.0, [])
    assert n_valid == w.B * w.Hq * w.L * (w.L + 1) // 2
    assert n_interp == 0
