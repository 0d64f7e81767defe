"""Float64 CPU oracle for depth-staggered Fibonacci-offset sparse attention.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline leg
are the only callers. The HIP library never imports, links or runs anything here, and this module
shares no code, table or helper with it.

What it computes is the plain definition, written out in float64 NumPy, vectorised over
(batch, head, query) and looping over one attention slot at a time. Citations name sections of
the paper "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static Schedules Beat Learned
Dilation and Extrapolate Where Dense Attention Fails" (C. A. Capps, arXiv 2606.28560):

* attended set, Fibonacci base, scaled offsets, interpolated shifted gather, RoPE before the
  gather: §2 "Attended set";
* alpha = 0.5 + sigmoid(theta) and the four per-layer schedules: §2 "Per-layer scalar";
* the power-of-two control base: §2 "Control base";
* integer offsets through a boolean mask are numerically identical to the gather, and the fixed
  and staggered variants have integer offsets: §2 "Implementation note";
* GQA 8 query / 2 key-value heads, head dim 64, RoPE theta 1e4: §3 "Models and training".

Readings taken where the paper is silent (each one is a definition choice, shared on paper with
the HIP path but not in code):

1. The window is the distances {0, 1, ..., W}: W + 1 slots, self included.
2. Offset d = alpha * f is read between rows i - floor(d) (weight 1 - t) and i - floor(d) - 1
   (weight t), t = d - floor(d): linear interpolation at distance d.
3. An offset whose d is integral after snapping (|d - rint(d)| <= 1e-9) is an integer slot. It is
   dropped when d <= W (the window already holds that distance: the attended set is a union)
   and otherwise reads row i - d, valid iff i >= d. A non-integral offset is never dropped; it is
   valid iff i >= floor(d) + 1, so the farther row is never before row 0.
4. RoPE uses half-split pairs (j, j + D/2) with frequency theta^(-2j/D). Rows are rotated at their
   own integer positions and then blended.
5. Scores are scaled by 1/sqrt(D). Query head h reads key-value head h // (Hq / Hkv).
6. Tensors are [B, H, L, D].
7. The slope of the read position in d is one-sided at an integral d; integer and dropped offsets
   contribute nothing to d(alpha).
8. The rounded-integer stagger (integer offsets for the static schedules) takes d_k = alpha f_k
   rounded to the nearest integer, ties to even, after snapping 2 d_k to an integer within the
   tolerance of reading 3 (so that a ramp value like 0.5 + 5/15 times 3 is the tie 2.5). Its
   attended set is the window and the distinct rounded distances >= 1 (a union: rungs that round
   to one distance are one slot); it is read with alpha = 1 through the plan of reading 3.
"""

from __future__ import annotations

import math
from typing import Iterator, List, NamedTuple, Sequence, Tuple

import numpy as np

# §2 "Attended set": the base sequence, K = 15.
FIB_BASE: Tuple[int, ...] = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)
# §2 "Control base": a reach-matched power-of-two base; this fixed list of 11 rungs ends at 1024.
POW2_BASE_1024: Tuple[int, ...] = tuple(2 ** n for n in range(11))
# The same control grown with the length: rungs up to 2048 at L = 4096.
POW2_BASE_2048: Tuple[int, ...] = tuple(2 ** n for n in range(12))
# §3 "Models and training": RoPE theta.
ROPE_THETA = 1.0e4
# Reading 3: absolute tolerance under which alpha * f counts as integral.
SNAP_TOL = 1.0e-9

DUP, INT, INTERP = "dup", "int", "interp"


# ----------------------------------------------------------------------------------------------
# Per-layer scalar and schedules (§2 "Per-layer scalar")
# ----------------------------------------------------------------------------------------------

def sigmoid(x: float) -> float:
    return 1.0 / (1.0 + math.exp(-x))


def alpha_from_theta(theta: float) -> float:
    """alpha = 0.5 + sigmoid(theta), in [0.5, 1.5]."""
    return 0.5 + sigmoid(theta)


def dalpha_dtheta(theta: float) -> float:
    s = sigmoid(theta)
    return s * (1.0 - s)


def alpha_fixed(layer: int, n_layers: int) -> float:
    """Fixed schedule: alpha = 1 in every layer."""
    return 1.0


def alpha_linear(layer: int, n_layers: int) -> float:
    """Linear stagger: alpha_l = 0.5 + l / (n_layers - 1), a ramp from 0.5 to 1.5."""
    return 0.5 + layer / (n_layers - 1)


def coprime_index(layer: int, n_layers: int, stride: int = 7) -> int:
    """Coprime (HDC) reassignment l -> stride * l mod n_layers, with stride 7."""
    return (stride * layer) % n_layers


def alpha_coprime(layer: int, n_layers: int, stride: int = 7) -> float:
    """Coprime stagger: the linear ramp's values reassigned to layers by l -> 7 l mod n_layers."""
    return alpha_linear(coprime_index(layer, n_layers, stride), n_layers)


# ----------------------------------------------------------------------------------------------
# Offset plan (§2 "Attended set": d_k = alpha f_k, read at i - d_k by interpolation)
# ----------------------------------------------------------------------------------------------

class Offset(NamedTuple):
    kind: str     # DUP, INT or INTERP
    f: int        # base rung f_k
    d: float      # alpha * f_k after snapping
    a: int        # floor(d): distance of the nearer row
    t: float      # d - a: weight of the farther row (0 for INT and DUP)
    reach: int    # smallest query index at which the slot is valid: ceil(d)


def plan_offsets(alpha: float, W: int, offsets: Sequence[int]) -> List[Offset]:
    plan = []
    for f in offsets:
        d = alpha * float(f)
        r = float(round(d))
        if abs(d - r) <= SNAP_TOL:
            d = r
        a = math.floor(d)
        if d == a:
            kind = DUP if a <= W else INT
            plan.append(Offset(kind, int(f), d, int(a), 0.0, int(a)))
        else:
            plan.append(Offset(INTERP, int(f), d, int(a), d - a, int(a) + 1))
    return plan


def rounded_offsets(alpha: float, offsets: Sequence[int]) -> Tuple[int, ...]:
    """Reading 8 (§2 "Implementation note": the static variants have integer offsets): the
    distinct values >= 1 of round-half-even(alpha f_k), increasing."""
    out = set()
    for f in offsets:
        d2 = 2.0 * alpha * float(f)
        r2 = float(round(d2))
        if abs(d2 - r2) <= SNAP_TOL:
            d2 = r2                      # an exact integer or half-integer distance
        n = int(round(d2 / 2.0))         # Python rounds an exact half to the even integer
        if n >= 1:
            out.add(n)
    return tuple(sorted(out))


# ----------------------------------------------------------------------------------------------
# RoPE at true positions (§2 "Attended set"; theta from §3 "Models and training")
# ----------------------------------------------------------------------------------------------

def rope_cos_sin(L: int, D: int, theta: float = ROPE_THETA) -> Tuple[np.ndarray, np.ndarray]:
    pos = np.arange(L, dtype=np.float64)[:, None]
    j = np.arange(D // 2, dtype=np.float64)[None, :]
    omega = theta ** (-2.0 * j / D)
    ang = pos * omega
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate each row of x [..., L, D] at its own position p by angles p * theta^(-2j/D)."""
    L, D = x.shape[-2], x.shape[-1]
    c, s = rope_cos_sin(L, D, theta)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_transpose(g: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Apply the transpose of each row's rotation (the adjoint used by the backward pass)."""
    L, D = g.shape[-2], g.shape[-1]
    c, s = rope_cos_sin(L, D, theta)
    g1, g2 = g[..., : D // 2], g[..., D // 2:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


# ----------------------------------------------------------------------------------------------
# Slots: the attended set of every query, one slot at a time
# ----------------------------------------------------------------------------------------------

def shift_down(x: np.ndarray, a: int) -> np.ndarray:
    """y[..., i, :] = x[..., i - a, :] for i >= a; zero rows where i - a < 0."""
    L = x.shape[-2]
    y = np.zeros_like(x)
    if a < L:
        y[..., a:, :] = x[..., : L - a, :]
    return y


def shift_up(x: np.ndarray, a: int) -> np.ndarray:
    """Adjoint of shift_down: y[..., j, :] = x[..., j + a, :] for j + a < L; zero elsewhere."""
    L = x.shape[-2]
    y = np.zeros_like(x)
    if a < L:
        y[..., : L - a, :] = x[..., a:, :]
    return y


class Slot(NamedTuple):
    label: str           # "win", "int" or "interp"
    a: int               # distance of the nearer row
    t: float             # weight of the farther row a + 1 (0 unless interp)
    f: int               # base rung (0 for window slots)
    valid: np.ndarray    # [L] bool: slot present for query i


def slots(L: int, W: int, plan: Sequence[Offset]) -> List[Slot]:
    """The attended set: window distances 0..W, then the kept offsets in base order."""
    i = np.arange(L)
    out = [Slot("win", dist, 0.0, 0, i >= dist) for dist in range(W + 1)]
    for off in plan:
        if off.kind == INT:
            out.append(Slot("int", off.a, 0.0, off.f, i >= off.a))
        elif off.kind == INTERP:
            out.append(Slot("interp", off.a, off.t, off.f, i >= off.a + 1))
    return out


def gather(x: np.ndarray, slot: Slot) -> np.ndarray:
    """Rows read by `slot` for every query: x[i - a], or (1 - t) x[i - a] + t x[i - a - 1]."""
    near = shift_down(x, slot.a)
    if slot.label != "interp":
        return near
    far = shift_down(x, slot.a + 1)
    return (1.0 - slot.t) * near + slot.t * far


def _expand_heads(x: np.ndarray, Hq: int) -> np.ndarray:
    """Key-value heads [B, Hkv, L, D] to query heads [B, Hq, L, D]: head h reads h // (Hq/Hkv)."""
    Hkv = x.shape[1]
    return np.repeat(x, Hq // Hkv, axis=1)


def _sum_groups(x: np.ndarray, Hkv: int) -> np.ndarray:
    B, Hq, L, D = x.shape
    return x.reshape(B, Hkv, Hq // Hkv, L, D).sum(axis=2)


# ----------------------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------------------

def _as64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def forward(q, k, v, alpha: float, W: int, offsets: Sequence[int], rope_theta: float = ROPE_THETA,
            return_probs: bool = False):
    """o [B, Hq, L, D] and lse [B, Hq, L] (natural log) of the sparse attention."""
    q, k, v = _as64(q, k, v)
    B, Hq, L, D = q.shape
    scale = 1.0 / math.sqrt(D)
    qrot, krot = rope(q, rope_theta), rope(k, rope_theta)
    sl = slots(L, W, plan_offsets(alpha, W, offsets))
    S = np.empty((B, Hq, L, len(sl)))
    for n, slot in enumerate(sl):
        key = _expand_heads(gather(krot, slot), Hq)
        s = scale * np.einsum("bhld,bhld->bhl", qrot, key)
        S[..., n] = np.where(slot.valid, s, -np.inf)
    m = S.max(axis=-1)
    e = np.exp(S - m[..., None])
    z = e.sum(axis=-1)
    P = e / z[..., None]
    lse = m + np.log(z)
    o = np.zeros_like(q)
    for n, slot in enumerate(sl):
        val = _expand_heads(gather(v, slot), Hq)
        o += P[..., n, None] * val
    if return_probs:
        return o, lse, P, sl
    return o, lse


# ----------------------------------------------------------------------------------------------
# Backward (chain rule through softmax, the interpolated gather and RoPE)
# ----------------------------------------------------------------------------------------------

def backward(q, k, v, do, alpha: float, W: int, offsets: Sequence[int],
             rope_theta: float = ROPE_THETA):
    """Gradients (dq, dk, dv, dalpha) of sum(do * o) with respect to q, k, v and alpha."""
    q, k, v, do = _as64(q, k, v, do)
    B, Hq, L, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D)
    o, _, P, sl = forward(q, k, v, alpha, W, offsets, rope_theta, return_probs=True)
    qrot, krot = rope(q, rope_theta), rope(k, rope_theta)
    delta = np.einsum("bhld,bhld->bhl", do, o)
    dqrot = np.zeros_like(q)
    dkrot = np.zeros_like(k)
    dv = np.zeros_like(v)
    dalpha = 0.0
    for n, slot in enumerate(sl):
        key = _expand_heads(gather(krot, slot), Hq)
        val = _expand_heads(gather(v, slot), Hq)
        p = P[..., n]
        dp = np.einsum("bhld,bhld->bhl", do, val)
        ds = p * (dp - delta)
        dqrot += scale * ds[..., None] * key
        dkey = _sum_groups(scale * ds[..., None] * qrot, Hkv)
        dval = _sum_groups(p[..., None] * do, Hkv)
        if slot.label == "interp":
            w_near, w_far = 1.0 - slot.t, slot.t
            dkrot += w_near * shift_up(dkey, slot.a) + w_far * shift_up(dkey, slot.a + 1)
            dv += w_near * shift_up(dval, slot.a) + w_far * shift_up(dval, slot.a + 1)
            # d(row read)/dt = x[i - a - 1] - x[i - a]; dt/dalpha = f.
            dk_dir = shift_down(krot, slot.a + 1) - shift_down(krot, slot.a)
            dv_dir = shift_down(v, slot.a + 1) - shift_down(v, slot.a)
            dt = np.sum(dkey * dk_dir) + np.sum(dval * dv_dir)
            dalpha += slot.f * dt
        else:
            dkrot += shift_up(dkey, slot.a)
            dv += shift_up(dval, slot.a)
    dq = rope_transpose(dqrot, rope_theta)
    dk = rope_transpose(dkrot, rope_theta)
    return dq, dk, dv, dalpha


def valid_slot_count(L: int, W: int, plan: Sequence[Offset]) -> np.ndarray:
    """Number of valid slots of each query position [L] (used for the FLOP accounting)."""
    return np.sum([s.valid for s in slots(L, W, plan)], axis=0)
