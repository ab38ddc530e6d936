"""Scalar pure-Python formulation of the MoE layer, for tiny inputs only.

TEST INFRASTRUCTURE (see oracle/__init__.py).  Independent of oracle/moe.py: no numpy
arithmetic, explicit loops, exactly rounded sums (math.fsum), selection by sorting
(-score, index) tuples.  Same definition: LongCat-Flash article (itouyu.top), section
"Zero-computation experts" -- softmax router over N FFN plus Z identity experts, the
expert bias added for selection only, K picks, gates equal to the unbiased router
probabilities, identity experts returning their input.
"""
from __future__ import annotations

import math
import struct


def _f32(v: float) -> float:
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("f", struct.pack("f", v))[0]


def _dot(a, b) -> float:
    return math.fsum(ai * bi for ai, bi in zip(a, b))


def route_token(x_t, w_router, bias, K):
    """(picks, probs) of one token: picks ordered by (s desc, index asc)."""
    E = len(w_router)
    logits = [_dot(w_router[i], x_t) for i in range(E)]
    m = max(logits)
    ex = [math.exp(l - m) for l in logits]
    tot = math.fsum(ex)
    p = [v / tot for v in ex]
    s = [_f32(_f32(p[i]) + _f32(bias[i])) for i in range(E)]
    picks = [i for _, i in sorted((-s[i], i) for i in range(E))[:K]]
    return picks, p


def _silu(a: float) -> float:
    if a < -700.0:
        return 0.0
    return a / (1.0 + math.exp(-a))


def expert_out(x_t, wg, wu, wd):
    I = len(wg)
    h = [_silu(_dot(wg[j], x_t)) * _dot(wu[j], x_t) for j in range(I)]
    return [_dot(wd[c], h) for c in range(len(wd))]


def forward(x, w_router, bias, w_gate, w_up, w_down, N, K):
    """Lists in, lists out: (idx [T][K], gate [T][K], y [T][d])."""
    idx, gates, y = [], [], []
    for x_t in x:
        picks, p = route_token(x_t, w_router, bias, K)
        terms = []
        for i in picks:
            out = expert_out(x_t, w_gate[i], w_up[i], w_down[i]) if i < N else list(x_t)
            terms.append([p[i] * v for v in out])
        y.append([math.fsum(col) for col in zip(*terms)])
        idx.append(picks)
        gates.append([p[i] for i in picks])
    return idx, gates, y
