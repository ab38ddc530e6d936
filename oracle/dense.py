"""Dense-masked formulation of the MoE layer combine, for pinning the oracle.

TEST INFRASTRUCTURE (see oracle/__init__.py).  Every FFN expert runs on every token and
the results are mixed with a [T, N+Z] gate matrix that is zero outside each token's
picks; identity experts add their gate times x.  It uses no permutation, no slot table
and no per-pick loop, so it checks oracle/moe.py's permute/combine bookkeeping
independently (LongCat-Flash article, itouyu.top, section "Zero-computation experts":
the layer output is the gate-weighted sum of the chosen experts' outputs, a
zero-computation expert outputting its input).
"""
from __future__ import annotations

import numpy as np


def gate_matrix(idx: np.ndarray, gate: np.ndarray, E: int) -> np.ndarray:
    G = np.zeros((idx.shape[0], E))
    np.put_along_axis(G, np.asarray(idx, np.int64), gate, axis=1)
    return G


def forward(x, G, w_gate, w_up, w_down, N):
    """x [T,d], gate matrix G [T,E], stacked fp64 weights [N,...] -> y [T,d]."""
    x = np.asarray(x, np.float64)
    y = G[:, N:].sum(axis=1, keepdims=True) * x
    for e in range(N):
        g = x @ w_gate[e].T
        u = x @ w_up[e].T
        with np.errstate(over="ignore"):
            h = g / (1.0 + np.exp(-g)) * u
        y += G[:, e:e + 1] * (h @ w_down[e].T)
    return y
