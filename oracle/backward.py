"""Plain CPU oracle of the backward pass of the grouped SwiGLU FFN of the MoE layer (fp64).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the GPU library.

The layer (LongCat-Flash article, itouyu.top / kqgmpj.cn / dhxrcw.cn, section
"Zero-computation experts") sums, per token t, g * E_i(x_t) over its K picks: an FFN
expert's SwiGLU output for i < N, x_t itself for a zero-computation expert.  The pages
describe training (section "Model scaling and multi-stage training") but no backward
pass; the reading taken here is the plain gradient of that sum with the routing held
fixed: given the picks and their gates (as the forward produced them) and an upstream
gradient dy of the layer output, the gradients of L = sum_t <dy_t, y_t> with respect to
x and the expert weights.  The router's own gradient (through the gates and the
softmax) is not part of it.

For an FFN pick (t, i) with gate g, with G = W_gate x_t, U = W_up x_t, s = sigmoid(G),
a = G * s (silu), H = a * U, y-term = g * W_down H:
    dY      = g * dy_t
    dH      = W_down^T dY                dW_down += dY H^T
    dG      = dH * U * (s + a * (1 - s))      (silu'(G) = s * (1 + G * (1 - s)))
    dU      = dH * a
    dW_gate += dG x_t^T                  dW_up   += dU x_t^T
    dx_t    += W_gate^T dG + W_up^T dU
For a zero-computation pick with gate g: dx_t += g * dy_t.
"""
from __future__ import annotations

import numpy as np

from . import moe


def sigmoid(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def expert_backward(X, dY, w_gate, w_up, w_down, want_dw=True):
    """One FFN expert on its rows X [m,d] with output gradients dY [m,d] (gates already
    applied).  Returns (dX [m,d], dW_gate [I,d], dW_up [I,d], dW_down [d,I]), fp64; the
    three weight gradients are None when want_dw is False."""
    G = X @ w_gate.T
    U = X @ w_up.T
    s = sigmoid(G)
    a = G * s
    H = a * U
    dH = dY @ w_down
    dG = dH * U * (s + a * (1.0 - s))
    dU = dH * a
    dX = dG @ w_gate + dU @ w_up
    if not want_dw:
        return dX, None, None, None
    return dX, dG.T @ X, dU.T @ X, dY.T @ H


def ffn_backward(x, dy, idx, gate, experts, N, dw_experts=None):
    """Gradients of L = sum_t <dy_t, y_t> for fixed picks idx [T,K] and gates gate [T,K].

    x, dy [T,d] (fp64); ``experts(e)`` returns fp64 (W_gate, W_up, W_down) of FFN expert e.
    Returns (dx [T,d], dw) with dw = {e: (dW_gate, dW_up, dW_down)} for the experts in
    ``dw_experts`` (all FFN experts with rows when None; experts without rows have zero
    gradients and are left out).  Each token's dx sums its FFN picks' terms in pick order,
    then its zero picks' gates times dy_t.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    idx = np.asarray(idx)
    gate = np.asarray(gate, np.float64)
    T, K = idx.shape
    offsets, perm_token, slot_row = moe.permute(idx, N)
    g_row = np.zeros(perm_token.size)
    ts, ks = np.nonzero(idx < N)
    g_row[slot_row[ts, ks]] = gate[ts, ks]
    dX_perm = np.zeros((perm_token.size, x.shape[1]))
    dw = {}
    for e in range(N):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        rows = perm_token[r0:r1]
        wg, wu, wd = experts(e)
        want = dw_experts is None or e in dw_experts
        dX, dWg, dWu, dWd = expert_backward(x[rows], g_row[r0:r1, None] * dy[rows], wg, wu, wd, want)
        dX_perm[r0:r1] = dX
        if want:
            dw[e] = (dWg, dWu, dWd)
    dx = np.zeros_like(x)
    for k in range(K):
        is_ffn = idx[:, k] < N
        dx[is_ffn] += dX_perm[slot_row[is_ffn, k]]
    gz = moe.zero_gate_sum(idx, gate, N)
    dx += gz[:, None] * dy
    return dx, dw
