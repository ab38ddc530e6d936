"""Plain CPU oracle of the zero-computation-expert MoE layer forward (fp64, numpy).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the GPU library.

What the layer computes (LongCat-Flash article, itouyu.top / kqgmpj.cn / dhxrcw.cn,
section "Zero-computation experts"; the displayed MoE equation of that section was an
image and is lost, only its variable glossary survives, so the formula below is the
plainest reading of the glossary plus the surrounding text):

  p_t      = softmax over all N+Z experts of the router scores W_r x_t      (R, softmax router)
  s_t,i    = p_t,i + b_i        expert bias, used only to choose experts     (bias paragraph)
  S_t      = the K experts with the largest s_t,i; equal s -> lower index first
  g_t,i    = p_t,i for i in S_t (unbiased, no renormalisation)
  E_i(x)   = W_down,i (silu(W_gate,i x) * (W_up,i x))      FFN expert, i < N (SwiGLU)
  E_i(x)   = x                                             zero-computation expert, i >= N
  y_t      = sum over i in S_t of g_t,i E_i(x_t), summed in the order of S_t

Readings where the pages are silent:
  * the bias enters the selection score, which is the softmax output, never the gate;
  * the selection decision (an integer result decided by floating point) is taken on
    fp32 scores, the GPU kernel's precision: p is rounded to fp32 and b (fp32) is added
    in fp32; everything else here is fp64;
  * top-K output order is (s descending, index ascending);
  * the expert permutation lists each FFN expert's picks in (token, pick) order, i.e.
    ascending token order (a token picking an expert twice, which the router never does,
    would get two consecutive rows).

Expert weights are given per expert through ``experts(e) -> (W_gate[I,d], W_up[I,d],
W_down[d,I])`` in fp64, so a caller can stream them one expert at a time.
"""
from __future__ import annotations

import numpy as np


def router_probs(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Softmax router R over all N+Z experts, fp64.  x [T,d], W_r [E,d] -> p [T,E]."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    shifted = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(shifted)
    return e / e.sum(axis=1, keepdims=True)


def selection_scores(p: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """s = p + b, formed in fp32 (the precision in which the GPU takes the decision)."""
    return p.astype(np.float32) + np.asarray(bias, np.float32)[None, :]


def select_topk(s: np.ndarray, K: int) -> np.ndarray:
    """The K largest scores per row, ordered by (s descending, index ascending)."""
    order = np.argsort(-s, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def route(x, w_router, bias, K):
    """Router + biased top-K.  Returns (topk_idx int32 [T,K], topk_gate fp64 [T,K], p)."""
    p = router_probs(x, w_router)
    idx = select_topk(selection_scores(p, bias), K)
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return idx, gate, p


def expert_load(idx: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, pick) pairs that chose each of the N+Z experts."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def ffn_count(idx: np.ndarray, N: int) -> np.ndarray:
    """Per-token number of FFN experts among its K picks (0..K)."""
    return (np.asarray(idx) < N).sum(axis=1).astype(np.int64)


def permute(idx: np.ndarray, N: int):
    """Expert-contiguous order of the FFN picks.

    Returns offsets [N+1] (exclusive prefix sum of the FFN experts' loads),
    perm_token [nnz] (the token of each row; (token, pick) order within each expert) and
    slot_row [T,K] (row of pick (t,k), -1 for a zero-computation pick).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    ts, ks = np.nonzero(idx < N)                 # row-major: token order, then k
    es = idx[ts, ks]
    order = np.argsort(es, kind="stable")        # stable: ascending token inside an expert
    load = np.bincount(es, minlength=N)[:N]
    offsets = np.concatenate([[0], np.cumsum(load)]).astype(np.int64)
    perm_token = ts[order].astype(np.int64)
    slot_row = np.full((T, K), -1, dtype=np.int64)
    slot_row[ts[order], ks[order]] = np.arange(order.size)
    return offsets, perm_token, slot_row


def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_expert(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray):
    """One FFN expert on rows X [m,d]: W_down (silu(W_gate x) * (W_up x)), fp64."""
    G = X @ w_gate.T
    U = X @ w_up.T
    return (silu(G) * U) @ w_down.T


def combine(x, y_perm, idx, gate, slot_row, N):
    """y_t = sum over the token's picks, in pick order, of g times the expert output:
    the FFN output row for an FFN pick, x_t itself for a zero-computation pick."""
    y = np.zeros_like(x)
    for k in range(idx.shape[1]):
        contrib = x.copy()                           # identity expert: E_i(x) = x
        is_ffn = idx[:, k] < N
        contrib[is_ffn] = y_perm[slot_row[is_ffn, k]]
        y += gate[:, k:k + 1] * contrib
    return y


def zero_gate_sum(idx, gate, N):
    """Per token, the sum of the gates of its zero-computation picks (their experts all
    return x_t, so together they add this sum times x_t)."""
    return (np.asarray(gate, np.float64) * (np.asarray(idx) >= N)).sum(axis=1)


def moe_forward(x, w_router, bias, experts, N, K, tokens=None):
    """Whole layer forward in fp64.

    x [T,d] fp64, W_r [E,d], b [E]; ``experts(e)`` returns fp64 (W_gate, W_up, W_down)
    of FFN expert e.  With ``tokens`` given, only those rows are routed and combined
    (each token's result depends on its own row only).
    Returns dict(idx, gate, y, y_ffn, gz, load, ffn_count, offsets, perm_token, slot_row):
    y_ffn is the FFN picks' part of y (the zero picks' part is gz * x, gz = zero_gate_sum).
    """
    return moe_forward_batches([dict(x=x, w_router=w_router, bias=bias, K=K, tokens=tokens)],
                               experts, N)[0]


def moe_forward_batches(batches, experts, N, expert_fn=None):
    """moe_forward of several token batches through one layer's experts (for instance a
    prefill batch and decode batches of the same layer), with one pass over the experts:
    ``experts(e)`` is called once for every expert that any batch routes a token to.
    batches: list of dict(x, w_router, bias, K, tokens=None); returns one moe_forward result
    per batch, each equal to moe_forward on that batch alone.  expert_fn(X, wg, wu, wd)
    evaluates one expert on its rows (default swiglu_expert; the FP8 MFMA layer passes
    oracle.fp8.fp8_act_expert)."""
    expert_fn = swiglu_expert if expert_fn is None else expert_fn
    prep = []
    for b in batches:
        x = np.asarray(b["x"], np.float64)
        if b.get("tokens") is not None:
            x = x[np.asarray(b["tokens"])]
        idx, gate, _ = route(x, b["w_router"], b["bias"], b["K"])
        offsets, perm_token, slot_row = permute(idx, N)
        prep.append(dict(x=x, E=b["w_router"].shape[0], idx=idx, gate=gate, offsets=offsets,
                         perm_token=perm_token, slot_row=slot_row,
                         y_perm=np.zeros((perm_token.size, x.shape[1]))))
    for e in range(N):
        if all(q["offsets"][e + 1] == q["offsets"][e] for q in prep):
            continue
        wg, wu, wd = experts(e)
        for q in prep:
            r0, r1 = q["offsets"][e], q["offsets"][e + 1]
            if r1 > r0:
                q["y_perm"][r0:r1] = expert_fn(q["x"][q["perm_token"][r0:r1]], wg, wu, wd)
    out = []
    for q in prep:
        x, idx, gate, slot_row = q["x"], q["idx"], q["gate"], q["slot_row"]
        y = combine(x, q["y_perm"], idx, gate, slot_row, N)
        y_ffn = combine(np.zeros_like(x), q["y_perm"], idx, gate, slot_row, N)
        out.append(dict(idx=idx, gate=gate, y=y, y_ffn=y_ffn, gz=zero_gate_sum(idx, gate, N),
                        load=expert_load(idx, q["E"]), ffn_count=ffn_count(idx, N),
                        offsets=q["offsets"], perm_token=q["perm_token"], slot_row=slot_row))
    return out


def selection_margin_ok(p: np.ndarray, bias: np.ndarray, K: int, rel: float = 1e-4,
                        ulp_rel: float = 1e-6) -> np.ndarray:
    """Tokens whose first K+1 selection scores are separated well enough.

    A GPU computes p in fp32 with its own summation order; an order between two scores
    is reproducible only if their fp64 gap exceeds both p's relative error (rel * p) and
    the fp32 rounding of s (ulp_rel * |s|).  Returns a boolean per token.
    """
    s = p + np.asarray(bias, np.float64)[None, :]
    top = np.argsort(-s, axis=1, kind="stable")[:, :K + 1]
    st = np.take_along_axis(s, top, axis=1)
    pt = np.take_along_axis(p, top, axis=1)
    gap = st[:, :-1] - st[:, 1:]
    need = rel * (pt[:, :-1] + pt[:, 1:]) + ulp_rel * (np.abs(st[:, :-1]) + np.abs(st[:, 1:]))
    return np.all(gap > need, axis=1)
