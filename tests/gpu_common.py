"""Helpers shared by the GPU tests: seeded inputs on the device, oracle references."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

from inputs import configs
from inputs.generate import expert_weights, routing_inputs, weights_f64
from oracle import moe as orc

BF16_TOL = 2e-2      # relative L2 error bound for bf16 outputs
F32_TOL = 1e-5       # relative L2 error bound for fp32 outputs
U32 = 2.0 ** -24


def gate_rtol(d):
    """Relative bound on a GPU gate (fp32 softmax) against the fp64 oracle, for width d.

    A router logit is an fp32 dot product of d terms of unit scale; under the
    probabilistic rounding model its absolute error is about u*sqrt(d/2) (u = 2^-24:
    3.3e-6 at d = 6144, 4.8e-7 at d = 128), and exp(L) turns an absolute logit error into
    a relative error of p_i; the max subtraction, exp, sum and division add a few ulp.
    The bound is 16 of those standard deviations plus 8 ulp.  Largest deviations seen:
    1.2e-5 at d = 6144 and 1.0e-5 at d = 4096 (against 5.3e-5 and 4.3e-5 here).  A wrong
    expert, scale or normalisation moves a gate by 1e-3 or more."""
    return 16.0 * U32 * (d / 2.0) ** 0.5 + 8.0 * U32


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def audited(wl, modify=None, drop_cols=(), max_rounds=30):
    """Routing inputs of an ad-hoc workload with near-tie tokens redrawn (oracle audit).

    ``modify(ri)`` edits the inputs (planted ties, biases) before each audit; columns in
    ``drop_cols`` are exact duplicates of other experts and are left out of the audit
    (their ties are exact on both sides and resolved by index).
    """
    res = {}
    keep = np.array([e for e in range(wl.E) if e not in set(drop_cols)])
    for _ in range(max_rounds):
        ri = routing_inputs(wl, beta=0.0, resample=sorted(res.items()))
        if modify is not None:
            modify(ri)
        p = orc.router_probs(ri.x_f64(), ri.w_router)
        bad = np.nonzero(~orc.selection_margin_ok(p[:, keep], ri.bias[keep], min(wl.K, keep.size - 1)))[0]
        if bad.size == 0:
            return ri
        for t in bad:
            res[int(t)] = res.get(int(t), 0) + 1
    raise RuntimeError("audit did not converge")


def adhoc(name="adhoc", **kw):
    base = dict(name=name, T=300, d=136, N=12, Z=5, K=4, I=200, dtype="bf16", seed_key=(100,),
                expert_std=1.0 / np.sqrt(136), bias=("uniform", 0.02))
    base.update(kw)
    return configs.Workload(**base)


@dataclasses.dataclass
class Case:
    wl: object
    ri: object
    x: object
    w_router: object
    bias: object
    w: dict


def make_case(wl, ri=None, weights=True):
    dev = device()
    ri = ri if ri is not None else routing_inputs(wl)
    w = expert_weights(wl, dev) if weights else None
    return Case(wl, ri, ri.x_torch(dev), ri.w_router_torch(dev), ri.bias_torch(dev), w)


def oracle_route(case):
    return orc.route(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, case.wl.K)


def oracle_forward(case, tokens=None):
    w = case.w
    cache = {}

    def experts(e):
        if e not in cache:
            cache.clear()
            cache[e] = (weights_f64(w["gate"][e]), weights_f64(w["up"][e]), weights_f64(w["down"][e]))
        return cache[e]

    return orc.moe_forward(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, experts,
                           case.wl.N, case.wl.K, tokens=tokens)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def worst_token_rel(got, ref):
    num = np.linalg.norm(np.asarray(got, np.float64) - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return float((num / den).max())


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()
