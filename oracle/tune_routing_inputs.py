"""Offline tuning of the synthetic routing inputs; writes inputs/routing_tables.json.

TEST INFRASTRUCTURE.  Run from the repository root:  python -m oracle.tune_routing_inputs
It calls only the oracle (fp64 routing) and the seeded input generator.

For every named workload:
  1. zero-expert bias shift beta (workloads whose recipe asks for it): bisection until the
     share of picks that land on zero-computation experts is within 0.002 of the target
     (the pages tie the zero-expert selection frequency to a bias controller; the
     controller's converged state is what this stands in for -- LongCat-Flash article,
     itouyu.top, section "Zero-computation experts");
  2. selection-margin audit: a token whose first K+1 selection scores are closer than
     the fp32 error budget (see oracle.moe.selection_margin_ok) gets its x row redrawn;
  3. repeat until both hold at once.
"""
from __future__ import annotations

import json
import sys
import time

import numpy as np

from inputs import configs
from inputs.generate import TABLE_PATH, bias_vector, routing_inputs
from oracle.moe import router_probs, select_topk, selection_margin_ok, selection_scores

SHARE_TOL = 0.002


def zero_share(p, b, K, N):
    idx = select_topk(selection_scores(p, b), K)
    return float((idx >= N).mean()), idx


def _edge(wl, p, lo, hi, above):
    """Bisection for the beta where the share first exceeds ``above`` (share(lo) <= above)."""
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if zero_share(p, bias_vector(wl, mid), wl.K, wl.N)[0] > above:
            hi = mid
        else:
            lo = mid
        if hi - lo < 1e-13:
            break
    return lo, hi


def tune_beta(wl, p):
    """Middle of the beta interval whose zero-expert share is closest to the target.

    The share is a step function of beta; its steps sit exactly where some token has a
    zero and an FFN expert with equal selection score, so beta is kept away from them.
    """
    target = wl.target_share
    K, N = wl.K, wl.N
    lo, hi = -0.5, 0.5
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if zero_share(p, bias_vector(wl, mid), K, N)[0] < target:
            lo = mid
        else:
            hi = mid
        if hi - lo < 1e-13:
            break
    s_lo = zero_share(p, bias_vector(wl, lo), K, N)[0]
    s_hi = zero_share(p, bias_vector(wl, hi), K, N)[0]
    level = s_lo if abs(s_lo - target) <= abs(s_hi - target) else s_hi
    probe = lo if level == s_lo else hi
    # plateau [a, b] of the chosen share level around ``probe``
    below = zero_share(p, bias_vector(wl, -0.5), K, N)[0]
    a = -0.5 if below >= level else _edge(wl, p, -0.5, probe, level - 1e-12)[1]
    b = _edge(wl, p, probe, 0.5, level)[0]
    return 0.5 * (a + b)


def tune(wl, max_rounds=40):
    resample = {}
    beta = 0.0
    t0 = time.time()
    p = None
    for rnd in range(max_rounds):
        ri = routing_inputs(wl, beta=beta, resample=sorted(resample.items()))
        p = router_probs(ri.x_f64(), ri.w_router)
        b = bias_vector(wl, beta)
        share, idx = zero_share(p, b, wl.K, wl.N)
        share_ok = wl.target_share is None or abs(share - wl.target_share) <= SHARE_TOL
        if wl.tuned and (rnd == 0 or not share_ok):
            beta = tune_beta(wl, p)
            b = bias_vector(wl, beta)
            share, idx = zero_share(p, b, wl.K, wl.N)
            share_ok = abs(share - wl.target_share) <= SHARE_TOL
        ok = selection_margin_ok(p, b, wl.K)
        bad = np.nonzero(~ok)[0]
        print(f"  {wl.name} round {rnd}: beta={beta:.9g} share={share:.5f} near-ties={bad.size}",
              flush=True)
        if bad.size == 0 and share_ok:
            ffn = (idx < wl.N).sum(axis=1)
            hist = np.bincount(ffn, minlength=wl.K + 1)
            load = np.bincount(idx.ravel(), minlength=wl.E)
            return dict(beta=float(beta), resample=[[int(t), int(a)] for t, a in sorted(resample.items())],
                        share=share, mean_ffn_per_token=float(ffn.mean()),
                        ffn_count_hist=[int(h) for h in hist],
                        ffn_rows=int(load[:wl.N].sum()), max_expert_rows=int(load[:wl.N].max()),
                        touched_ffn_experts=int((load[:wl.N] > 0).sum()),
                        seconds=round(time.time() - t0, 1))
        for t in bad:
            resample[int(t)] = resample.get(int(t), 0) + 1
    raise RuntimeError(f"{wl.name}: tuning did not converge")


def main(names=None):
    table = {}
    try:
        with open(TABLE_PATH) as f:
            table = json.load(f)
    except FileNotFoundError:
        pass
    for name, wl in configs.WORKLOADS.items():
        if names and name not in names:
            continue
        print(f"tuning {name} ({wl.description})", flush=True)
        table[name] = tune(wl)
        with open(TABLE_PATH, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
    return table


if __name__ == "__main__":
    main(sys.argv[1:] or None)
