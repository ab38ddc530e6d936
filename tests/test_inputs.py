"""The seeded workload generator and its offline routing table (no GPU)."""
import numpy as np
import pytest

from inputs import configs
from inputs.generate import (bf16_bits_to_f64, f64_to_bf16_bits, load_table, routing_inputs)
from oracle import bruteforce
from oracle import moe as orc


def test_bf16_rounding_is_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1.
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20, 0.0])
    bits = f64_to_bf16_bits(vals)
    back = bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7, 0.0])


def test_generator_is_reproducible():
    wl = configs.get("small")
    a, b = routing_inputs(wl), routing_inputs(wl)
    assert (a.x == b.x).all() and (a.w_router == b.w_router).all() and (a.bias == b.bias).all()


def test_expert_weights_reproducible_cpu():
    import torch
    from inputs.generate import expert_weights
    wl = configs.get("tiny")
    w1, w2 = expert_weights(wl), expert_weights(wl)
    for k in ("gate", "up", "down"):
        assert torch.equal(w1[k], w2[k])
    assert w1["gate"].shape == (8, 256, 128) and w1["down"].shape == (8, 128, 256)
    assert abs(float(w1["gate"].std()) - wl.expert_std) < 0.01


@pytest.mark.parametrize("name", [n for n in configs.WORKLOADS])
def test_table_shares_and_margins(name):
    wl = configs.get(name)
    entry = load_table()[name]
    ri = routing_inputs(wl)
    p = orc.router_probs(ri.x_f64(), ri.w_router)
    assert orc.selection_margin_ok(p, ri.bias, wl.K).all()
    idx = orc.select_topk(orc.selection_scores(p, ri.bias), wl.K)
    share = float((idx >= wl.N).mean())
    assert share == pytest.approx(entry["share"], abs=1e-12)
    if wl.target_share is not None:
        assert abs(share - wl.target_share) <= 0.002
    ffn = (idx < wl.N).sum(axis=1)
    assert np.bincount(ffn, minlength=wl.K + 1).tolist() == entry["ffn_count_hist"]
    if name == "skewed":        # per-token FFN count spans 0..K; loads heavy-tailed
        assert ffn.min() == 0 and ffn.max() == wl.K
        load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
        assert load.max() > 30 * np.median(load)
        assert (ffn[ri.easy_tokens] <= 1).mean() > 0.5 and (ffn[ri.hard_tokens] == wl.K).mean() > 0.5


def test_tiny_workload_routing_matches_bruteforce():
    wl = configs.get("tiny")
    ri = routing_inputs(wl)
    x = ri.x_f64()
    idx, gate, _ = orc.route(x, ri.w_router.astype(np.float64), ri.bias, wl.K)
    wr = ri.w_router.astype(np.float64).tolist()
    b = ri.bias.astype(np.float64).tolist()
    for t in range(wl.T):
        picks, p = bruteforce.route_token(x[t].tolist(), wr, b, wl.K)
        assert idx[t].tolist() == picks
        np.testing.assert_allclose(gate[t], [p[i] for i in picks], rtol=1e-13)


def test_tiny_workload_forward_matches_bruteforce():
    from inputs.generate import expert_weights, weights_f64
    wl = configs.get("tiny")
    ri = routing_inputs(wl)
    w = {k: weights_f64(v) for k, v in expert_weights(wl).items()}
    x = ri.x_f64()
    rows = list(range(0, 64, 8))
    out = orc.moe_forward(x, ri.w_router.astype(np.float64), ri.bias,
                          lambda e: (w["gate"][e], w["up"][e], w["down"][e]), wl.N, wl.K, tokens=rows)
    L = lambda a: np.asarray(a).tolist()
    bidx, _, by = bruteforce.forward(L(x[rows]), L(ri.w_router.astype(np.float64)), L(ri.bias.astype(np.float64)),
                                     L(w["gate"]), L(w["up"]), L(w["down"]), wl.N, wl.K)
    assert out["idx"].tolist() == bidx
    np.testing.assert_allclose(out["y"], by, rtol=1e-12, atol=1e-14)
