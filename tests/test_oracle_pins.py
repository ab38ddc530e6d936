"""Pins of the CPU oracle against things other than itself (no GPU).

The pages print no worked example for the layer, so the oracle is pinned by: hand-derived
closed forms (tests/golden/closed_form_cases.json), an independent scalar brute force,
an independent dense-masked formulation, and invariants / special cases that follow from
the definition (LongCat-Flash article, itouyu.top, section "Zero-computation experts").
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import bruteforce, dense
from oracle import moe as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def micro(seed, T=12, d=10, N=4, Z=3, K=3, I=6, bias_scale=0.05):
    g = np.random.default_rng(seed)
    E = N + Z
    return dict(
        x=g.standard_normal((T, d)), w_router=g.standard_normal((E, d)) / math.sqrt(d),
        bias=(g.uniform(-bias_scale, bias_scale, E)).astype(np.float32).astype(np.float64),
        w_gate=g.standard_normal((N, I, d)) / math.sqrt(d), w_up=g.standard_normal((N, I, d)) / math.sqrt(d),
        w_down=g.standard_normal((N, d, I)) / math.sqrt(I), N=N, K=K)


def run_oracle(c):
    return orc.moe_forward(c["x"], c["w_router"], c["bias"],
                           lambda e: (c["w_gate"][e], c["w_up"][e], c["w_down"][e]), c["N"], c["K"])


def run_brute(c):
    L = lambda a: np.asarray(a).tolist()
    return bruteforce.forward(L(c["x"]), L(c["w_router"]), L(c["bias"]), L(c["w_gate"]), L(c["w_up"]),
                              L(c["w_down"]), c["N"], c["K"])


# ---- closed forms -------------------------------------------------------------------

def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_closed_form_cases(case):
    c = {k: np.asarray(case[k], np.float64) for k in ("x", "w_router", "bias", "w_gate", "w_up", "w_down")}
    c["N"], c["K"] = case["N"], case["K"]
    out = run_oracle(c)
    assert out["idx"].tolist() == case["idx"]
    np.testing.assert_allclose(out["gate"], case["gate"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(out["y"], case["y"], rtol=1e-13, atol=1e-15)
    bidx, bgate, by = run_brute(c)
    assert bidx == case["idx"]
    np.testing.assert_allclose(by, case["y"], rtol=1e-13, atol=1e-15)


# ---- router / selection ---------------------------------------------------------------

def test_softmax_normalised_and_shift_invariant():
    c = micro(1)
    p = orc.router_probs(c["x"], c["w_router"])
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (p > 0).all()
    # adding the same vector to every router row adds a per-token constant to the logits
    shift = np.random.default_rng(7).standard_normal(c["x"].shape[1])
    p2 = orc.router_probs(c["x"], c["w_router"] + shift[None, :])
    np.testing.assert_allclose(p2, p, rtol=1e-12)


def test_softmax_matches_scalar_bruteforce():
    c = micro(2, T=6, d=9, N=5, Z=4)
    p = orc.router_probs(c["x"], c["w_router"])
    for t in range(6):
        _, pb = bruteforce.route_token(c["x"][t].tolist(), c["w_router"].tolist(), c["bias"].tolist(), 3)
        np.testing.assert_allclose(p[t], pb, rtol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_bruteforce(seed):
    c = micro(10 + seed, T=20, N=6, Z=5, K=4)
    idx, gate, p = orc.route(c["x"], c["w_router"], c["bias"], c["K"])
    for t in range(20):
        picks, pb = bruteforce.route_token(c["x"][t].tolist(), c["w_router"].tolist(), c["bias"].tolist(), c["K"])
        assert idx[t].tolist() == picks
        np.testing.assert_allclose(gate[t], [pb[i] for i in picks], rtol=1e-13)


def test_zero_input_uniform_router_picks_first_k():
    c = micro(3, N=5, Z=4, K=4)
    c["x"][:] = 0.0
    idx, gate, _ = orc.route(c["x"], c["w_router"], np.zeros(9), 4)
    assert (idx == np.arange(4)).all()
    np.testing.assert_allclose(gate, 1.0 / 9, rtol=1e-15)


def test_planted_bias_set_is_selected():
    c = micro(4, N=6, Z=5, K=3)
    b = np.zeros(11)
    S = [2, 7, 9]
    b[S] = 2.0
    idx, _, p = orc.route(c["x"], c["w_router"], b, 3)
    for t in range(idx.shape[0]):
        assert sorted(idx[t].tolist()) == S
        # inside S the order is by p (equal bias), descending
        assert list(idx[t]) == sorted(S, key=lambda i: (-p[t, i], i))


def test_duplicate_router_rows_tie_lower_index_first():
    c = micro(5, N=4, Z=3, K=7)
    c["w_router"][5] = c["w_router"][1]
    b = np.zeros(7)
    idx, _, _ = orc.route(c["x"], c["w_router"], b, 7)
    for t in range(idx.shape[0]):
        row = idx[t].tolist()
        assert row.index(1) + 1 == row.index(5)


def test_no_zero_experts_unbiased_is_topk_of_logits():
    c = micro(6, N=9, Z=0, K=4)
    idx, gate, _ = orc.route(c["x"], c["w_router"], np.zeros(9), 4)
    logits = c["x"] @ c["w_router"].T
    ref = np.argsort(-logits, axis=1)[:, :4]
    assert (idx == ref).all()


def test_bias_only_affects_selection_not_gates():
    c = micro(8, N=5, Z=3, K=8)  # K = E: every expert chosen whatever the bias
    idx0, g0, p = orc.route(c["x"], c["w_router"], np.zeros(8), 8)
    idx1, g1, _ = orc.route(c["x"], c["w_router"], np.linspace(-1, 1, 8), 8)
    for t in range(idx0.shape[0]):
        assert dict(zip(idx0[t], g0[t])) == pytest.approx(dict(zip(idx1[t], g1[t])), rel=0, abs=0)


# ---- load / permutation ----------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_load_and_ffn_count_invariants(seed):
    c = micro(20 + seed, T=50, N=5, Z=4, K=4, bias_scale=0.2)
    out = run_oracle(c)
    T, K, N = 50, 4, 5
    assert out["load"].sum() == T * K
    assert ((out["ffn_count"] >= 0) & (out["ffn_count"] <= K)).all()
    assert out["load"][:N].sum() == out["ffn_count"].sum() == out["offsets"][N]
    assert (out["load"] == np.bincount(out["idx"].ravel(), minlength=9)).all()


def test_permutation_properties():
    c = micro(30, T=64, N=5, Z=3, K=3, bias_scale=0.3)
    idx, _, _ = orc.route(c["x"], c["w_router"], c["bias"], 3)
    offsets, perm_token, slot_row = orc.permute(idx, 5)
    assert offsets[0] == 0 and (np.diff(offsets) >= 0).all()
    seen = set()
    for e in range(5):
        toks = perm_token[offsets[e]:offsets[e + 1]]
        assert (np.diff(toks) > 0).all()                # ascending, no repeats
        assert sorted(toks.tolist()) == sorted(np.nonzero((idx == e).any(axis=1))[0].tolist())
    for t in range(64):
        for k in range(3):
            if idx[t, k] < 5:
                r = slot_row[t, k]
                assert perm_token[r] == t and offsets[idx[t, k]] <= r < offsets[idx[t, k] + 1]
                assert r not in seen
                seen.add(r)
            else:
                assert slot_row[t, k] == -1
    assert len(seen) == perm_token.size


# ---- whole layer ------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_forward_matches_bruteforce_micro(seed):
    c = micro(40 + seed, T=10, d=8, N=3, Z=2, K=3, I=5, bias_scale=0.1)
    out = run_oracle(c)
    bidx, bgate, by = run_brute(c)
    assert out["idx"].tolist() == bidx
    np.testing.assert_allclose(out["gate"], bgate, rtol=1e-13)
    np.testing.assert_allclose(out["y"], by, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("Z", [0, 3])
def test_forward_matches_dense_masked(Z):
    c = micro(50 + Z, T=40, d=16, N=6, Z=Z, K=4, I=12)
    out = run_oracle(c)
    G = dense.gate_matrix(out["idx"], out["gate"], 6 + Z)
    y = dense.forward(c["x"], G, c["w_gate"], c["w_up"], c["w_down"], 6)
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-14)


def test_all_zero_selection_gives_gate_sum_times_x():
    c = micro(60, N=4, Z=3, K=3)
    b = np.array([-2.0] * 4 + [2.0] * 3)
    out = orc.moe_forward(c["x"], c["w_router"], b, lambda e: pytest.fail("FFN expert ran"), 4, 3)
    assert (out["idx"] >= 4).all() and (out["ffn_count"] == 0).all()
    np.testing.assert_allclose(out["y"], out["gate"].sum(axis=1, keepdims=True) * c["x"], rtol=1e-15)


def test_zero_up_projection_removes_ffn_term():
    c = micro(61, N=4, Z=3, K=3)
    c["w_up"][:] = 0.0
    out = run_oracle(c)
    zg = np.where(out["idx"] >= 4, out["gate"], 0.0).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out["y"], zg * c["x"], rtol=1e-15, atol=0)


def test_token_subset_equals_full_rows():
    c = micro(62, T=30, N=4, Z=3, K=3)
    full = run_oracle(c)
    sub = orc.moe_forward(c["x"], c["w_router"], c["bias"],
                          lambda e: (c["w_gate"][e], c["w_up"][e], c["w_down"][e]), 4, 3, tokens=[3, 17, 29])
    np.testing.assert_allclose(sub["y"], full["y"][[3, 17, 29]], rtol=1e-14)
    assert (sub["idx"] == full["idx"][[3, 17, 29]]).all()


def test_batches_share_one_pass_over_the_experts():
    """moe_forward_batches equals moe_forward on each batch alone (bitwise: the same steps
    per batch), fetches each expert's weights once, and splits y into the FFN part and
    the zero picks' gate sum times x."""
    c = micro(63, T=40, N=5, Z=3, K=3, bias_scale=0.2)
    d = micro(64, T=7, N=5, Z=3, K=3, bias_scale=0.2)
    e = micro(65, T=20, N=5, Z=3, K=3, bias_scale=0.2)
    W = (c["w_gate"], c["w_up"], c["w_down"])          # one layer's experts for all batches
    calls = []

    def experts(k):
        calls.append(k)
        return W[0][k], W[1][k], W[2][k]

    batches = [dict(x=b["x"], w_router=b["w_router"], bias=b["bias"], K=3) for b in (c, d)]
    batches.append(dict(x=e["x"], w_router=e["w_router"], bias=e["bias"], K=3, tokens=[0, 5, 19]))
    outs = orc.moe_forward_batches(batches, experts, 5)
    assert sorted(calls) == sorted(set(calls))            # once per expert
    for b, out in zip(batches, outs):
        one = orc.moe_forward(b["x"], b["w_router"], b["bias"], lambda k: (W[0][k], W[1][k], W[2][k]), 5, 3,
                              tokens=b.get("tokens"))
        for key in ("idx", "gate", "y", "y_ffn", "gz", "load", "offsets", "perm_token", "slot_row"):
            np.testing.assert_array_equal(out[key], one[key], err_msg=key)
        x = np.asarray(b["x"])[b["tokens"]] if b.get("tokens") is not None else np.asarray(b["x"])
        np.testing.assert_allclose(out["y"], out["y_ffn"] + out["gz"][:, None] * x, rtol=1e-13, atol=1e-15)
        zg = np.where(out["idx"] >= 5, out["gate"], 0.0).sum(axis=1)
        np.testing.assert_allclose(out["gz"], zg, rtol=1e-15)
    # and against the scalar brute force with that layer's experts
    bidx, _, by = bruteforce.forward(np.asarray(d["x"]).tolist(), np.asarray(d["w_router"]).tolist(),
                                     np.asarray(d["bias"]).tolist(), W[0].tolist(), W[1].tolist(),
                                     W[2].tolist(), 5, 3)
    assert outs[1]["idx"].tolist() == bidx
    np.testing.assert_allclose(outs[1]["y"], by, rtol=1e-12, atol=1e-14)


def test_permute_repeated_picks_get_one_row_each():
    """A caller's picks may repeat an expert within a token: every (token, pick) gets its
    own row, in (token, pick) order, and the load counts each pick."""
    idx = np.array([[2, 0, 2], [1, 7, 1], [2, 2, 2], [0, 5, 6]])
    offsets, perm_token, slot_row = orc.permute(idx, 5)
    assert offsets.tolist() == [0, 2, 4, 9, 9, 9]
    assert perm_token.tolist() == [0, 3, 1, 1, 0, 0, 2, 2, 2]
    assert slot_row.tolist() == [[4, 0, 5], [2, -1, 3], [6, 7, 8], [1, -1, -1]]
    assert orc.expert_load(idx, 8).tolist() == [2, 2, 5, 0, 0, 1, 1, 1]


# ---- the pins have teeth: plant mistakes in (a copy of) the oracle ------------------------

def _mutant_checks(monkeypatch, name, fn):
    monkeypatch.setattr(orc, name, fn)
    c = micro(70, T=10, d=8, N=3, Z=2, K=3, I=5, bias_scale=0.05)
    out = run_oracle(c)
    bidx, _, by = run_brute(c)
    return out["idx"].tolist() == bidx and np.allclose(out["y"], by, rtol=1e-12, atol=1e-14)


def test_planted_mistakes_are_caught(monkeypatch):
    real_silu, real_scores, real_expert = orc.silu, orc.selection_scores, orc.swiglu_expert
    mutants = {
        "silu": lambda a: a / (1.0 + np.exp(a)),                                  # sign error
        "selection_scores": lambda p, b: p.astype(np.float32) - np.asarray(b, np.float32)[None, :],
        "swiglu_expert": lambda X, wg, wu, wd: (real_silu(X @ wu.T) * (X @ wg.T)) @ wd.T,  # gate/up swapped
    }
    for name, fn in mutants.items():
        with monkeypatch.context() as m:
            assert not _mutant_checks(m, name, fn), f"mutant {name} not caught"
    assert orc.silu is real_silu and orc.selection_scores is real_scores and orc.swiglu_expert is real_expert
