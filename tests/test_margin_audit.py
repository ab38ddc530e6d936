"""Pins of the selection-margin audit (oracle.moe.selection_margin_ok), no GPU.

The audit decides which synthetic tokens are well posed for bit-exact routing: a token
passes when every adjacent pair among its first K+1 selection scores (in the order
s descending, index ascending) is separated by more than
    rel * (p_j + p_j+1) + ulp_rel * (|s_j| + |s_j+1|).
These tests check it against a scalar brute-force scan written from that rule, against
planted near-ties on each side of the threshold at every position of the top K+1, and
against its purpose: any perturbation of p within half the relative margin, followed by
the fp32 rounding of p and of s = p + b, leaves the top-K of every passing token unchanged.
"""
import math

import numpy as np
import pytest

from oracle import moe as orc

REL, ULP = 1e-4, 1e-6


def brute_margin_ok(p_row, b_row, K, rel=REL, ulp_rel=ULP):
    """Scalar scan: sort all experts by (s desc, index asc), check the K gaps of the top K+1."""
    s = [float(p) + float(b) for p, b in zip(p_row, b_row)]
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))[:K + 1]
    for a, c in zip(order[:-1], order[1:]):
        gap = s[a] - s[c]
        need = rel * (float(p_row[a]) + float(p_row[c])) + ulp_rel * (abs(s[a]) + abs(s[c]))
        if not gap > need:
            return False
    return True


def random_tokens(T, E, seed, bias_scale=0.02, K=6, planted_frac=0.3):
    """Softmax rows and a bias vector; in a fraction of the tokens one pair of adjacent
    top-(K+1) scores is pulled to within 0..3 times the rule's threshold of each other."""
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E)) * 2.0
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    b = g.uniform(-bias_scale, bias_scale, E)
    for t in np.nonzero(g.random(T) < planted_frac)[0]:
        s = p[t] + b
        order = sorted(range(E), key=lambda i: (-s[i], i))
        q = int(g.integers(0, min(K, E - 1)))
        a, c = order[q], order[q + 1]
        need = REL * 2 * p[t, a] + ULP * 2 * abs(s[a])
        p[t, c] = max(s[a] - b[c] - g.uniform(0.0, 3.0) * need, 0.0)
    return p, b


@pytest.mark.parametrize("T,E,K,seed", [(400, 12, 2, 0), (300, 96, 6, 1), (200, 40, 8, 2)])
def test_matches_bruteforce_scan(T, E, K, seed):
    p, b = random_tokens(T, E, seed, K=K)
    got = orc.selection_margin_ok(p, b, K)
    want = np.array([brute_margin_ok(p[t], b, K) for t in range(T)])
    np.testing.assert_array_equal(got, want)
    assert 0 < got.sum() < T          # both outcomes occur on these inputs


def planted(K, E, pos, factor):
    """One token whose top K+1 scores are well separated except positions pos, pos+1, whose
    gap is `factor` times the rule's threshold for that pair."""
    p = np.full(E, 0.2 / (E - K - 1))
    top = np.linspace(0.5, 0.2, K + 1)       # descending, gaps of 0.3/K >> threshold
    p[:K + 1] = top / top.sum() * 0.8
    b = np.zeros(E)
    j, k = pos, pos + 1
    need = REL * (p[j] + p[k]) + ULP * (abs(p[j] + b[j]) + abs(p[k] + b[k]))
    # move expert k's bias so that s_j - s_k = factor * need (p unchanged)
    b[k] = (p[j] + b[j]) - factor * need - p[k]
    # the threshold depends on |s_k| too: iterate to the fixed point
    for _ in range(50):
        need = REL * (p[j] + p[k]) + ULP * (abs(p[j] + b[j]) + abs(p[k] + b[k]))
        b[k] = (p[j] + b[j]) - factor * need - p[k]
    return p[None, :], b


@pytest.mark.parametrize("K", [1, 4, 12])
def test_planted_near_ties_at_every_position(K):
    E = 3 * K + 8
    for pos in range(K):                                  # every adjacent pair of the top K+1
        p, b = planted(K, E, pos, 0.999)
        assert not orc.selection_margin_ok(p, b, K)[0], (K, pos)
        assert not brute_margin_ok(p[0], b, K)
        p, b = planted(K, E, pos, 1.001)
        assert orc.selection_margin_ok(p, b, K)[0], (K, pos)
        assert brute_margin_ok(p[0], b, K)


def test_pair_beyond_the_first_k_plus_one_is_ignored():
    """A tie outside the first K+1 scores (between unselected experts) does not matter."""
    p = np.array([[0.4, 0.25, 0.15, 0.1, 0.05, 0.05]])
    b = np.zeros(6)
    assert orc.selection_margin_ok(p, b, 3)[0]           # tie at 0-based positions 4/5
    assert orc.selection_margin_ok(p, b, 4)[0]           # position 5 is the first not checked
    assert not orc.selection_margin_ok(p, b, 5)[0]       # now the tie decides the K-th pick


def test_exact_tie_fails():
    p = np.array([[0.3, 0.3, 0.2, 0.2]])
    b = np.zeros(4)
    assert not orc.selection_margin_ok(p, b, 1)[0]
    assert not orc.selection_margin_ok(p, b, 3)[0]


def test_bias_scale_term():
    """With a large bias |s| is large while p is small: the ulp_rel term decides."""
    p = np.array([[0.01, 0.01, 0.98]])
    s_gap_needed = REL * 0.02 + ULP * (2 * 5.0)
    b = np.array([5.0, 5.0 - 0.9 * s_gap_needed, -5.0])
    assert not orc.selection_margin_ok(p, b, 1)[0]
    b[1] = 5.0 - 1.2 * s_gap_needed
    assert orc.selection_margin_ok(p, b, 1)[0]
    # without the ulp term (a plausible slip) the first case would pass
    assert orc.selection_margin_ok(p, np.array([5.0, 5.0 - 0.9 * s_gap_needed, -5.0]), 1, ulp_rel=0.0)[0]


@pytest.mark.parametrize("seed", [3, 4])
def test_passing_tokens_survive_fp32_perturbation(seed):
    """The audit's purpose.  Each p_i is perturbed by a relative error of up to rel/2 (the
    GPU's fp32 softmax error is below 2e-5), rounded to fp32, and b is added in fp32: the
    top-K of every token that passed must equal the unperturbed fp32 selection."""
    T, E, K = 2000, 64, 6
    p, b = random_tokens(T, E, seed, bias_scale=0.002, K=K)
    ok = orc.selection_margin_ok(p, b, K)
    ref = orc.select_topk(orc.selection_scores(p, b), K)
    g = np.random.default_rng(seed + 100)
    changed_fail = 0
    for trial in range(5):
        delta = g.uniform(-0.5 * REL, 0.5 * REL, p.shape)
        pp = p * (1.0 + delta)
        got = orc.select_topk(orc.selection_scores(pp, b), K)
        diff = (got != ref).any(1)
        assert not (diff & ok).any(), f"trial {trial}: a passing token changed its top-K"
        changed_fail += int((diff & ~ok).sum())
    # the perturbation is strong enough to reorder some of the rejected tokens
    assert (~ok).sum() > 0 and changed_fail > 0


def test_margin_rule_uses_fp64_gap_not_fp32():
    """s is formed in fp64 for the gap: a gap of 1e-9 that fp32 would round away is still
    measured (and rejected), not mistaken for an exact tie resolved by index."""
    p = np.array([[0.5, 0.5 - 1e-9, 0.0]])
    b = np.zeros(3)
    assert not orc.selection_margin_ok(p, b, 1)[0]
    assert math.isclose(float(p[0, 0] - p[0, 1]), 1e-9, rel_tol=1e-6)
