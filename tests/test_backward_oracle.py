"""Pins of the FFN backward oracle (oracle.backward), no GPU.

  * central finite differences of L = sum <dy, y> through the oracle's own forward pieces
    (permutation, SwiGLU expert, combine; already pinned in test_oracle_pins.py) with the
    picks and gates held fixed, in x and in sampled entries of every expert matrix;
  * torch autograd (fp64, CPU) of an independently written dense-masked form of the layer
    (every expert on every token, times the one-hot gate matrix), for dx and every dW;
  * the closed form at d = I = 1;
  * invariants: all-zero picks give dx = (sum of gates) * dy and no weight gradient;
    experts without rows get none;
  * planted mistakes (a wrong silu derivative, gate/up swapped) are caught.
"""
import math

import numpy as np
import pytest

from oracle import backward as ob
from oracle import moe as orc


def micro(seed, T=9, d=6, N=3, Z=2, K=3, I=5, bias_scale=0.2):
    g = np.random.default_rng(seed)
    E = N + Z
    c = dict(x=g.standard_normal((T, d)), w_router=g.standard_normal((E, d)) / math.sqrt(d),
             bias=g.uniform(-bias_scale, bias_scale, E).astype(np.float32).astype(np.float64),
             w_gate=g.standard_normal((N, I, d)) / math.sqrt(d), w_up=g.standard_normal((N, I, d)) / math.sqrt(d),
             w_down=g.standard_normal((N, d, I)) / math.sqrt(I), dy=g.standard_normal((T, d)), N=N, K=K)
    idx, gate, _ = orc.route(c["x"], c["w_router"], c["bias"], K)
    c["idx"], c["gate"] = idx, gate
    return c


def fixed_route_loss(x, wg, wu, wd, c):
    """L = sum <dy, y> with the picks and gates of c held fixed (the oracle's forward pieces)."""
    offsets, perm_token, slot_row = orc.permute(c["idx"], c["N"])
    y_perm = np.zeros((perm_token.size, x.shape[1]))
    for e in range(c["N"]):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            y_perm[r0:r1] = orc.swiglu_expert(x[perm_token[r0:r1]], wg[e], wu[e], wd[e])
    y = orc.combine(x, y_perm, c["idx"], c["gate"], slot_row, c["N"])
    return float((c["dy"] * y).sum())


def run(c, **kw):
    return ob.ffn_backward(c["x"], c["dy"], c["idx"], c["gate"],
                           lambda e: (c["w_gate"][e], c["w_up"][e], c["w_down"][e]), c["N"], **kw)


@pytest.mark.parametrize("seed", range(3))
def test_finite_differences(seed):
    c = micro(80 + seed)
    dx, dw = run(c)
    h = 1e-6
    args = [c["x"].copy(), c["w_gate"].copy(), c["w_up"].copy(), c["w_down"].copy()]
    grads = [dx] + [np.stack([dw[e][m] if e in dw else np.zeros_like(args[m + 1][e]) for e in range(c["N"])])
                    for m in range(3)]
    g = np.random.default_rng(seed)
    for a, grad in zip(range(4), grads):
        arr = args[a]
        picks = [tuple(int(v) for v in np.unravel_index(i, arr.shape)) for i in g.choice(arr.size, 12, replace=False)]
        for p in picks:
            old = arr[p]
            arr[p] = old + h
            lp = fixed_route_loss(*args, c)
            arr[p] = old - h
            lm = fixed_route_loss(*args, c)
            arr[p] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[p]) <= 1e-6 * (1 + abs(fd)), (a, p, fd, grad[p])


@pytest.mark.parametrize("Z", [0, 2])
def test_torch_autograd_of_dense_masked_form(Z):
    import torch
    c = micro(90 + Z, T=14, d=8, N=4, Z=Z, K=3, I=6)
    dx, dw = run(c)
    E = c["N"] + Z
    Gm = np.zeros((c["x"].shape[0], E))
    np.put_along_axis(Gm, c["idx"].astype(np.int64), c["gate"], axis=1)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    x, wg, wu, wd = t(c["x"]), t(c["w_gate"]), t(c["w_up"]), t(c["w_down"])
    Gt = torch.tensor(Gm)
    y = Gt[:, c["N"]:].sum(dim=1, keepdim=True) * x
    for e in range(c["N"]):
        gpre = x @ wg[e].T
        y = y + Gt[:, e:e + 1] * ((torch.nn.functional.silu(gpre) * (x @ wu[e].T)) @ wd[e].T)
    (torch.tensor(c["dy"]) * y).sum().backward()
    np.testing.assert_allclose(dx, x.grad.numpy(), rtol=1e-12, atol=1e-13)
    for e in range(c["N"]):
        if e in dw:
            for m, ref in enumerate((wg.grad[e], wu.grad[e], wd.grad[e])):
                np.testing.assert_allclose(dw[e][m], ref.numpy(), rtol=1e-12, atol=1e-13)
        else:
            assert float(wg.grad[e].abs().max()) == 0.0


def test_closed_form_d1_i1():
    """d = I = 1, one FFN expert, K = 1, gate g: y = g * w_d * silu(w_g x) * (w_u x)."""
    x, wg, wu, wd, g, dy = 0.7, 1.3, -0.4, 2.1, 0.6, 1.5
    G, U = wg * x, wu * x
    s = 1 / (1 + math.exp(-G))
    a = G * s
    H = a * U
    dH = wd * g * dy
    dG = dH * U * (s + a * (1 - s))
    dU = dH * a
    want = dict(dx=dG * wg + dU * wu, dwg=dG * x, dwu=dU * x, dwd=g * dy * H)
    dx, dw = ob.ffn_backward(np.array([[x]]), np.array([[dy]]), np.array([[0]]), np.array([[g]]),
                             lambda e: (np.array([[wg]]), np.array([[wu]]), np.array([[wd]])), 1)
    assert dx[0, 0] == pytest.approx(want["dx"], rel=1e-14)
    assert dw[0][0][0, 0] == pytest.approx(want["dwg"], rel=1e-14)
    assert dw[0][1][0, 0] == pytest.approx(want["dwu"], rel=1e-14)
    assert dw[0][2][0, 0] == pytest.approx(want["dwd"], rel=1e-14)
    # by hand: silu'(G) = s (1 + G (1 - s)) at G = 0.91
    assert (s + a * (1 - s)) == pytest.approx(s * (1 + G * (1 - s)), rel=1e-15)


def test_all_zero_picks_and_empty_experts():
    c = micro(95, N=4, Z=3, K=3)
    c["idx"] = np.array([[4, 5, 6]] * c["x"].shape[0])
    dx, dw = run(c)
    assert dw == {}
    np.testing.assert_allclose(dx, c["gate"].sum(axis=1, keepdims=True) * c["dy"], rtol=1e-15)
    c = micro(96, N=4, Z=3, K=2)
    c["idx"][:, 0] = 1
    c["idx"][:, 1] = 5
    dx, dw = run(c)
    assert set(dw) == {1}


def test_planted_mistakes_are_caught(monkeypatch):
    c = micro(97)
    ref_dx, _ = run(c)

    def wrong_silu_grad(X, dY, wg, wu, wd, want_dw=True):  # silu'(G) taken as sigmoid(G)
        G, U = X @ wg.T, X @ wu.T
        s = ob.sigmoid(G)
        dH = dY @ wd
        dG, dU = dH * U * s, dH * G * s
        return dG @ wg + dU @ wu, dG.T @ X, dU.T @ X, dY.T @ (G * s * U)

    def swapped(X, dY, wg, wu, wd, want_dw=True):
        return real(X, dY, wu, wg, wd, want_dw)

    real = ob.expert_backward
    for fn in (wrong_silu_grad, swapped):
        with monkeypatch.context() as m:
            m.setattr(ob, "expert_backward", fn)
            dx, _ = run(c)
        assert not np.allclose(dx, ref_dx, rtol=1e-6), fn.__name__
