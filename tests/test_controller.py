"""The expert-bias controller oracle (oracle/controller.py) against closed forms of the
discrete PID law and against the closed-loop behaviour the pages describe: the bias
follows usage so that the picks settle on their targets (LongCat-Flash article, section
"Zero-computation experts", bias paragraph)."""
import numpy as np
import pytest

from oracle import controller as ctl
from oracle import moe as orc

T, K, N, Z = 512, 4, 16, 8
E = N + Z


def const_load():
    """A fixed load vector off target: the first expert gets 3 extra picks from the last."""
    tgt = ctl.share_targets(N, Z, 0.25)
    load = np.round(tgt * T * K).astype(np.int64)
    load[0] += 3
    load[-1] -= 3
    assert load.sum() == T * K
    return load, tgt


def run(load, tgt, steps, kp, ki, kd, b0=0.1):
    b, i, pe = np.full(E, b0), np.zeros(E), np.zeros(E)
    out = []
    for _ in range(steps):
        b, i, pe = ctl.pid_step(b, i, pe, load, tgt, T, K, kp, ki, kd)
        out.append(b.copy())
    return out


def test_share_targets():
    t = ctl.share_targets(N, Z, 0.25)
    assert t.sum() == pytest.approx(1.0, abs=1e-15)
    assert np.all(t[:N] == t[0]) and t[0] * N == pytest.approx(0.75)
    assert t[N:].sum() == pytest.approx(0.25)
    t0 = ctl.share_targets(N, 0, 0.25)
    assert t0.size == N and t0.sum() == pytest.approx(1.0)


def test_proportional_only_is_linear_in_steps():
    load, tgt = const_load()
    e = tgt - load / (T * K)
    bs = run(load, tgt, 7, kp=0.8, ki=0.0, kd=0.0)
    for n, b in enumerate(bs, 1):
        np.testing.assert_allclose(b, 0.1 + n * 0.8 * e, rtol=0, atol=1e-15)
    assert bs[0][0] < 0.1 and bs[0][-1] > 0.1       # over-used expert loses bias, under-used gains


def test_integral_only_is_triangular():
    load, tgt = const_load()
    e = tgt - load / (T * K)
    bs = run(load, tgt, 6, kp=0.0, ki=0.3, kd=0.0)
    for n, b in enumerate(bs, 1):
        np.testing.assert_allclose(b, 0.1 + 0.3 * e * n * (n + 1) / 2, rtol=0, atol=1e-15)


def test_derivative_only_kicks_once():
    load, tgt = const_load()
    e = tgt - load / (T * K)
    bs = run(load, tgt, 4, kp=0.0, ki=0.0, kd=2.0)
    np.testing.assert_allclose(bs[0], 0.1 + 2.0 * e, rtol=0, atol=1e-15)
    for b in bs[1:]:
        np.testing.assert_array_equal(b, bs[0])


def test_at_set_point_nothing_moves():
    tgt = ctl.share_targets(N, Z, 0.25)
    load = np.round(tgt * T * K).astype(np.int64)
    assert np.all(load / (T * K) == tgt)
    b, i, pe = ctl.pid_step(np.full(E, -0.2), np.zeros(E), np.zeros(E), load, tgt, T, K, 1.0, 1.0, 1.0)
    assert np.all(b == -0.2) and np.all(i == 0) and np.all(pe == 0)


def closed_loop(step_fn, steps=80, zero_share=0.5, gains=(0.5, 0.05, 0.0), seed=0):
    rng = np.random.default_rng(seed)
    d = 64
    wr = rng.normal(0, 1 / np.sqrt(d), (E, d))
    tgt = ctl.share_targets(N, Z, zero_share)
    b, i, pe = np.zeros(E), np.zeros(E), np.zeros(E)
    zs, cv = [], []
    for _ in range(steps):
        x = rng.normal(0, 1, (T, d))
        idx, _, _ = orc.route(x, wr, b.astype(np.float32), K)
        load = orc.expert_load(idx, E)
        zs.append(load[N:].sum() / (T * K))
        cv.append(load[:N].std() / load[:N].mean())
        b, i, pe = step_fn(b, i, pe, load, tgt, T, K, *gains)
    return np.array(zs), np.array(cv)


def test_closed_loop_reaches_the_zero_share_and_balances():
    zs, cv = closed_loop(ctl.pid_step)
    assert abs(zs[0] - Z / E) < 0.05                 # starts near the unbiased share 1/3
    assert abs(zs[-10:].mean() - 0.5) < 0.01          # settles on the 50% target
    assert cv[-10:].mean() < 0.85 * cv[:5].mean()      # FFN loads even out


def test_closed_loop_catches_a_sign_error():
    def flipped(b, i, pe, load, tgt, T_, K_, kp, ki, kd):
        return ctl.pid_step(b, i, pe, 2 * np.asarray(tgt) * T_ * K_ - load, tgt, T_, K_, kp, ki, kd)
    zs, _ = closed_loop(flipped, steps=30)
    assert abs(zs[-10:].mean() - 0.5) > 0.1
