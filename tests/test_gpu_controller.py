"""GPU parity of the expert-bias controller (lc_moe_bias_update) against the fp64 oracle
(oracle/controller.py), one step and in closed loop with the GPU router."""
import numpy as np
import pytest

from oracle import controller as ctl
from oracle import moe as orc
from tests.gpu_common import device, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def tolerance(b, integral_old, integral_new, e, prev, tgt, share, kp, ki, kd):
    """Bound on |b_gpu - b_oracle| for one fp32 step: the share load/(T*K) is rounded (and
    T*K itself when above 2^24) and enters e with the magnitude of the share and the
    target, e enters the three terms, and each add and multiply rounds once."""
    mag = (np.abs(b) + (abs(kp) + abs(ki) + abs(kd)) * (np.abs(tgt) + np.abs(share))
           + abs(ki) * (np.abs(integral_old) + np.abs(integral_new)) + abs(kd) * (np.abs(e) + np.abs(prev))
           + abs(kp) * np.abs(e))
    return 6 * U * mag + 1e-30


def check_bias(got, ref, tol, what):
    ratio = np.abs(np.asarray(got, np.float64) - ref) / tol
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= 1.0, f"{what}: expert {worst} off by {ratio[worst]:.2f}x the bound"


@pytest.mark.parametrize("gains", [(0.5, 0.05, 0.0), (2.0, 0.0, 0.7), (0.0, 1.5, 0.0), (1.0, 0.2, 0.3)])
def test_bias_update_one_step(gains):
    import torch
    import mixture_experts_layer_router_amd as lm
    dev = device()
    rng = np.random.default_rng(11)
    T, K, N, Z = 16384, 12, 512, 256
    E = N + Z
    say(f"bias update E={E} gains={gains}")
    tgt = ctl.share_targets(N, Z, 1 / 3).astype(np.float32)
    load = rng.multinomial(T * K, np.full(E, 1 / E)).astype(np.int32)
    b = rng.normal(0, 1e-3, E).astype(np.float32)
    integ = rng.normal(0, 1e-3, E).astype(np.float32)
    prev = rng.normal(0, 1e-4, E).astype(np.float32)
    tb, ti, tp = (torch.tensor(a, device=dev) for a in (b, integ, prev))
    lm.bias_update(torch.tensor(load, device=dev), torch.tensor(tgt, device=dev), tb, ti, tp, T, K, N, *gains)
    rb, ri, rp = ctl.pid_step(b, integ, prev, load, tgt, T, K, *gains)
    gb, gi, gp = (t.cpu().numpy().astype(np.float64) for t in (tb, ti, tp))
    share = load / float(T * K)
    check_bias(gp, rp, 4 * U * (np.abs(tgt) + share) + 1e-30, "prev_err")
    check_bias(gi, ri, 4 * U * (np.abs(tgt) + share + np.abs(integ) + np.abs(ri)) + 1e-30, "integral")
    check_bias(gb, rb, tolerance(b, integ, ri, rp, prev, tgt, share, *gains), "bias")


def test_bias_update_zero_pool_and_edges():
    """Z = 0 and a single-expert pool; loads at the extremes (all picks on one expert)."""
    import torch
    import mixture_experts_layer_router_amd as lm
    dev = device()
    for T, K, N, Z in ((7, 1, 1, 0), (33, 3, 5, 0), (1, 4, 2, 3)):
        E = N + Z
        say(f"bias update edge T={T} K={K} N={N} Z={Z}")
        tgt = ctl.share_targets(N, Z, 0.4).astype(np.float32)
        load = np.zeros(E, np.int32)
        load[E - 1] = T * K
        z = np.zeros(E, np.float32)
        tb, ti, tp = (torch.tensor(z, device=dev) for _ in range(3))
        lm.bias_update(torch.tensor(load, device=dev), torch.tensor(tgt, device=dev), tb, ti, tp, T, K, N, 1.0, 0.5, 0.25)
        rb, ri, rp = ctl.pid_step(z, z, z, load, tgt, T, K, 1.0, 0.5, 0.25)
        np.testing.assert_allclose(tb.cpu().numpy(), rb, rtol=4 * U, atol=1e-12)
        np.testing.assert_allclose(ti.cpu().numpy(), ri, rtol=4 * U, atol=1e-12)
        np.testing.assert_allclose(tp.cpu().numpy(), rp, rtol=4 * U, atol=1e-12)


def test_closed_loop_on_gpu():
    """GPU router -> GPU loads -> GPU controller for 60 steps on fresh seeded tokens.  Each
    step's picks equal the oracle's routing under the GPU's bias (tokens whose scores are
    too close to order reliably are skipped; a few per thousand), the loads are the
    histogram of the picks, each bias update matches the oracle's, and the zero share
    settles on its target."""
    import torch
    import mixture_experts_layer_router_amd as lm
    dev = device()
    T, K, N, Z, d = 512, 4, 16, 8, 64
    E = N + Z
    rng = np.random.default_rng(5)
    wr = rng.normal(0, 1 / np.sqrt(d), (E, d)).astype(np.float32)
    tgt = ctl.share_targets(N, Z, 0.5).astype(np.float32)
    gains = (0.5, 0.05, 0.0)
    twr, ttgt = torch.tensor(wr, device=dev), torch.tensor(tgt, device=dev)
    tb, ti, tp = (torch.zeros(E, dtype=torch.float32, device=dev) for _ in range(3))
    shape = lm.make_shape(T, d, N, Z, K, 8, lm.F32)
    ws = lm.workspace_for(shape, dev)
    zs, compared = [], 0
    for step in range(60):
        x = rng.normal(0, 1, (T, d)).astype(np.float32)
        b_before = tb.cpu().numpy().copy()
        i_before, p_before = ti.cpu().numpy().copy(), tp.cpu().numpy().copy()
        idx, _ = lm.route(torch.tensor(x, device=dev), twr, tb, K, N, workspace=ws)
        load, _ = lm.expert_load(idx, N, E, workspace=ws, d=d, dtype=lm.F32)
        lm.bias_update(load, ttgt, tb, ti, tp, T, K, N, *gains)
        gl = load.cpu().numpy()
        p = orc.router_probs(x.astype(np.float64), wr.astype(np.float64))
        ok = orc.selection_margin_ok(p, b_before, K)
        ridx = orc.select_topk(orc.selection_scores(p, b_before), K)
        np.testing.assert_array_equal(idx.cpu().numpy()[ok], ridx[ok])
        np.testing.assert_array_equal(gl, orc.expert_load(idx.cpu().numpy(), E))
        compared += int(ok.sum())
        rb, ri, rp = ctl.pid_step(b_before, i_before, p_before, gl, tgt, T, K, *gains)
        check_bias(tb.cpu().numpy(), rb, tolerance(b_before, i_before, ri, rp, p_before, tgt,
                                                   gl / float(T * K), *gains), f"bias step {step}")
        zs.append(gl[N:].sum() / (T * K))
    say(f"closed loop: {compared}/{60 * T} tokens compared with the oracle's routing; "
        f"zero share {zs[0]:.3f} -> {np.mean(zs[-10:]):.4f}")
    assert compared >= 0.99 * 60 * T
    assert abs(np.mean(zs[-10:]) - 0.5) < 0.01
