"""Backward of the grouped SwiGLU FFN (lc_moe_ffn_backward) against the fp64 oracle
(oracle/backward.py), through the C-ABI.  The picks and gates are the oracle's routing of
the seeded inputs (gates rounded to fp32), given to both sides.  dx is compared on every
token and dW on every expert (relative L2 per matrix, the bf16 bound 2e-2); experts
without rows must get exact zeros; two calls give the same bits.  Shapes: one token block
(T <= 256) and several, ragged N-tiles (d = 160, I = 96), an expert spanning several
256-row M-tiles, empty experts, Z = 0, all-zero picks; then full-size decode and prefill
layers (dx on every token, dW on sampled experts incl. the most loaded)."""
import numpy as np
import pytest

from gpu_common import BF16_TOL, adhoc, audited, make_case, rel_l2, say, to_np
from inputs import configs
from inputs.generate import bf16_bits_to_f64, upstream_grad, weights_f64
from oracle import backward as ob
from oracle import moe as orc

pytestmark = pytest.mark.gpu


def run_backward(case, idx, gate32):
    import torch
    import mixture_experts_layer_router_amd as lm
    dev = case.x.device
    dy_bits = upstream_grad(case.wl)
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    out = lm.ffn_backward(case.x, case.w["gate"], case.w["up"], case.w["down"],
                          torch.from_numpy(idx.astype(np.int32)).to(dev), torch.from_numpy(gate32).to(dev),
                          dy, case.wl.Z)
    torch.cuda.synchronize()
    return out, bf16_bits_to_f64(dy_bits)


def routing(case):
    idx, gate, _ = orc.route(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, case.wl.K)
    return idx, gate.astype(np.float32)


def check(case, idx, gate32, out, dy, dw_experts=None):
    wl = case.wl
    cache = {}

    def experts(e):
        return tuple(weights_f64(case.w[k][e]) for k in ("gate", "up", "down"))

    dx_ref, dw_ref = ob.ffn_backward(case.ri.x_f64(), dy, idx, gate32.astype(np.float64), experts, wl.N,
                                     dw_experts=dw_experts)
    dx = to_np(out["dx"])
    err = rel_l2(dx, dx_ref)
    tok = np.linalg.norm(dx - dx_ref, axis=1) / np.maximum(np.linalg.norm(dx_ref, axis=1), 1e-30)
    worst_dw = 0.0
    for e, (g, u, d) in dw_ref.items():
        for name, ref in (("dw_gate", g), ("dw_up", u), ("dw_down", d)):
            got = to_np(out[name][e])
            ew = rel_l2(got, ref)
            worst_dw = max(worst_dw, ew)
            assert ew <= BF16_TOL, (e, name, ew)
    load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
    empty = np.nonzero(load == 0)[0]
    for e in empty[:16]:
        for name in ("dw_gate", "dw_up", "dw_down"):
            assert not bool(out[name][int(e)].any()), (int(e), name)
    say(f"   dx rel L2 {err:.2e} (worst token {tok.max():.2e}); dW worst {worst_dw:.2e} over {len(dw_ref)} "
        f"experts; {empty.size} empty experts zero")
    assert err <= BF16_TOL and tok.max() <= BF16_TOL
    return err


CASES = [dict(T=300, d=256, N=12, Z=5, K=4, I=192), dict(T=64, d=128, N=8, Z=4, K=3, I=96),
         dict(T=700, d=160, N=6, Z=3, K=3, I=96), dict(T=257, d=64, N=9, Z=0, K=2, I=64),
         # experts of about 500 rows (two 256-row M-tiles, the second ragged); d and I past
         # one 256-wide tile, both ragged
         dict(T=1500, d=320, N=4, Z=2, K=3, I=288)]


@pytest.mark.parametrize("kw", CASES, ids=lambda k: f"T{k['T']}_d{k['d']}_I{k['I']}_Z{k['Z']}")
def test_backward_matches_oracle(kw):
    wl = adhoc(name=f"bwd_{kw['T']}_{kw['d']}", seed_key=(700, kw["T"]), expert_std=1 / np.sqrt(kw["d"]),
               bias=("uniform", 0.3), **kw)
    say(f"[backward] {wl.name}: T={wl.T} d={wl.d} N={wl.N} Z={wl.Z} K={wl.K} I={wl.I}")
    case = make_case(wl, ri=audited(wl))
    idx, gate32 = routing(case)
    load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
    say(f"   expert rows: max {load.max()}, empty {int((load == 0).sum())}")
    out, dy = run_backward(case, idx, gate32)
    check(case, idx, gate32, out, dy)
    out2, _ = run_backward(case, idx, gate32)
    import torch
    for k in out:
        assert torch.equal(out[k].view(torch.int16), out2[k].view(torch.int16)), k


def test_backward_all_zero_picks():
    import torch
    wl = adhoc(name="bwd_allzero", T=100, d=64, N=4, Z=3, K=3, I=64, seed_key=(701,), expert_std=0.125)
    case = make_case(wl, ri=audited(wl))
    idx = np.tile(np.array([4, 5, 6]), (wl.T, 1))
    gate32 = np.random.default_rng(7).uniform(0.1, 0.3, (wl.T, 3)).astype(np.float32)
    out, dy = run_backward(case, idx, gate32)
    for name in ("dw_gate", "dw_up", "dw_down"):
        assert not bool(out[name].any())
    want = gate32.astype(np.float64).sum(1, keepdims=True) * dy
    assert rel_l2(to_np(out["dx"]), want) <= 2 ** -8


@pytest.mark.parametrize("name", ["decode_T256_z33", "prefill"])
def test_backward_full_size(name):
    """dx on every token; dW on the most loaded expert, a median one and the least loaded
    one with rows."""
    wl = configs.get(name)
    say(f"[backward full size] {wl.description}")
    case = make_case(wl)
    idx, gate32 = routing(case)
    load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
    has = np.nonzero(load > 0)[0]
    order = has[np.argsort(load[has], kind="stable")]
    pick = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    out, dy = run_backward(case, idx, gate32)
    check(case, idx, gate32, out, dy, dw_experts=set(pick))
