"""Seeded random shapes through every path each shape admits, against the fp64 oracle.

The shapes are drawn once from a fixed seed within the header's limits: bf16 (d and I
multiples of 8, half of them multiples of 64) and fp32 (multiples of 4), 1 to 64 FFN
experts, 0 to 20 zero experts, K from 1 to 8, T from 1 to 2500 (one token block or
several, the 64-row and 320-row tile forms, experts over several M-tiles).  Each shape runs:
  * the layer on row-major weights: picks bit-exact, output within the bf16 (fp32) bound
    per token and pooled; the permutation of the oracle's picks exact; the staged and the
    allocation-free forwards, and replays of the forward captured in a HIP graph (two input
    sets in turn, eager work between replays), bitwise equal to it;
  * for d and I multiples of 32: the layer on packed weights and on block-FP8 weights, and
    the FFN backward (dx per token, dW per expert);
  * for d and I multiples of 64: the FP8 MFMA layer (FP8 activations).
The checks are those of the dedicated tests (test_gpu_parity, test_gpu_packed,
test_gpu_fp8, test_gpu_fp8_mfma, test_gpu_backward); this file adds the breadth of shapes.
Routing inputs are audited as everywhere (near-tie tokens redrawn)."""
import numpy as np
import pytest

from tests import test_gpu_backward as tb
from tests import test_gpu_fp8 as t8
from tests import test_gpu_fp8_mfma as tm
from oracle import moe as orc
from tests.gpu_common import BF16_TOL, F32_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, to_np, \
    worst_token_rel

pytestmark = pytest.mark.gpu


def _shapes(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        unit = 4 if dtype == "f32" else (64 if rng.random() < 0.5 else 8)
        d = int(unit * rng.integers(1, max(2, 640 // unit)))
        I = int(unit * rng.integers(1, max(2, 640 // unit)))
        N = int(rng.choice([1, 2, 3, 5, 8, 12, 17, 33, 64]))
        Z = int(rng.choice([0, 0, 1, 2, 5, 9, 20]))
        K = int(rng.integers(1, min(8, N + Z) + 1))
        T = int(rng.choice([1, 2, 3, 7, 31, 64, 65, 100, 255, 256, 257, 300, 513, 700, 1000, 1600, 2500]))
        out.append((dtype, T, d, I, N, Z, K))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=lambda i: "{}_T{}_d{}_I{}_N{}_Z{}_K{}".format(*SHAPES[i]))
def test_random_shape(i):
    import mixture_experts_layer_router_amd as lm
    dtype, T, d, I, N, Z, K = SHAPES[i]
    say(f"[sweep {i}] {dtype} T={T} d={d} I={I} N={N} Z={Z} K={K}")
    wl = adhoc(name=f"sweep{i}", T=T, d=d, N=N, Z=Z, K=K, I=I, dtype=dtype, seed_key=(910, i, T, d, I),
               expert_std=1 / np.sqrt(d), bias=("uniform", 0.5 / (N + Z)))
    case = make_case(wl, ri=audited(wl))
    ref = oracle_forward(case)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], K)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), ref["idx"])
    y = to_np(out["y"])
    err, worst = rel_l2(y, ref["y"]), worst_token_rel(y, ref["y"])
    say(f"   layer rel L2 {err:.2e} (worst token {worst:.2e})")
    assert err <= tol and (dtype == "f32" or worst <= tol)
    _check_permute(case, ref["idx"])
    _check_same_bits(case, out)
    _check_graph(case, out)
    if dtype != "bf16" or d % 32 or I % 32:
        return
    p = lm.pack_weights(case.w["gate"], case.w["up"], case.w["down"])
    yp = to_np(lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], K,
                         packed=p)["y"])
    assert rel_l2(yp, ref["y"]) <= BF16_TOL and worst_token_rel(yp, ref["y"]) <= BF16_TOL
    del p
    q = lm.quantize_weights(case.w["gate"], case.w["up"], case.w["down"])
    y8 = to_np(lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], K,
                         fp8=q)["y"])
    r8 = t8.oracle_fp8_forward(case)
    e8 = rel_l2(y8, r8["y"])
    say(f"   FP8-weight layer rel L2 {e8:.2e}")
    assert e8 <= BF16_TOL
    if d % 64 == 0 and I % 64 == 0:
        got = tm.run(case, q)
        tm.check_layer(got["y"], got["topk_idx"], tm.act_oracle(case), "   FP8 MFMA layer")
    del q
    idx, gate32 = tb.routing(case)
    bo, dy = tb.run_backward(case, idx, gate32)
    tb.check(case, idx, gate32, bo, dy)


def _check_permute(case, ridx):
    """lc_moe_permute on the oracle's picks: offsets, permutation and slots exact, the rows
    past the FFN rows untouched, the gathered rows bit-exact."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = case.wl
    out = lm.permute(case.x, torch.from_numpy(ridx.astype(np.int32)).to(case.x.device), wl.N, wl.E)
    offsets, perm_token, slot_row = orc.permute(ridx, wl.N)
    nnz = int(offsets[-1])
    assert (to_np(out["ffn_offsets"]) == offsets).all()
    pt = to_np(out["perm_token"])
    assert (pt[:nnz] == perm_token).all() and (pt[nnz:] == -7).all()
    assert (to_np(out["slot_row"]) == slot_row).all()
    assert (to_np(out["load"]) == orc.expert_load(ridx, wl.E)).all()
    xp, xr = out["x_perm"][:nnz], case.x[torch.from_numpy(perm_token).to(case.x.device)]
    assert torch.equal(xp.view(torch.int16), xr.view(torch.int16)) if xp.dtype == torch.bfloat16 else torch.equal(xp, xr)


def _check_same_bits(case, out):
    """The staged forward and (where the shape fits its array) the allocation-free forward
    give the plain forward's bits."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = case.wl
    events = [torch.cuda.Event(enable_timing=True) for _ in range(lm.NUM_STAGES + 1)]
    for e in events:  # torch creates the HIP event on its first record
        e.record()
    st = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], wl.K,
                    stage_events=events)
    torch.cuda.synchronize()
    for k in out:
        assert torch.equal(st[k], out[k]), ("staged", k)
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16 if wl.dtype == "bf16" else lm.F32)
    if lm.lc_moe_workspace_size(shape) > lm.STATIC_WORKSPACE_BYTES:
        return
    na = {k: torch.empty_like(v) for k, v in out.items()}
    wts = lm._weights(case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"])
    lm.lc_moe_forward_noalloc(shape, case.x, wts, na["y"], na["topk_idx"], na["topk_gate"], na["load"])
    torch.cuda.synchronize()
    for k in out:
        assert torch.equal(na[k], out[k]), ("noalloc", k)


def _check_graph(case, out):
    """The forward captured in a graph and replayed on two input sets in turn, with eager
    forwards on the same workspace between replays: every replay gives the eager bits."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = case.wl
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16 if wl.dtype == "bf16" else lm.F32)
    ws = lm.workspace_for(shape, case.x.device)
    wts = lm._weights(case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"])
    x_static, x_other = case.x.clone(), (case.x.float() * -0.5).to(case.x.dtype)
    g_out = {k: torch.empty_like(v) for k, v in out.items()}
    eager_other = lm.forward(x_other, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], wl.K)

    def fwd(x, o):
        lm.lc_moe_forward(shape, x, wts, o["y"], o["topk_idx"], o["topk_gate"], o["load"], ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        fwd(x_static, g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(x_static, g_out)
    torch.cuda.synchronize()
    for rep, (src, want) in enumerate(((case.x, out), (x_other, eager_other), (case.x, out))):
        for v in g_out.values():
            v.zero_()
        x_static.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        for k in g_out:
            assert torch.equal(g_out[k], want[k]), ("graph", rep, k)
        fwd(x_other, {k: torch.empty_like(v) for k, v in out.items()})  # eager work in between
        torch.cuda.synchronize()
