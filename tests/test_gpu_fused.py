"""The forward of layers of one token block (T <= 256) runs top-K and the permutation as one
kernel (the workgroup that finishes its top-K last permutes every token's picks).  Its
picks and gates must equal the separate top-K kernel's (lc_moe_route) bit for bit, its
loads the separate histogram's (lc_moe_expert_load), and the layer the oracle: on a single
token, a single workgroup, the 4096-expert pool (full permutation masks) at T = 255, and a
full last workgroup at T = 256; twice in a row on one workspace (the done-counter is reset
by the router kernel before each call)."""
import numpy as np
import pytest

from gpu_common import BF16_TOL, F32_TOL, adhoc, audited, gate_rtol, make_case, oracle_forward, rel_l2, say, to_np

pytestmark = pytest.mark.gpu

CASES = [("bf16", 1, 64, 4, 2, 2, 64), ("f32", 3, 128, 8, 4, 3, 64), ("bf16", 255, 64, 2048, 2048, 16, 64),
         ("bf16", 256, 256, 40, 8, 4, 160), ("bf16", 97, 6144, 512, 256, 12, 128)]


@pytest.mark.parametrize("dtype,T,d,N,Z,K,I", CASES)
def test_fused_topk_permute(dtype, T, d, N, Z, K, I):
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = adhoc(name=f"fused_{dtype}_{T}_{N + Z}", T=T, d=d, N=N, Z=Z, K=K, I=I, dtype=dtype, seed_key=(600, T),
               expert_std=1.0 / np.sqrt(d), bias=("uniform", 0.5 / (N + Z)))
    say(f"[fused top-K + permutation] {dtype} T={T} d={d} E={N + Z} K={K}")
    case = make_case(wl, ri=audited(wl))
    shape = lm.make_shape(T, d, N, Z, K, I, case.x.dtype)
    ws = lm.workspace_for(shape, case.x.device)
    outs = []
    for _ in range(2):
        out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], K,
                         workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_gate", "load"):
        assert torch.equal(outs[0][k], outs[1][k]), k
    assert torch.equal(outs[0]["y"].view(torch.int16) if dtype == "bf16" else outs[0]["y"],
                       outs[1]["y"].view(torch.int16) if dtype == "bf16" else outs[1]["y"])
    idx, gate = lm.route(case.x, case.w_router, case.bias, K, N)
    assert torch.equal(outs[0]["topk_idx"], idx)
    assert torch.equal(outs[0]["topk_gate"], gate)
    load, _ = lm.expert_load(idx, N, N + Z, d=d, dtype=lm.BF16 if dtype == "bf16" else lm.F32)
    assert torch.equal(outs[0]["load"], load)
    ref = oracle_forward(case)
    assert (to_np(idx) == ref["idx"]).all()
    np.testing.assert_allclose(to_np(gate), ref["gate"], rtol=gate_rtol(d), atol=0)
    err = rel_l2(to_np(outs[0]["y"]), ref["y"])
    say(f"   picks, gates and loads equal the separate kernels'; rel L2 vs oracle {err:.2e}")
    assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL)
