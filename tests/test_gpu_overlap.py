"""Two layers on two streams at once (the single-GPU form of the shortcut-connected MoE
overlap of the LongCat-Flash article, section "Shortcut-connected MoE": a dense FFN runs
beside the MoE layer).  The dense FFN is the layer with one FFN expert, no zero experts
and K = 1 (the router over one expert gives gate 1 exactly).  Running both concurrently
gives bitwise the results of running them one after the other, and the dense FFN matches
the oracle."""
import numpy as np
import pytest

from inputs.generate import routing_inputs
from tests.gpu_common import BF16_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, to_np

pytestmark = pytest.mark.gpu


def test_dense_ffn_beside_layer_on_two_streams():
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = adhoc(name="ovl", T=256, d=256, N=24, Z=12, K=6, I=192, seed_key=(500,), expert_std=1 / np.sqrt(256))
    dense = adhoc(name="ovl_dense", T=256, d=256, N=1, Z=0, K=1, I=512, seed_key=(501,),
                  expert_std=1 / np.sqrt(256))
    say("two streams: MoE layer T=256 d=256 + dense FFN I=512")
    mc = make_case(wl, ri=audited(wl))
    dc = make_case(dense, ri=routing_inputs(dense, beta=0.0))

    def setup(case):
        shape = lm.make_shape(case.wl.T, case.wl.d, case.wl.N, case.wl.Z, case.wl.K, case.wl.I, lm.BF16)
        ws = lm.workspace_for(shape, mc.x.device)
        wts = lm._weights(case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"])
        dev = mc.x.device
        outs = dict(y=torch.empty_like(case.x), idx=torch.empty((case.wl.T, case.wl.K), dtype=torch.int32, device=dev),
                    gate=torch.empty((case.wl.T, case.wl.K), dtype=torch.float32, device=dev),
                    load=torch.empty(case.wl.E, dtype=torch.int32, device=dev))
        return shape, ws, wts, outs

    ms, mws, mwts, mo = setup(mc)
    ds, dws, dwts, do = setup(dc)
    run = lambda case, shape, wts, o, ws, s: lm.lc_moe_forward(  # noqa: E731
        shape, case.x, wts, o["y"], o["idx"], o["gate"], o["load"], ws, stream=s)
    s0, s1 = torch.cuda.current_stream(), torch.cuda.Stream()
    run(mc, ms, mwts, mo, mws, s0)
    run(dc, ds, dwts, do, dws, s0)
    torch.cuda.synchronize()
    serial = {k: v.clone() for k, v in mo.items()}, {k: v.clone() for k, v in do.items()}
    for rep in range(3):
        for o in (mo, do):
            for v in o.values():
                v.zero_()
        torch.cuda.synchronize()
        s1.wait_stream(s0)
        run(mc, ms, mwts, mo, mws, s0)
        run(dc, ds, dwts, do, dws, s1)
        s0.wait_stream(s1)
        torch.cuda.synchronize()
        for got, ref in ((mo, serial[0]), (do, serial[1])):
            for k in got:
                assert torch.equal(got[k], ref[k]), (rep, k)
    assert torch.all(do["idx"] == 0) and torch.all(do["gate"] == 1.0)
    # the dense FFN against the oracle: the layer with one FFN expert and K = 1
    ref = oracle_forward(dc)["y"]
    err = rel_l2(to_np(do["y"]), ref)
    say(f"  concurrent results bitwise equal to serial; dense FFN rel L2 {err:.2e}")
    assert err <= BF16_TOL
