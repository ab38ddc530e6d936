"""The whole layer captured into a HIP graph (torch.cuda.CUDAGraph records HIP graph
nodes on ROCm) and replayed: every replay equals the eager call bitwise, with eager work
and host synchronisation between the replays, and the replayed outputs stay in tolerance
of the oracle.  The layer launches kernels only (no memset, allocation or host sync), so
its graph holds kernel nodes alone."""
import numpy as np
import pytest

from tests.gpu_common import BF16_TOL, F32_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,T,d,I,wfmt", [("bf16", 64, 512, 256, "rows"), ("bf16", 200, 256, 96, "rows"),
                                              ("f32", 48, 128, 64, "rows"), ("bf16", 64, 512, 256, "packed"),
                                              ("bf16", 200, 256, 96, "fp8"), ("bf16", 200, 256, 128, "fp8act"),
                                              ("bf16", 300, 256, 192, "fp8act")])
def test_forward_graph_replay(dtype, T, d, I, wfmt):
    """wfmt: row-major bf16/fp32 weights, packed bf16 weights, block-FP8 weights, or block-FP8
    weights and activations (the FP8 MFMA layer; 64-row and 320-row tile forms)."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = adhoc(name=f"graph_{dtype}_{T}_{wfmt}", T=T, d=d, N=24, Z=12, K=6, I=I, dtype=dtype, seed_key=(300, T),
               expert_std=1.0 / np.sqrt(d))
    say(f"graph replay {wl.name}")
    case = make_case(wl, ri=audited(wl))
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, case.x.dtype)
    ws = lm.workspace_for(shape, case.x.device)
    w = case.w
    if wfmt == "packed":
        extra = lm.pack_weights(w["gate"], w["up"], w["down"])
        wts = lm._weights(case.w_router, case.bias, None, None, None, None, extra)
    elif wfmt in ("fp8", "fp8act"):
        extra = lm.quantize_weights(w["gate"], w["up"], w["down"])
        wts = lm._weights(case.w_router, case.bias, None, None, None, extra, None, wfmt == "fp8act")
    else:
        wts = lm._weights(case.w_router, case.bias, w["gate"], w["up"], w["down"])
    dev = case.x.device

    def outs():
        return dict(y=torch.empty_like(case.x), idx=torch.empty((T, wl.K), dtype=torch.int32, device=dev),
                    gate=torch.empty((T, wl.K), dtype=torch.float32, device=dev),
                    load=torch.empty(wl.E, dtype=torch.int32, device=dev))

    # static input buffer the graph reads; two input sets copied into it in turn
    x_static = case.x.clone()
    x_other = (case.x.float() * -0.5).to(case.x.dtype)
    eager = {}
    for name, src in (("a", case.x), ("b", x_other)):
        o = outs()
        x_static.copy_(src)
        lm.lc_moe_forward(shape, x_static, wts, o["y"], o["idx"], o["gate"], o["load"], ws)
        torch.cuda.synchronize()
        eager[name] = {k: v.clone() for k, v in o.items()}

    g_out = outs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch recommends
        lm.lc_moe_forward(shape, x_static, wts, g_out["y"], g_out["idx"], g_out["gate"], g_out["load"], ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lm.lc_moe_forward(shape, x_static, wts, g_out["y"], g_out["idx"], g_out["gate"], g_out["load"], ws)
    torch.cuda.synchronize()

    for rep, name in enumerate(("a", "b", "a", "b")):
        for v in g_out.values():
            v.zero_()
        x_static.copy_(case.x if name == "a" else x_other)
        g.replay()
        torch.cuda.synchronize()
        for k in g_out:
            assert torch.equal(g_out[k], eager[name][k]), (rep, name, k)
        # eager work between replays on the same workspace
        o = outs()
        lm.lc_moe_forward(shape, x_other if name == "a" else case.x, wts, o["y"], o["idx"], o["gate"], o["load"], ws)
        torch.cuda.synchronize()

    if wfmt == "fp8":  # the oracle of the layer on the dequantized weights
        from tests.test_gpu_fp8 import oracle_fp8_forward
        y_ref = oracle_fp8_forward(case)["y"]
    elif wfmt == "fp8act":  # the oracle of the FP8 MFMA layer
        from tests.test_gpu_fp8_mfma import act_oracle
        y_ref = act_oracle(case)["ref"]["y"]
    else:
        y_ref = oracle_forward(case)["y"]
    err = rel_l2(to_np(eager["a"]["y"]), y_ref)
    say(f"  replays bitwise equal to eager; rel L2 vs oracle {err:.2e}")
    assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL)
