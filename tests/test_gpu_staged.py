"""lc_moe_forward_staged (the forward with a HIP event recorded at each stage boundary, which
bench.py times) computes the same bits as lc_moe_forward, and its stage spans are
non-negative and add up to the first-to-last span."""
import numpy as np
import pytest

from tests.gpu_common import adhoc, audited, make_case, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,d,I", [(64, 512, 256), (700, 256, 160)])
def test_forward_staged_equals_forward(T, d, I):
    """T=64: the few-row kernels and the one-block permutation; T=700: the 320-row form."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = adhoc(name=f"staged_{T}", T=T, d=d, N=24, Z=12, K=6, I=I, seed_key=(440, T), expert_std=1 / np.sqrt(d))
    say(f"staged forward T={T} d={d} I={I}")
    case = make_case(wl, ri=audited(wl))
    dev = case.x.device
    shape = lm.make_shape(T, d, wl.N, wl.Z, wl.K, I, lm.BF16)
    ws = lm.workspace_for(shape, dev)
    wts = lm._weights(case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"])

    def outs():
        return dict(y=torch.empty_like(case.x), idx=torch.empty((T, wl.K), dtype=torch.int32, device=dev),
                    gate=torch.empty((T, wl.K), dtype=torch.float32, device=dev),
                    load=torch.empty(wl.E, dtype=torch.int32, device=dev))

    a, b = outs(), outs()
    lm.lc_moe_forward(shape, case.x, wts, a["y"], a["idx"], a["gate"], a["load"], ws)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(lm.NUM_STAGES + 1)]
    for e in events:  # torch creates the HIP event on its first record
        e.record()
    torch.cuda.synchronize()
    lm.lc_moe_forward_staged(shape, case.x, wts, b["y"], b["idx"], b["gate"], b["load"], ws, stage_events=events)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    spans = [events[i].elapsed_time(events[i + 1]) for i in range(lm.NUM_STAGES)]
    total = events[0].elapsed_time(events[-1])
    say("  stages " + ", ".join(f"{lm.stage_name(i)} {v * 1e3:.1f} us" for i, v in enumerate(spans)))
    assert all(v >= 0 for v in spans)
    assert abs(sum(spans) - total) <= 1e-3 * max(total, 1e-3) + 1e-3
