"""lc_moe_forward_noalloc (workspace in a static device array) against lc_moe_forward.

Two calls in a row through the C-ABI, the second on a smaller input, each compared with
lc_moe_forward on the same inputs (bitwise: same kernels) and with the oracle (the
tolerance of every bf16 layer); a full-size decode pair (T=256 then T=64); and a shape
whose workspace exceeds the array, rejected with its outputs untouched.
"""
import numpy as np
import pytest

from gpu_common import BF16_TOL, adhoc, audited, gate_rtol, make_case, oracle_forward, rel_l2, say, to_np
from inputs import configs

pytestmark = pytest.mark.gpu


def outputs(case):
    import torch
    wl, dev = case.wl, case.x.device
    return dict(y=torch.full_like(case.x, 7.0), idx=torch.full((wl.T, wl.K), -3, dtype=torch.int32, device=dev),
                gate=torch.full((wl.T, wl.K), -1.0, dtype=torch.float32, device=dev),
                load=torch.full((wl.E,), -5, dtype=torch.int32, device=dev))


def both(case):
    """(noalloc outputs, lc_moe_forward outputs) on the case's inputs."""
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = case.wl
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16)
    wts = lm._weights(case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"])
    a, b = outputs(case), outputs(case)
    lm.lc_moe_forward_noalloc(shape, case.x, wts, a["y"], a["idx"], a["gate"], a["load"])
    ws = lm.workspace_for(shape, case.x.device)
    lm.lc_moe_forward(shape, case.x, wts, b["y"], b["idx"], b["gate"], b["load"], ws)
    torch.cuda.synchronize()
    return a, b


def assert_same(a, b):
    import torch
    for k in ("y", "idx", "gate", "load"):
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), k


def test_noalloc_two_calls_second_smaller():
    first = adhoc(name="noalloc_a", T=300, d=256, N=16, Z=5, K=4, I=192, seed_key=(500,),
                  expert_std=1 / np.sqrt(256))
    second = adhoc(name="noalloc_b", T=37, d=256, N=16, Z=5, K=4, I=192, seed_key=(501,),
                   expert_std=1 / np.sqrt(256), weight_key=(500,))
    for wl in (first, second):
        say(f"[noalloc] T={wl.T} d={wl.d} N={wl.N} Z={wl.Z} K={wl.K} I={wl.I}")
        case = make_case(wl, ri=audited(wl))
        a, b = both(case)
        assert_same(a, b)
        ref = oracle_forward(case)
        assert (to_np(a["idx"]) == ref["idx"]).all()
        np.testing.assert_allclose(to_np(a["gate"]), ref["gate"], rtol=gate_rtol(wl.d), atol=0)
        err = rel_l2(to_np(a["y"]), ref["y"])
        say(f"   bitwise equal to lc_moe_forward; rel L2 vs oracle {err:.2e}")
        assert err <= BF16_TOL


def test_noalloc_decode_full_size_then_smaller():
    big, small = configs.get("decode_T256_z33"), configs.get("decode_T64_z33")
    assert big.weight_seed_key == small.weight_seed_key
    cb = make_case(big)
    cs = make_case(small, weights=False)
    cs.w = cb.w
    for case in (cb, cs):
        say(f"[noalloc] {case.wl.description}")
        a, b = both(case)
        assert_same(a, b)


def test_noalloc_rejects_shape_beyond_the_array():
    import torch
    import mixture_experts_layer_router_amd as lm
    wl = configs.get("prefill")
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16)
    assert lm.lc_moe_workspace_size(shape) > lm.STATIC_WORKSPACE_BYTES
    dev = torch.device("cuda:0")
    x = torch.zeros((8, wl.d), dtype=torch.bfloat16, device=dev)   # never read
    y = torch.full((8, wl.d), 3.0, dtype=torch.bfloat16, device=dev)
    wts = lm._weights(x, x, x, x, x)
    with pytest.raises(lm.LcMoeError) as ei:
        lm.lc_moe_forward_noalloc(shape, x, wts, y, None, None, None)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
