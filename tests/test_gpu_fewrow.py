"""The few-row FFN kernels (64-row M-tiles, two workgroups per CU), which run for layers of
at most 256 tokens, against the oracle on every weight format, with routing skewed so that
experts get more rows than one 64-row M-tile holds (several M-tiles reading one weight
tile), ragged n-tiles (I % 128, d % 256) and single rows.  T = 257 and 65 sit on either
side of the switch to the 320-row form and of one 64-row M-tile; both forms must give the
oracle's results.  Row-major weights with K a multiple of 64 (d for gate/up, I for down)
take the whole-line kernel: d=320, I=192 (ragged n-tiles in both GEMMs) and d=I=64 (one K
chunk: two stages) reach it; d=288, I=160 keep the pipelined kernel's few-row form."""
import numpy as np
import pytest

from tests.gpu_common import BF16_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, to_np

pytestmark = pytest.mark.gpu

HOT = (3, 9)  # FFN experts every token selects (bias far above the rest)


@pytest.mark.parametrize("T", [256, 257, 64, 65, 1])
@pytest.mark.parametrize("wfmt", ["rows", "packed", "fp8"])
@pytest.mark.parametrize("d,I", [(288, 160), (320, 192), (64, 64)])
def test_fewrow_skewed_against_oracle(T, wfmt, d, I):
    import torch
    import mixture_experts_layer_router_amd as lm
    N, Z, K = 20, 6, 4
    wl = adhoc(name=f"fewrow_{T}_{wfmt}_{d}_{I}", T=T, d=d, N=N, Z=Z, K=K, I=I, seed_key=(430, T, d),
               expert_std=1 / np.sqrt(d))

    def modify(ri):
        ri.bias[list(HOT)] = np.float32(1.0)

    say(f"few-row form T={T} weights={wfmt} d={d} I={I} N={N} Z={Z} K={K}")
    case = make_case(wl, ri=audited(wl, modify=modify))
    w, dev = case.w, case.x.device
    shape = lm.make_shape(T, d, N, Z, K, I, lm.BF16)
    if wfmt == "packed":
        packed = lm.pack_weights(w["gate"], w["up"], w["down"])
        wts = lm._weights(case.w_router, case.bias, None, None, None, None, packed)
    elif wfmt == "fp8":
        fp8 = lm.quantize_weights(w["gate"], w["up"], w["down"])
        wts = lm._weights(case.w_router, case.bias, None, None, None, fp8)
    else:
        wts = lm._weights(case.w_router, case.bias, w["gate"], w["up"], w["down"])
    out = dict(y=torch.empty_like(case.x), idx=torch.empty((T, K), dtype=torch.int32, device=dev),
               gate=torch.empty((T, K), dtype=torch.float32, device=dev),
               load=torch.empty(N + Z, dtype=torch.int32, device=dev))
    lm.lc_moe_forward(shape, case.x, wts, out["y"], out["idx"], out["gate"], out["load"],
                      lm.workspace_for(shape, dev))
    if wfmt == "fp8":  # the layer on the dequantized weights
        from tests.test_gpu_fp8 import oracle_fp8_forward
        ref = oracle_fp8_forward(case)
    else:
        ref = oracle_forward(case)
    np.testing.assert_array_equal(to_np(out["idx"]), ref["idx"])
    load = to_np(out["load"])
    assert all(load[e] == T for e in HOT)
    if T >= 65:
        assert int(load[:N].max()) > 64  # an expert spans several 64-row M-tiles
    err = rel_l2(to_np(out["y"]), ref["y"])
    say(f"  rel L2 {err:.2e}; FFN rows per expert {sorted(load[:N].tolist(), reverse=True)[:6]}")
    assert err <= BF16_TOL
