"""Full-size parity on every token, in the benchmark's launch configuration.

The prefill layer (T=16384) and its nine decode batches (T in 64/128/256, zero share
0/33/66%) run on one set of expert weights, as one layer would serve them; the skewed
layer (T=32768, Zipf-loaded experts) has its own.  For every token of every layer:
  * top-K indices and expert loads bit-exact, gates within gate_rtol(d);
  * y within 2e-2 relative L2 per token (and pooled);
  * the FFN part alone: y - gz * x (gz = the token's zero-pick gate sum, from the GPU's own
    gates) against the oracle's FFN part, per token, within 2e-2 of that part's norm plus
    2^-8 of |y| (the one bf16 rounding of y, which cannot be attributed to the FFN).  An
    expert's output row reaches y scaled by its gate beside the identity term, so a wrong
    output tile shows up here first.
The oracle streams each expert's weights once for all the layers that share them
(oracle.moe.moe_forward_batches).

Block-FP8 weights at full size: every token of the skewed layer's head expert's first
M-tile (320 rows, the tile that spans the expert's first rows), against the fp64 oracle
on the oracle's own dequantized weights, within 2e-3 relative L2; the bf16-weight layer is
checked to lie outside that bound on the same tokens, so the test tells the two apart.
"""
import concurrent.futures

import numpy as np
import pytest

from gpu_common import BF16_TOL, gate_rtol, make_case, say, to_np
from inputs import configs
from inputs.generate import weights_f64
from oracle import fp8 as ofp8
from oracle import moe as orc

pytestmark = pytest.mark.gpu

DECODE = [f"decode_T{T}_z{z}" for T in configs.DECODE_T for z in configs.DECODE_SHARES]
FP8_TOL = 2e-3
Y_ROUND = 2.0 ** -8


def _lm():
    import mixture_experts_layer_router_amd as lm
    return lm


def run_layer(lm, case, fp8=None):
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"],
                     case.wl.K, fp8=fp8)
    return {k: to_np(v) for k, v in out.items()}


def oracle_batch(case, tokens=None):
    return dict(x=case.ri.x_f64(), w_router=case.ri.w_router.astype(np.float64), bias=case.ri.bias,
                K=case.wl.K, tokens=tokens)


def bf16_experts(w):
    def experts(e):
        return weights_f64(w["gate"][e]), weights_f64(w["up"][e]), weights_f64(w["down"][e])
    return experts


def check_all_tokens(name, case, got, ref):
    wl = case.wl
    x = case.ri.x_f64()
    idx, gate, y = got["topk_idx"], got["topk_gate"], got["y"]
    mism = np.nonzero((idx != ref["idx"]).any(axis=1))[0]
    assert mism.size == 0, f"{name}: {mism.size} tokens routed differently, first {mism[:5]}"
    np.testing.assert_allclose(gate, ref["gate"], rtol=gate_rtol(wl.d), atol=0)
    assert (got["load"] == ref["load"]).all()
    ny = np.linalg.norm(ref["y"], axis=1)
    tok_err = np.linalg.norm(y - ref["y"], axis=1) / np.maximum(ny, 1e-300)
    pooled = float(np.linalg.norm(y - ref["y"]) / np.linalg.norm(ref["y"]))
    gz = np.where(idx >= wl.N, gate.astype(np.float64), 0.0).sum(axis=1)
    ffn_err = np.linalg.norm((y - gz[:, None] * x) - ref["y_ffn"], axis=1)
    nf = np.linalg.norm(ref["y_ffn"], axis=1)
    allow = BF16_TOL * nf + Y_ROUND * ny
    worst_ffn = float(np.max(ffn_err / np.maximum(nf, 1e-300), where=nf > 0, initial=0.0))
    say(f"   {name}: pooled {pooled:.2e}, worst token {tok_err.max():.2e}, worst FFN part "
        f"{worst_ffn:.2e} ({int((nf > 0).sum())} tokens with FFN picks, T={wl.T})")
    assert pooled <= BF16_TOL
    bad = np.nonzero(tok_err > BF16_TOL)[0]
    assert bad.size == 0, f"{name}: tokens {bad[:5]} above {BF16_TOL} ({tok_err[bad[:5]]})"
    bad = np.nonzero(ffn_err > allow)[0]
    assert bad.size == 0, f"{name}: FFN part of tokens {bad[:5]} off ({ffn_err[bad[:5]]} > {allow[bad[:5]]})"


@pytest.fixture(scope="module")
def prefill_family():
    """The prefill layer and its nine decode batches on the prefill layer's expert weights:
    GPU outputs and the oracle's, for every token."""
    lm = _lm()
    pre = configs.get("prefill")
    say("[full] prefill family: weights, 10 layers on the GPU")
    base = make_case(pre)
    cases = {"prefill": base}
    for name in DECODE:
        wl = configs.get(name)
        assert wl.weight_seed_key == pre.weight_seed_key and (wl.d, wl.N, wl.I) == (pre.d, pre.N, pre.I)
        c = make_case(wl, weights=False)
        c.w = base.w
        cases[name] = c
    got = {name: run_layer(lm, c) for name, c in cases.items()}
    say("[full] prefill family: oracle (one pass over the 512 experts)")
    refs = orc.moe_forward_batches([oracle_batch(c) for c in cases.values()], bf16_experts(base.w), pre.N)
    yield cases, got, dict(zip(cases, refs))
    del cases, got


@pytest.mark.parametrize("name", ["prefill"] + DECODE)
def test_every_token_prefill_and_decode(prefill_family, name):
    cases, got, refs = prefill_family
    check_all_tokens(name, cases[name], got[name], refs[name])


@pytest.fixture(scope="module")
def skewed_layer():
    lm = _lm()
    wl = configs.get("skewed")
    say("[full] skewed layer on the GPU")
    case = make_case(wl)
    got = run_layer(lm, case)
    say("[full] skewed layer: oracle")
    ref = orc.moe_forward_batches([oracle_batch(case)], bf16_experts(case.w), wl.N)[0]
    yield case, got, ref


def test_every_token_skewed(skewed_layer):
    case, got, ref = skewed_layer
    check_all_tokens("skewed", case, got, ref)
    ffn = ref["ffn_count"]
    assert ffn.min() == 0 and ffn.max() == case.wl.K      # easy and hard tokens present


def test_fp8_skewed_head_expert_first_tile(skewed_layer):
    lm = _lm()
    case, got16, ref16 = skewed_layer
    wl = case.wl
    load = np.diff(ref16["offsets"])
    head = int(np.argmax(load))
    tokens = ref16["perm_token"][ref16["offsets"][head]:ref16["offsets"][head] + 320]
    assert load[head] > 320 and tokens.size == 320
    q = lm.quantize_weights(case.w["gate"], case.w["up"], case.w["down"])
    got8 = run_layer(lm, case, fp8=q)
    del q
    assert (got8["topk_idx"] == got16["topk_idx"]).all()   # routing does not see the weights
    say(f"[fp8] skewed head expert {head} ({load[head]} rows): oracle on its first 320 tokens")

    def quantized(e):
        return tuple(ofp8.dequantize(*ofp8.quantize(weights_f64(case.w[k][e]))) for k in ("gate", "up", "down"))

    need = sorted(set(ref16["idx"][tokens][ref16["idx"][tokens] < wl.N].tolist()))
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        deq = dict(zip(need, ex.map(quantized, need)))
    ref8 = orc.moe_forward_batches([oracle_batch(case, tokens=tokens)], lambda e: deq[e], wl.N)[0]
    assert (got8["topk_idx"][tokens] == ref8["idx"]).all()
    y8, y16 = got8["y"][tokens], got16["y"][tokens]
    err8 = float(np.linalg.norm(y8 - ref8["y"]) / np.linalg.norm(ref8["y"]))
    err16 = float(np.linalg.norm(y16 - ref8["y"]) / np.linalg.norm(ref8["y"]))
    tok8 = np.linalg.norm(y8 - ref8["y"], axis=1) / np.linalg.norm(ref8["y"], axis=1)
    say(f"   FP8 layer vs oracle on dequantized weights: {err8:.2e} (worst token {tok8.max():.2e}); "
        f"bf16-weight layer vs the same: {err16:.2e}; {len(need)} experts")
    assert err8 <= FP8_TOL
    assert err16 > FP8_TOL
