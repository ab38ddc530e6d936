"""Block-FP8 expert weights on the GPU: the quantizer's codes and scales equal the oracle's
(oracle/fp8.py) bit for bit, and the layer run on them equals the fp64 oracle layer on the
dequantized weights within the bf16 tolerance."""
import numpy as np
import pytest

from inputs import configs
from oracle import fp8 as ofp8
from oracle import moe as orc
from inputs.generate import weights_f64
from tests.gpu_common import BF16_TOL, adhoc, audited, make_case, rel_l2, say, to_np, worst_token_rel

pytestmark = pytest.mark.gpu


def plan(N, d, I):
    """Byte offsets of the packed regions, as documented with lc_moe_quantize_weights."""
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    nt_gu, nt_d, nrb_i, nrb_d = -(-I // 128), -(-d // 256), -(-I // 128), -(-d // 128)
    o, out = 0, {}
    for name, size in (("codes_gu", N * nt_gu * (d // 32) * 8192), ("codes_d", N * nt_d * (I // 32) * 8192),
                       ("scales_gu", N * 2 * nrb_i * nrb_d * 4), ("scales_d", N * nrb_d * nrb_i * 4)):
        out[name] = o
        o = al(o + size)
    out.update(total=o, nt_gu=nt_gu, nt_d=nt_d, nrb_i=nrb_i, nrb_d=nrb_d)
    return out


def swz4(p):
    return (((p >> 1) & 1) << 1) ^ ((p >> 2) & 1) ^ (((p >> 3) & 1) << 1)


def code_offsets(p, N, d, I, mat, e, r, k):
    """Byte offsets of the codes of rows r, columns k (broadcast) of matrix mat (0 gate,
    1 up, 2 down) of expert e: n-tile, pair-row, half and swizzled 16-byte chunk."""
    C = d if mat < 2 else I
    if mat < 2:
        nt, rt, base, ntc = r // 128, r % 128, p["codes_gu"], p["nt_gu"]
        pr, half = rt, mat
    else:
        nt, rt, base, ntc = r // 256, r % 256, p["codes_d"], p["nt_d"]
        pr, half = (rt >> 6) * 32 + (rt & 31), (rt >> 5) & 1
    g = (k % 32) // 8
    return base + ((e * ntc + nt) * (C // 32) + k // 32) * 8192 + pr * 64 + ((g ^ swz4(pr)) * 16) + half * 8 + k % 8


def unpack(buf, p, N, d, I, mat, e):
    """Codes [R][C] and scale exponents of matrix mat (0 gate, 1 up, 2 down) of expert e."""
    R, C = (I, d) if mat < 2 else (d, I)
    codes = buf[code_offsets(p, N, d, I, mat, e, np.arange(R)[:, None], np.arange(C)[None, :])]
    nrb, ncb = -(-R // 128), -(-C // 128)
    if mat < 2:
        s0 = p["scales_gu"] + ((e * 2 + mat) * nrb) * ncb * 4
    else:
        s0 = p["scales_d"] + (e * nrb) * ncb * 4
    sc = buf[s0:s0 + nrb * ncb * 4].view(np.float32).reshape(nrb, ncb).astype(np.float64)
    ks = np.log2(sc)
    assert np.all(ks == np.round(ks)), "scales must be powers of two"
    return codes, ks.astype(np.int64)


def quantize_on_gpu(w):
    import mixture_experts_layer_router_amd as lm
    return lm.quantize_weights(w["gate"], w["up"], w["down"])


def test_quantizer_bit_exact():
    import torch
    wl = adhoc(name="fp8q", T=8, d=288, N=5, Z=2, K=2, I=224, seed_key=(400,), expert_std=1 / np.sqrt(288))
    say("fp8 quantizer: d=288 I=224 N=5 (ragged tiles and blocks)")
    case = make_case(wl)
    w = case.w
    with torch.no_grad():
        w["gate"][1, :128, 128:256] *= 1000          # a block on another scale
        w["up"][2, 128:, :128] = 0                   # an all-zero (partial) block
        g = w["gate"][0]
        g[0, 0] = 448.0                              # block amax 448 -> k = 0, then ties:
        for c, v in enumerate((1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, 15 * 2.0 ** -10), 1):
            g[0, c] = v
    torch.cuda.synchronize()
    buf = quantize_on_gpu(w).cpu().numpy()
    p = plan(wl.N, wl.d, wl.I)
    assert buf.size >= p["total"]
    for mat, name in enumerate(("gate", "up", "down")):
        for e in range(wl.N):
            ref_codes, ref_ks = ofp8.quantize(weights_f64(w[name][e]))
            codes, ks = unpack(buf, p, wl.N, wl.d, wl.I, mat, e)
            np.testing.assert_array_equal(ks, ref_ks, err_msg=f"{name}[{e}] scales")
            np.testing.assert_array_equal(codes, ref_codes, err_msg=f"{name}[{e}] codes")
    got = unpack(buf, p, wl.N, wl.d, wl.I, 0, 0)[0][0, :7]
    assert list(got) == [0x7E, 0x38, 0x3A, 0x02, 0x00, 0xB8, 0x08]
    # tile rows past I (gate/up) and past d (down) are zero
    for mat, R, rpt in ((0, wl.I, 128), (1, wl.I, 128), (2, wl.d, 256)):
        C = wl.d if mat < 2 else wl.I
        pad = np.arange(R, -(-R // rpt) * rpt)[:, None]
        assert pad.size > 0
        for e in range(wl.N):
            assert not buf[code_offsets(p, wl.N, wl.d, wl.I, mat, e, pad, np.arange(C)[None, :])].any()


def oracle_fp8_forward(case, tokens=None):
    cache = {}

    def experts(e):
        if e not in cache:
            cache.clear()
            cache[e] = tuple(ofp8.dequantize(*ofp8.quantize(weights_f64(case.w[k][e])))
                             for k in ("gate", "up", "down"))
        return cache[e]

    return orc.moe_forward(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, experts,
                           case.wl.N, case.wl.K, tokens=tokens)


@pytest.mark.parametrize("T,d,I,N,Z,K", [(300, 256, 160, 12, 5, 4), (96, 512, 384, 40, 20, 6), (1, 64, 32, 3, 1, 2)])
def test_forward_fp8_matches_oracle(T, d, I, N, Z, K):
    import mixture_experts_layer_router_amd as lm
    wl = adhoc(name=f"fp8f{T}", T=T, d=d, N=N, Z=Z, K=K, I=I, seed_key=(401, T), expert_std=1 / np.sqrt(d))
    say(f"fp8 forward T={T} d={d} I={I} N={N} Z={Z} K={K}")
    case = make_case(wl, ri=audited(wl))
    q = quantize_on_gpu(case.w)
    # low-level call with the bf16 weight pointers NULL: the FFN reads only the FP8 form
    import torch
    shape = lm.make_shape(T, d, N, Z, K, I, lm.BF16)
    ws = lm.workspace_for(shape, case.x.device)
    out = dict(y=torch.empty_like(case.x), topk_idx=torch.empty((T, K), dtype=torch.int32, device=case.x.device),
               gate=torch.empty((T, K), dtype=torch.float32, device=case.x.device),
               load=torch.empty(N + Z, dtype=torch.int32, device=case.x.device))
    lm.lc_moe_forward(shape, case.x, lm._weights(case.w_router, case.bias, None, None, None, q), out["y"],
                      out["topk_idx"], out["gate"], out["load"], ws)
    ref = oracle_fp8_forward(case)
    np.testing.assert_array_equal(out["topk_idx"].cpu().numpy(), ref["idx"])
    y = to_np(out["y"])
    err, worst = rel_l2(y, ref["y"]), worst_token_rel(y, ref["y"])
    # the bf16 layer on the original weights is farther from this reference
    y16 = to_np(lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], K)["y"])
    say(f"  rel L2 {err:.2e} (worst token {worst:.2e}); bf16-weight layer vs it {rel_l2(y16, ref['y']):.2e}")
    assert err <= BF16_TOL


def quantized_experts(w, need, workers=8):
    """The oracle's dequantized weights of the experts in `need` (quantized in threads)."""
    import concurrent.futures

    def one(e):
        return tuple(ofp8.dequantize(*ofp8.quantize(weights_f64(w[k][e]))) for k in ("gate", "up", "down"))

    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(zip(need, ex.map(one, need)))


@pytest.mark.parametrize("name", ["decode_T64_z66", "decode_T256_z33"])
def test_forward_fp8_decode_full_size(name):
    """The decode layer at full size (768-expert pool, d=6144, I=2048) on FP8 weights,
    every token checked against the oracle on its own dequantized weights."""
    import mixture_experts_layer_router_amd as lm
    wl = configs.get(name)
    say(f"fp8 forward full size: {wl.description}")
    case = make_case(wl)
    q = quantize_on_gpu(case.w)
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], wl.K, fp8=q)
    idx = out["topk_idx"].cpu().numpy()
    need = sorted(set(idx[idx < wl.N].tolist()))
    deq = quantized_experts(case.w, need)
    ref = orc.moe_forward(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, lambda e: deq[e],
                          wl.N, wl.K)
    np.testing.assert_array_equal(idx, ref["idx"])
    y = to_np(out["y"])
    err, worst = rel_l2(y, ref["y"]), worst_token_rel(y, ref["y"])
    say(f"  rel L2 {err:.2e} (worst token {worst:.2e}) over {wl.T} tokens, {len(need)} experts")
    assert err <= BF16_TOL and worst <= BF16_TOL


def test_forward_fp8_prefill_full_size_sampled():
    """The prefill layer at full size on FP8 weights, in the benchmark's launch
    configuration.  The oracle checks the token with the most FFN picks and the token with
    the most FFN picks among those routed to the most loaded expert (each oracle expert costs
    a fraction of a second of CPU quantization; the skewed layer's FP8 check in
    test_gpu_full.py covers a whole M-tile)."""
    import mixture_experts_layer_router_amd as lm
    wl = configs.get("prefill")
    say(f"fp8 forward full size: {wl.description}")
    case = make_case(wl)
    q = quantize_on_gpu(case.w)
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], wl.K, fp8=q)
    idx = out["topk_idx"].cpu().numpy()
    load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
    top = int(np.argmax(load))
    ffn = (idx < wl.N).sum(1)
    on_top = np.nonzero((idx == top).any(1))[0]
    tokens = sorted({int(np.argmax(ffn)), int(on_top[np.argmax(ffn[on_top])])})
    say(f"  sampled tokens {tokens} with {ffn[tokens].tolist()} FFN experts; expert {top} has {load[top]} rows")
    sub = idx[tokens]
    deq = quantized_experts(case.w, sorted(set(sub[sub < wl.N].tolist())))
    ref = orc.moe_forward(case.ri.x_f64(), case.ri.w_router.astype(np.float64), case.ri.bias, lambda e: deq[e],
                          wl.N, wl.K, tokens=tokens)
    np.testing.assert_array_equal(idx[tokens], ref["idx"])
    y = to_np(out["y"])[tokens]
    err = rel_l2(y, ref["y"])
    say(f"  rel L2 {err:.2e}")
    assert err <= BF16_TOL
