"""The FP8 MFMA layer on the GPU (block-FP8 weights and activations on the FP8 matrix cores).

  * the activation quantizer (lc_moe_quantize_activations) equals the oracle's
    quantize_rows bit for bit: codes and E8M0 scale bytes, with planted ties, an all-zero
    block, blocks on far-apart scales and a partial last block;
  * the layer (lc_moe_weights.fp8_act) equals the fp64 oracle layer whose experts run
    oracle.fp8.fp8_act_expert on the dequantized weights, on small layers that cover both
    tile forms (320 and 64 rows), ragged M-tiles, a partial last n-tile, more than 64
    scale blocks per row in either projection, and one token;
  * at full size: sampled prefill tokens, and the whole first 320-row tile of the skewed
    layer's most loaded expert.
The weights-only FP8 layer is at least 2 times farther from the reference than the FP8
MFMA layer (12 times on most shapes, 2.5 with I = 64: the activations are seen to be
quantized).

Tolerance.  The kernel's arithmetic differs from the oracle's in three places: G and U are
sums formed by the FP8 matrix cores (the products of FP8 codes and power-of-two scales are
exact, the sums are not fp32-exact, see below), Y rows and the output are rounded to bf16,
and H = silu(G) U is formed in fp32 before it is quantized.  Rounding Y and y moves a
token's output by at most 2^-9 (||y_t|| + sum_k g_k ||Y_k||), taken with a factor 2 of
margin.  Where H lies next to an E4M3 rounding boundary, the kernel's H and the oracle's
fp64 H may take neighbouring codes, a step of 6-12% of that element.  The scaled FP8 MFMA
adds its 64 products and the accumulator with about 12 bits below the largest addend: run
as the K loop runs it (1 to 96 steps into one accumulator, operands spread like
block-quantized data), its error stayed below 2^-13 (|G| + rss(G's products)) over 262144
sums per length, far above one fp32 rounding per step.  So each H element's uncertainty is
  eG = 2^-11 (|G| + rss(G terms)), eU alike (4 times the largest error seen),
  eH = |U silu'(G)| eG + |silu(G)| eU + 8 u |H|,   u = 2^-24,
and oracle.fp8.rows_requant_bound turns it into the largest move of each quantized H
element; a token may differ by sum_k g_k sum_i delta_ki ||W_down[:, i]|| more.  Elements
away from a boundary have delta = 0, so a wrong code there still fails.  That per-token
bound is sound but loose (it lets every element near a boundary move); the layer's error
pooled over all checked tokens must also stay within 2^-7, where the real code changes,
rare and independent, leave it near the bf16 rounding level (about 2e-3)."""
import collections
import concurrent.futures

import numpy as np
import pytest

from inputs import configs
from inputs.generate import weights_f64
from oracle import fp8 as ofp8
from oracle import moe as orc
from tests.gpu_common import U32, adhoc, audited, make_case, rel_l2, say, to_np, worst_token_rel

pytestmark = pytest.mark.gpu

# Accumulation error of the FP8 matrix cores, relative to |G| + rss(G's products): 4 times
# the largest seen when chaining 1 to 96 scaled FP8 MFMAs (64 K each) into one accumulator.
MFMA_ACC = 2.0 ** -11
# Relative L2 error of the layer pooled over the checked tokens (bf16 rounding is about 2e-3).
POOLED_TOL = 2.0 ** -7


def _lm():
    import mixture_experts_layer_router_amd as lm
    return lm


def test_quantize_activations_bit_exact():
    import torch
    lm = _lm()
    g = np.random.default_rng(500)
    rows, cols = 37, 320                                  # 3 blocks per row, the last of 64 columns
    a = g.standard_normal((rows, cols)) * np.exp2(g.integers(-20, 20, (rows, 1)))
    a[3, 128:256] = 0.0                                   # an all-zero block
    a[4, :128] *= 2.0 ** 60                               # far-apart scales in one row
    a[4, 128:256] *= 2.0 ** -60
    a[5, 7:128] = g.uniform(-1, 1, 121)                  # block max 448 (k = 0), then ties:
    a[5, :7] = [448.0, 1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, 15 * 2.0 ** -10]
    a[6, 256:] = -a[6, 256:]
    x = torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)
    codes, scales = lm.quantize_activations(x.cuda())
    ref_codes, ref_k = ofp8.quantize_rows(weights_f64(x))
    np.testing.assert_array_equal(scales.cpu().numpy().astype(np.int64), ref_k + 127)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)
    assert list(codes[5, :7].cpu().numpy()) == [0x7E, 0x38, 0x3A, 0x02, 0x00, 0xB8, 0x08]
    assert int(scales[3, 1]) == 127 and not codes[3, 128:256].cpu().numpy().any()


def audited_expert(rows):
    """expert_fn for the oracle layer: oracle.fp8.fp8_act_expert, and per FFN row (appended
    to `rows` in the oracle's call order = permuted row order) ||Y_row|| and the H-rounding
    allowance sum_i delta_i ||W_down[:, i]||."""
    from scipy.special import expit

    def fn(X, wg, wu, wd):
        Y = ofp8.fp8_act_expert(X, wg, wu, wd)
        Xq, G, U, H = ofp8.fp8_act_hidden(X, wg, wu)
        eG = MFMA_ACC * (np.abs(G) + np.sqrt((Xq ** 2) @ (wg ** 2).T))
        eU = MFMA_ACC * (np.abs(U) + np.sqrt((Xq ** 2) @ (wu ** 2).T))
        s = expit(G)
        eH = np.abs(U * s * (1 + G * (1 - s))) * eG + np.abs(G * s) * eU + 8 * U32 * np.abs(H)
        delta = ofp8.rows_requant_bound(H, eH)
        rows.append((np.linalg.norm(Y, axis=1), delta @ np.linalg.norm(wd, axis=0), int((delta > 0).sum())))
        return Y
    return fn


def act_oracle(case, tokens=None, deq=None):
    """The oracle layer of the FP8 MFMA path (experts quantized on demand unless given),
    with per-token bounds: dict(ref, base, allow, flagged)."""
    def experts(e):
        if deq is not None:
            return deq(e)
        return tuple(ofp8.dequantize(*ofp8.quantize(weights_f64(case.w[k][e]))) for k in ("gate", "up", "down"))

    batch = dict(x=case.ri.x_f64(), w_router=case.ri.w_router.astype(np.float64), bias=case.ri.bias,
                 K=case.wl.K, tokens=tokens)
    rows = []
    ref = orc.moe_forward_batches([batch], experts, case.wl.N, expert_fn=audited_expert(rows))[0]
    P = ref["perm_token"].size
    ynorm = np.concatenate([r[0] for r in rows]) if rows else np.zeros(0)
    allow_row = np.concatenate([r[1] for r in rows]) if rows else np.zeros(0)
    assert ynorm.size == P
    idx, gate, slot = ref["idx"], ref["gate"], ref["slot_row"]
    ffn = idx < case.wl.N
    g = np.where(ffn, gate, 0.0)
    sl = np.where(ffn, slot, 0)
    pick = lambda v: (g * (v[sl] if P else 0.0)).sum(axis=1)  # noqa: E731
    base = 2.0 ** -8 * (np.linalg.norm(ref["y"], axis=1) + pick(ynorm))
    return dict(ref=ref, base=base, allow=pick(allow_row), flagged=sum(r[2] for r in rows))


def check_layer(got_y, got_idx, o, label):
    ref = o["ref"]
    np.testing.assert_array_equal(got_idx, ref["idx"])
    dev = np.linalg.norm(got_y - ref["y"], axis=1)
    err, worst = rel_l2(got_y, ref["y"]), worst_token_rel(got_y, ref["y"])
    over_base = int((dev > o["base"]).sum())
    say(f"  {label}: rel L2 {err:.2e} (worst token {worst:.2e}); {over_base} of {dev.size} tokens past the "
        f"rounding bound, {o['flagged']} H elements near a boundary")
    bad = np.nonzero(dev > o["base"] + o["allow"])[0]
    assert bad.size == 0, (f"{label}: tokens {bad[:5]} off by {dev[bad[:5]]} > "
                           f"{o['base'][bad[:5]]} + {o['allow'][bad[:5]]}")
    assert err <= POOLED_TOL, (label, err)
    return err


def run(case, q, fp8_act=True):
    lm = _lm()
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], case.wl.K,
                     fp8=q, fp8_act=fp8_act)
    return {k: to_np(v) for k, v in out.items()}


SHAPES = [
    # T, d, I, N, Z, K: 320-row tiles (several per expert, ragged) and a partial last n-tile
    (1200, 256, 192, 4, 2, 4),
    # 64-row tiles (few tokens)
    (96, 512, 384, 40, 20, 6),
    # 65 scale blocks per row of x (gate/up), then of H (down)
    (300, 8256, 64, 3, 1, 2),
    (300, 64, 8256, 3, 1, 2),
    (40, 8256, 128, 4, 2, 2),
    (1, 64, 64, 3, 1, 2),
]


@pytest.mark.parametrize("T,d,I,N,Z,K", SHAPES)
def test_forward_fp8_act_matches_oracle(T, d, I, N, Z, K):
    lm = _lm()
    wl = adhoc(name=f"fp8a{T}_{d}_{I}", T=T, d=d, N=N, Z=Z, K=K, I=I, seed_key=(501, T, d, I),
               expert_std=1 / np.sqrt(d))
    say(f"fp8 MFMA forward T={T} d={d} I={I} N={N} Z={Z} K={K}")
    case = make_case(wl, ri=audited(wl))
    q = lm.quantize_weights(case.w["gate"], case.w["up"], case.w["down"])
    got = run(case, q)
    o = act_oracle(case)
    err = check_layer(got["y"], got["topk_idx"], o, "layer")
    # the weights-only FP8 layer (x and H in bf16) is much farther from this reference
    w8 = run(case, q, fp8_act=False)
    err8 = rel_l2(w8["y"], o["ref"]["y"])
    say(f"  weights-only FP8 layer vs it: rel L2 {err8:.2e} ({err8 / err:.1f} times the FP8 MFMA layer's)")
    assert err8 >= 2 * err
    # deterministic
    again = run(case, q)
    assert np.array_equal(again["y"], got["y"])


class Prefetch:
    """experts(e) for the oracle, quantized in threads a few experts ahead of use, in the
    ascending order the oracle asks for them (memory for a window of experts only)."""

    def __init__(self, w, need, window=8):
        self.w, self.order, self.window = w, list(need), window
        self.ex = concurrent.futures.ThreadPoolExecutor(max_workers=window)
        self.q = collections.deque()
        self.next = 0
        self._fill()

    def _one(self, e):
        return tuple(ofp8.dequantize(*ofp8.quantize(weights_f64(self.w[k][e]))) for k in ("gate", "up", "down"))

    def _fill(self):
        while len(self.q) < self.window and self.next < len(self.order):
            e = self.order[self.next]
            self.q.append((e, self.ex.submit(self._one, e)))
            self.next += 1

    def __call__(self, e):
        e0, fut = self.q.popleft()
        assert e0 == e, (e0, e)
        self._fill()
        return fut.result()


def check_tokens(case, got, tokens, label):
    idx = got["topk_idx"][tokens]
    need = sorted(set(idx[idx < case.wl.N].tolist()))
    say(f"  {label}: oracle on {len(tokens)} tokens, {len(need)} experts")
    o = act_oracle(case, tokens=tokens, deq=Prefetch(case.w, need))
    check_layer(got["y"][tokens], idx, o, label)


def test_fp8_act_prefill_full_size_sampled():
    """The prefill layer at full size in the benchmark's launch configuration: the token with
    the most FFN picks and the one with the most among those routed to the most loaded
    expert."""
    lm = _lm()
    wl = configs.get("prefill")
    say(f"fp8 MFMA forward full size: {wl.description}")
    case = make_case(wl)
    q = lm.quantize_weights(case.w["gate"], case.w["up"], case.w["down"])
    got = run(case, q)
    del q
    idx = got["topk_idx"]
    load = np.bincount(idx.ravel(), minlength=wl.E)[:wl.N]
    top = int(np.argmax(load))
    ffn = (idx < wl.N).sum(1)
    on_top = np.nonzero((idx == top).any(1))[0]
    tokens = sorted({int(np.argmax(ffn)), int(on_top[np.argmax(ffn[on_top])])})
    check_tokens(case, got, tokens, "prefill")


def test_fp8_act_skewed_head_expert_first_tile():
    """The skewed layer at full size: every token of the first 320-row tile of its most
    loaded expert (a whole tile of the 320-row form)."""
    lm = _lm()
    wl = configs.get("skewed")
    say(f"fp8 MFMA forward full size: {wl.description}")
    case = make_case(wl)
    q = lm.quantize_weights(case.w["gate"], case.w["up"], case.w["down"])
    got = run(case, q)
    del q
    idx = got["topk_idx"]
    offsets, perm_token, _ = orc.permute(idx, wl.N)
    head = int(np.argmax(np.diff(offsets)))
    assert offsets[head + 1] - offsets[head] > 320
    tokens = perm_token[offsets[head]:offsets[head] + 320]
    check_tokens(case, got, tokens, f"skewed head expert {head}")
