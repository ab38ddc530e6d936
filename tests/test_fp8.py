"""Block-FP8 weight oracle (oracle/fp8.py) against the E4M3 definition: printed-format
special values, brute-force nearest-value search, tie cases, the block-scale rule and the
error bound of round-to-nearest."""
import math

import numpy as np
import pytest

from oracle import fp8


def test_e4m3_special_values():
    v = fp8.E4M3_TABLE
    assert v[0x00] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    assert v[0x01] == 2.0 ** -9                    # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                # largest subnormal
    assert v[0x08] == 2.0 ** -6                    # smallest normal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0  # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                # codes ascend with value


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.E4M3_TABLE[codes]), codes)


def test_encode_ties_to_even():
    # midpoints: 1.0|1.125 -> 1.0 (0x38); 1.125|1.25 -> 1.25 (0x3A); 2^-10 (0|2^-9) -> 0;
    # 3*2^-10 (2^-9|2^-8) -> 2^-8 (0x02); 15*2^-10 (7*2^-9|2^-6) -> 2^-6 (0x08);
    # 432 (416|448) -> 448 (0x7E); 400 (384|416) -> 384 (0x7C)
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, -1.0625: 0xB8,
             15 * 2.0 ** -10: 0x08, 432.0: 0x7E, 400.0: 0x7C}
    for v, c in cases.items():
        assert int(fp8.e4m3_encode(np.array([v]))[0]) == c, v


def test_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 3000), rng.normal(0, 2.0 ** -7, 3000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000)])
    got = fp8.e4m3_encode(v)
    finite = np.array([c for c in range(256) if not np.isnan(fp8.E4M3_TABLE[c])])
    vals = fp8.E4M3_TABLE[finite]
    for x, g in zip(v, got):
        d = np.abs(vals - x)
        best = finite[d == d.min()]
        best = best[np.sign(fp8.E4M3_TABLE[best]) * np.sign(x) >= 0] if x != 0 else best
        if len(best) > 1:                          # a tie (or +-0): the even code wins
            best = best[best % 2 == 0]
        assert g in best, (x, g, best)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))


def test_block_exponent_rule():
    assert fp8.block_exponent(448.0) == 0
    assert fp8.block_exponent(449.0) == 1
    assert fp8.block_exponent(224.0) == -1
    assert fp8.block_exponent(224.5) == 0
    assert fp8.block_exponent(0.0) == 0
    for amax in np.random.default_rng(1).lognormal(0, 6, 500):
        k = fp8.block_exponent(float(amax))
        assert amax <= 448 * 2.0 ** k and amax > 448 * 2.0 ** (k - 1)


def test_quantize_blocks_and_error_bound():
    rng = np.random.default_rng(7)
    R, C = 300, 260                                    # ragged blocks on both axes
    w = rng.normal(0, 0.02, (R, C))
    w[:128, :128] *= 1000                              # one block on another scale
    w[128:256, 128:256] = 0                            # an all-zero block
    w = w.astype(np.float32).astype(np.float64)
    codes, ks = fp8.quantize(w)
    assert ks.shape == (3, 3) and ks[1, 1] == 0 and ks[0, 0] > ks[0, 1]
    wq = fp8.dequantize(codes, ks)
    for i in range(3):
        for j in range(3):
            blk = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
            k = ks[i, j]
            a = np.abs(w[blk])
            assert np.abs(w[blk] / 2.0 ** k).max() <= 448
            # round to nearest: half an ulp, 2^-4 relative for normals, 2^-10 * 2^k below
            bound = np.maximum(a * 2.0 ** -4, 2.0 ** (k - 10))
            assert np.all(np.abs(wq[blk] - w[blk]) <= bound)
    # dequantized values are exact in bf16: at most 8 significant bits
    m, _ = np.frexp(wq[wq != 0])
    assert np.all((m * 256) == np.round(m * 256))


def test_quantize_planted_mistake_is_caught():
    """Truncation toward zero instead of rounding breaks the half-ulp bound used above."""
    rng = np.random.default_rng(9)
    w = rng.normal(0, 1, (128, 128))
    k = fp8.block_exponent(float(np.abs(w).max()))
    a = np.abs(w) / 2.0 ** k
    pos = fp8.E4M3_TABLE[:0x7F]
    trunc = pos[np.searchsorted(pos, a, side="right") - 1] * 2.0 ** k * np.sign(w)
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** (k - 10))
    assert np.any(np.abs(trunc - w) > bound)
    wq = fp8.dequantize(*fp8.quantize(w))
    assert np.all(np.abs(wq - w) <= bound)


# ---- activations: 1 x 128 blocks (the FP8 MFMA layer) -----------------------------------

def test_quantize_rows_matches_bruteforce_and_blocks():
    g = np.random.default_rng(11)
    x = g.standard_normal((5, 300)) * np.array([[1e-3], [1.0], [30.0], [0.0], [1e4]])
    x[3, :] = 0.0
    x[1, 130] = 448.0 * 2 ** -3       # a block maximum exactly on a scale boundary
    codes, ks = fp8.quantize_rows(x)
    assert codes.shape == (5, 300) and ks.shape == (5, 3)
    for r in range(5):
        for cb in range(3):
            blk = x[r, cb * 128:(cb + 1) * 128]
            k = fp8.block_exponent(float(np.abs(blk).max()))
            assert ks[r, cb] == k
            for j, v in enumerate(blk):
                # brute force: the nearest E4M3 value of v / 2^k, ties to the even code
                t = v / 2.0 ** k
                vals = fp8.E4M3_TABLE[:0x7F]
                dist = np.abs(np.abs(t) - vals)
                best = np.nonzero(dist == dist.min())[0]
                want = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
                want |= 0x80 if np.signbit(t) else 0
                assert codes[r, cb * 128 + j] == want, (r, cb, j, t)
    assert ks[1, 1] == -3 and codes[1, 130] == 0x7E      # 448 * 2^-3 -> k = -3, code 448
    assert (ks[3] == 0).all() and (codes[3] == 0).all()
    np.testing.assert_array_equal(fp8.dequantize_rows(codes, ks)[3], 0.0)
    # each dequantized value within half an E4M3 step (2^-4 relative for normals) of x
    d = fp8.dequantize_rows(codes, ks)
    big = np.abs(x) >= 2.0 ** -6 * 2.0 ** np.repeat(ks, 128, axis=1)[:, :300]
    assert np.all(np.abs(d - x)[big] <= np.abs(x)[big] * 2 ** -4 + 1e-300)


def test_fp8_act_expert_reduces_to_weight_only_on_exact_inputs():
    """Inputs and H already representable in their block FP8 make the FP8 MFMA expert equal
    the bf16-activation expert on the same dequantized weights; in general it differs by
    the activation rounding only (a few % at most)."""
    from oracle import moe as orc
    g = np.random.default_rng(12)
    X = fp8.dequantize_rows(*fp8.quantize_rows(g.standard_normal((7, 256))))
    wg = fp8.dequantize(*fp8.quantize(g.standard_normal((128, 256)) / 16))
    wu = fp8.dequantize(*fp8.quantize(g.standard_normal((128, 256)) / 16))
    wd = fp8.dequantize(*fp8.quantize(g.standard_normal((256, 128)) / 11))
    np.testing.assert_array_equal(fp8.dequantize_rows(*fp8.quantize_rows(X)), X)   # idempotent
    a = fp8.fp8_act_expert(X, wg, wu, wd)
    b = orc.swiglu_expert(X, wg, wu, wd)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 0 < rel < 0.05              # H's rounding is the only difference left
    Hq = fp8.dequantize_rows(*fp8.quantize_rows(orc.silu(X @ wg.T) * (X @ wu.T)))
    np.testing.assert_allclose(a, Hq @ wd.T, rtol=1e-13, atol=1e-15)


def test_fp8_act_hidden_is_the_first_half_of_the_expert():
    from oracle import moe as orc
    g = np.random.default_rng(13)
    X = g.standard_normal((5, 256))
    wg, wu = g.standard_normal((128, 256)) / 16, g.standard_normal((128, 256)) / 16
    wd = g.standard_normal((256, 128)) / 11
    Xq, G, U, H = fp8.fp8_act_hidden(X, wg, wu)
    np.testing.assert_array_equal(Xq, fp8.dequantize_rows(*fp8.quantize_rows(X)))
    # the expert as a plain SwiGLU block on Q(X), with H quantized before W_down
    np.testing.assert_allclose(H, orc.swiglu_expert(Xq, wg, wu, np.eye(128)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fp8.fp8_act_expert(X, wg, wu, wd),
                               fp8.dequantize_rows(*fp8.quantize_rows(H)) @ wd.T, rtol=1e-13, atol=1e-15)


def _deq_rows(a):
    return fp8.dequantize_rows(*fp8.quantize_rows(a))


def test_rows_requant_bound_zero_uncertainty_and_exact_cases():
    g = np.random.default_rng(14)
    a = g.standard_normal((4, 300)) * np.array([[1e-3], [1.0], [30.0], [1e4]])
    np.testing.assert_array_equal(fp8.rows_requant_bound(a, np.zeros_like(a)), 0.0)
    # block 0 of row 0: maximum 448 (k = 0); 1.0625 is the midpoint of 1.0 and 1.125, 1.0
    # is an E4M3 value, 1.03 is 0.03 from the nearest midpoint
    b = np.zeros((1, 128))
    b[0, :4] = [448.0, 1.0625, 1.0, 1.03]
    err = np.zeros_like(b)
    err[0, 1:4] = 1e-6
    d = fp8.rows_requant_bound(b, err)
    assert d[0, 1] == 0.125 and d[0, 2] == 0.0 and d[0, 3] == 0.0 and d[0, 0] == 0.0
    # the block maximum on the scale boundary 448 * 2^0 with any uncertainty: the scale may
    # change, so every element of the block is flagged
    err[0, 0] = 1e-9
    d = fp8.rows_requant_bound(b, err)
    assert (d[0] > 0).all()


def test_rows_requant_bound_holds_under_brute_force_perturbation():
    """Definition check: for random rows, uncertainties and perturbations within them (the
    endpoints included), the requantized values never move by more than the bound."""
    g = np.random.default_rng(15)
    R, C = 6, 260
    a = g.standard_normal((R, C)) * np.exp2(g.integers(-12, 12, (R, 1)))
    a[0, 5] = 448.0 * 2.0 ** -3                             # a block maximum on a scale boundary
    a[1, :] = 0.0
    a[1, 3] = 1e-30
    mids = (fp8.E4M3_TABLE[1:0x7F] + fp8.E4M3_TABLE[0:0x7E]) / 2     # planted midpoints (k = 0 block)
    a[2, 128:256] = g.choice(mids, 128) * g.choice([-1.0, 1.0], 128)
    a[2, 128] = 448.0
    err = np.abs(a) * 10.0 ** g.uniform(-7, -2, (R, C)) + 1e-40
    delta = fp8.rows_requant_bound(a, err)
    q0 = _deq_rows(a)
    flagged = int((delta > 0).sum())
    assert 0 < flagged < a.size
    for t in range(60):
        if t == 0:
            s = np.ones_like(a)
        elif t == 1:
            s = -np.ones_like(a)
        else:
            s = g.choice([-1.0, 1.0, 0.0], a.shape) * (g.uniform(0, 1, a.shape) if t % 2 else 1.0)
        q = _deq_rows(a + s * err)
        assert np.all(np.abs(q - q0) <= delta), t
    # and the bound is reached at planted midpoints: moving across one changes the code
    moved = _deq_rows(a + err) != q0
    assert moved[2, 129:256].any()

