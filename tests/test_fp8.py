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
