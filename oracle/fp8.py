"""Plain CPU oracle of the block-FP8 expert weights (numpy).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the GPU library.

The pages (LongCat-Flash article, itouyu.top / kqgmpj.cn / dhxrcw.cn, section
"System-level optimisation", quantization paragraph) say the model uses the same
fine-grained block-level quantization as DeepSeek-V3: FP8 values with one scale per block
of a weight matrix.  They fix neither the FP8 variant, the block shape nor the scale
format.  Readings taken here:
  * FP8 = OCP E4M3 (bias 7, no infinities, largest finite 448, NaN = S.1111.111);
  * blocks of 128 rows x 128 reduction columns of every expert matrix (W_gate and W_up
    [I][d], W_down [d][I]), the DeepSeek-V3 weight block; partial blocks at the edges;
  * the block scale is a power of two, 2^k with k the smallest integer such that the
    block's largest |w| <= 448 * 2^k (k = 0 for an all-zero block), so w / 2^k is exact
    and fits E4M3, and code * 2^k is exact in bf16;
  * each w / 2^k is rounded to the nearest E4M3 value, ties to the even code;
  * weights only: activations stay bf16, and the layer computed is the bf16 layer with
    every expert weight replaced by its dequantized value code * 2^k.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (OCP FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# all 256 codes; the finite non-negative ones in ascending order (codes 0x00..0x7E)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)])
_POS_CODES = np.arange(0x7F)
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each finite v with |v| <= 448, ties to the even code; the sign
    bit follows v's sign (negative zero -> 0x80)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or not np.all(np.isfinite(a)):
        raise ValueError("E4M3 encode: values must be finite with magnitude <= 448")
    hi = np.searchsorted(_POS_VALUES, a, side="left").clip(0, 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def block_exponent(amax: float) -> int:
    """Smallest integer k with amax <= 448 * 2^k (0 when amax == 0)."""
    if amax == 0:
        return 0
    k = int(np.ceil(np.log2(amax / E4M3_MAX)))
    while E4M3_MAX * 2.0 ** k < amax:
        k += 1
    while E4M3_MAX * 2.0 ** (k - 1) >= amax:
        k -= 1
    return k


def quantize(w):
    """Block-FP8 quantization of one matrix w [rows][cols] (values exact in fp64):
    returns (codes uint8 [rows][cols], k int [ceil(rows/128)][ceil(cols/128)])."""
    w = np.asarray(w, np.float64)
    R, C = w.shape
    nrb, ncb = -(-R // BLOCK), -(-C // BLOCK)
    pad = np.zeros((nrb * BLOCK, ncb * BLOCK))
    pad[:R, :C] = np.abs(w)
    amax = pad.reshape(nrb, BLOCK, ncb, BLOCK).max(axis=(1, 3))
    ks = np.array([[block_exponent(float(a)) for a in row] for row in amax], np.int64)
    scale = np.repeat(np.repeat(2.0 ** ks, BLOCK, axis=0), BLOCK, axis=1)[:R, :C]
    return e4m3_encode(w / scale), ks


def dequantize(codes, ks):
    """code * 2^k per element (fp64; exact)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    scale = np.repeat(np.repeat(2.0 ** np.asarray(ks, np.float64), BLOCK, axis=0), BLOCK, axis=1)[:R, :C]
    return E4M3_TABLE[codes] * scale
