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
FP8 activations too (the FP8 MFMA layer): the pages' DeepSeek-V3 scheme also quantizes
activations per block; readings taken: blocks of 1 row x 128 reduction columns (the
DeepSeek-V3 activation tile), the same scale and rounding rules.  The layer then computes
each FFN expert as G = Q(x) Q(W_gate)^T, U = Q(x) Q(W_up)^T, H = silu(G) * U,
Y = Q(H) Q(W_down)^T, with Q the block quantization of each operand (x quantized per
token, H per FFN row), and combines as the bf16 layer (zero-computation experts and the
router see the unquantized x).
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


_BF16_CODES = None


def bf16_code_table():
    """e4m3_encode of every bf16 value, indexed by its 16-bit pattern (a memo of that
    function for bf16 inputs); patterns whose value is not finite or exceeds 448 in
    magnitude are marked False in the second array."""
    global _BF16_CODES
    if _BF16_CODES is None:
        with np.errstate(invalid="ignore"):
            vals = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
            ok = np.isfinite(vals) & (np.abs(vals) <= E4M3_MAX)
        codes = np.zeros(65536, np.uint8)
        codes[ok] = e4m3_encode(vals[ok])
        _BF16_CODES = (codes, ok)
    return _BF16_CODES


def encode_scaled(q) -> np.ndarray:
    """e4m3_encode(q); when every q is a bf16 value (bf16 weights over a power-of-two
    scale always are), through the memo table of bf16_code_table."""
    q = np.asarray(q, np.float64)
    q32 = q.astype(np.float32)
    bits = q32.view(np.uint32)
    if np.array_equal(q32.astype(np.float64), q) and not np.any(bits & np.uint32(0xFFFF)):
        codes, ok = bf16_code_table()
        pat = bits >> np.uint32(16)
        if np.all(ok[pat]):
            return codes[pat]
    return e4m3_encode(q)


def quantize(w):
    """Block-FP8 quantization of one matrix w [rows][cols] (values exact in fp64):
    returns (codes uint8 [rows][cols], k int [ceil(rows/128)][ceil(cols/128)])."""
    w = np.asarray(w, np.float64)
    R, C = w.shape
    nrb, ncb = -(-R // BLOCK), -(-C // BLOCK)
    pad = np.zeros((nrb * BLOCK, ncb * BLOCK))
    pad[:R, :C] = w
    blocks = pad.reshape(nrb, BLOCK, ncb, BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3))
    ks = np.array([[block_exponent(float(a)) for a in row] for row in amax], np.int64)
    q = (blocks / (2.0 ** ks)[:, None, :, None]).reshape(nrb * BLOCK, ncb * BLOCK)[:R, :C]
    return encode_scaled(q), ks


def quantize_rows(a):
    """Block-FP8 quantization of the rows of a [rows][cols] in blocks of 1 row x 128
    columns (activations): returns (codes uint8 [rows][cols], k int [rows][ceil(cols/128)])."""
    a = np.asarray(a, np.float64)
    R, C = a.shape
    ncb = -(-C // BLOCK)
    pad = np.zeros((R, ncb * BLOCK))
    pad[:, :C] = a
    blocks = pad.reshape(R, ncb, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    ks = np.array([[block_exponent(float(v)) for v in row] for row in amax], np.int64)
    q = (blocks / (2.0 ** ks)[:, :, None]).reshape(R, ncb * BLOCK)[:, :C]
    return encode_scaled(q), ks


def dequantize_rows(codes, ks):
    """code * 2^k per element for 1 x 128 blocks (fp64; exact)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    ks = np.asarray(ks, np.float64)
    pad = np.zeros((R, ks.shape[1] * BLOCK))
    pad[:, :C] = E4M3_TABLE[codes]
    return (pad.reshape(R, ks.shape[1], BLOCK) * (2.0 ** ks)[:, :, None]).reshape(R, -1)[:, :C]


def fp8_act_hidden(X, wq_gate, wq_up):
    """The first half of one FFN expert of the FP8 MFMA layer on rows X [m,d] (fp64) with
    dequantized block-FP8 weights: (Q(X), G, U, H) with G = Q(X) Q(W_gate)^T,
    U = Q(X) Q(W_up)^T, H = silu(G) * U (Q(X) dequantized)."""
    from .moe import silu
    Xq = dequantize_rows(*quantize_rows(X))
    G = Xq @ wq_gate.T
    U = Xq @ wq_up.T
    return Xq, G, U, silu(G) * U


def fp8_act_expert(X, wq_gate, wq_up, wq_down):
    """One FFN expert of the FP8 MFMA layer on rows X [m,d] (fp64) with dequantized block-FP8
    weights: Y = Q(H) Q(W_down)^T with H = silu(Q(X) Q(W_gate)^T) * (Q(X) Q(W_up)^T)."""
    H = fp8_act_hidden(X, wq_gate, wq_up)[3]
    return dequantize_rows(*quantize_rows(H)) @ wq_down.T


def rows_requant_bound(a, err):
    """How far the row quantization of a can move when a is known only to within err.

    a [R][C] (fp64) is quantized in blocks of 1 row x 128 columns (quantize_rows); err [R][C]
    >= 0 is an absolute uncertainty per element (for instance the rounding error of a
    computation that produced a in another precision).  Returns delta [R][C] >= 0 with
    |dequantize_rows(quantize_rows(a'))[i] - dequantize_rows(quantize_rows(a))[i]| <=
    delta[i] for every a' with |a' - a| <= err elementwise; delta is 0 where neither the
    element's code nor its block's scale can change.
      * Block scale: the block maximum of |a'| lies in [lo, hi] (lo = max(|a| - err, 0),
        hi = max(|a| + err) over the block); if block_exponent(lo) != block_exponent(hi)
        the scale may change and every element of the block gets the coarse bound
        err + 2^-3 (|a| + err) + 2^(k_hi - 9): each side is within half an E4M3 step of
        its input (2^-4 of the value for normals, 2^(k - 10) below them).
      * Fixed scale 2^k: rounding to the nearest E4M3 value is monotone, so a' / 2^k rounds
        to a value between the roundings of (a - err) / 2^k and (a + err) / 2^k:
        delta = 2^k * max distance of those two from the rounding of a / 2^k.
    """
    a = np.asarray(a, np.float64)
    err = np.asarray(err, np.float64)
    R, C = a.shape
    ncb = -(-C // BLOCK)
    pad = lambda m: np.pad(m, ((0, 0), (0, ncb * BLOCK - C))).reshape(R, ncb, BLOCK)  # noqa: E731
    A, Er = pad(a), pad(err)
    lo = np.maximum(np.abs(A) - Er, 0.0).max(axis=2)
    hi = (np.abs(A) + Er).max(axis=2)
    k0 = np.array([[block_exponent(float(v)) for v in row] for row in np.abs(A).max(axis=2)], np.int64)
    k_lo = np.array([[block_exponent(float(v)) for v in row] for row in lo], np.int64)
    k_hi = np.array([[block_exponent(float(v)) for v in row] for row in hi], np.int64)
    sc = (2.0 ** k0)[:, :, None]
    fixed = (k_lo == k_hi)[:, :, None] & np.ones_like(A, bool)
    val = lambda t: E4M3_TABLE[e4m3_encode(np.where(fixed, t, 0.0))]  # noqa: E731
    q0, q_lo, q_hi = val(A / sc), val((A - Er) / sc), val((A + Er) / sc)
    delta = np.where(fixed, sc * np.maximum(np.abs(q_hi - q0), np.abs(q_lo - q0)),
                     Er + 2.0 ** -3 * (np.abs(A) + Er) + (2.0 ** (k_hi - 9))[:, :, None])
    return delta.reshape(R, ncb * BLOCK)[:, :C]


def dequantize(codes, ks):
    """code * 2^k per element (fp64; exact)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    ks = np.asarray(ks, np.float64)
    nrb, ncb = ks.shape
    pad = np.zeros((nrb * BLOCK, ncb * BLOCK))
    pad[:R, :C] = E4M3_TABLE[codes]
    out = pad.reshape(nrb, BLOCK, ncb, BLOCK) * (2.0 ** ks)[:, None, :, None]
    return out.reshape(nrb * BLOCK, ncb * BLOCK)[:R, :C]
