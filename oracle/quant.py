"""Fine-grained FP8 quantizers of the oracle (test infrastructure only).

What the pages fix ([why-be] and [thedaegu], the paragraphs on fine-grained
quantization): the maximum absolute value is computed online for every 1x128
activation tile (one row, 128 consecutive elements along the inner
dimension K) or every 128x128 weight block; a scaling factor is derived from
it so that this max-abs lands on the largest representable FP8 value
([thedaegu], dynamic-range paragraph), and the tile is then quantized to
E4M3.  The backward pass converts such activations from 1x128 tiles to
128x1 tiles (128 consecutive rows of one column), and for some activations
the scaling factors are integral powers of two ([why-be], SwiGLU/backward
paragraph).

Readings where the pages are silent (mirrored by the HIP path):
  * amax rule: s = RN32(amax / 448), floored at 2**-126; q = E4M3(RN32(x / s))
    with IEEE fp32 division (numpy float32 ``/``) -- two roundings.
  * pow2 rule: s = max(2**k, 2**-126) with k the smallest integer such that
    448 * 2**k >= amax (the ceiling of log2(amax / 448)); x / s is exact.
  * requantization 1x128 -> 128x1 starts from the FP8 1x128 tensor: the
    source value is RN32(dec(q1) * s1), then 128x1 quantization of that.
  * logical layouts: every function takes and returns row-major arrays in
    the orientation of its input (the 128x1 quantizer does not transpose;
    the tests compare against the HIP path's transposed output explicitly).

Parity: pinned by tests/test_oracle_quant.py -- end-to-end brute force in
exact rational arithmetic on tiny tiles, the closed form "amax maps to
+-448", the per-element rounding-error bound, power-of-two exactness and
idempotence, metamorphic relations (scaling by 2**k, negation, permutation
within a tile), 128x1(X) == 1x128(X^T) and the one-ulp agreement of the
two tilings.
"""

import numpy as np

from .e4m3 import encode, decode, E4M3_MAX

SCALE_AMAX = 0
SCALE_POW2 = 1

TILE = 128
_F32_MIN_NORMAL = np.float32(2.0 ** -126)


def bf16_bits_to_f32(bits):
    """Interpret uint16 bf16 bit patterns as float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("oracle quantizers take float32 values "
                        "(bf16 inputs are widened exactly first)")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    return x


def amax_scale(amax):
    """s = max(RN32(amax / 448), 2**-126) for float32 amax values."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.maximum(s, _F32_MIN_NORMAL)


def pow2_scale(amax):
    """s = max(2**k, 2**-126), k the least integer with 448 * 2**k >= amax.

    The exponent is first estimated in float64 and then corrected with exact
    comparisons (448 * 2**k is exact in float64 for every k used here).
    """
    amax = np.asarray(amax, dtype=np.float32).astype(np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    k = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # enforce: 448 * 2**k >= amax and 448 * 2**(k-1) < amax
    for _ in range(2):
        too_small = np.ldexp(E4M3_MAX, k) < amax
        k = np.where(too_small, k + 1, k)
        too_big = np.ldexp(E4M3_MAX, k - 1) >= amax
        k = np.where(too_big & (amax > 0), k - 1, k)
    k = np.where(amax > 0, k, -126)
    k = np.maximum(k, -126)
    return np.ldexp(1.0, k).astype(np.float32)


def _scale(amax, rule):
    if rule == SCALE_AMAX:
        return amax_scale(amax)
    if rule == SCALE_POW2:
        return pow2_scale(amax)
    raise ValueError("unknown scale rule %r" % (rule,))


def _quantize_with(x, s_expanded):
    y = (x / s_expanded).astype(np.float32)   # IEEE fp32 division, RN
    return encode(y)


def quantize_1x128(x, rule=SCALE_AMAX):
    """1x128 tiles along each row.  x: float32 [R][C], C % 128 == 0.

    Returns (q uint8 [R][C], s float32 [R][C/128]).
    """
    x = _as_f32(x)
    R, C = x.shape
    if C % TILE:
        raise ValueError("columns must be a multiple of 128")
    t = x.reshape(R, C // TILE, TILE)
    amax = np.max(np.abs(t), axis=2) if R and C else np.zeros((R, C // TILE), np.float32)
    s = _scale(amax, rule)
    q = _quantize_with(t, s[:, :, None]).reshape(R, C)
    return q, s


def quantize_128x1(x, rule=SCALE_AMAX):
    """128x1 tiles: 128 consecutive rows of one column.  x: float32 [R][C],
    R % 128 == 0.  Returns (q uint8 [R][C], s float32 [R/128][C]) in the
    input's orientation."""
    x = _as_f32(x)
    R, C = x.shape
    if R % TILE:
        raise ValueError("rows must be a multiple of 128")
    t = x.reshape(R // TILE, TILE, C)
    amax = np.max(np.abs(t), axis=1) if R and C else np.zeros((R // TILE, C), np.float32)
    s = _scale(amax, rule)
    q = _quantize_with(t, s[:, None, :]).reshape(R, C)
    return q, s


def quantize_128x128(w, rule=SCALE_AMAX):
    """128x128 blocks.  w: float32 [R][C], both multiples of 128.

    Returns (q uint8 [R][C], s float32 [R/128][C/128])."""
    w = _as_f32(w)
    R, C = w.shape
    if R % TILE or C % TILE:
        raise ValueError("both dimensions must be multiples of 128")
    t = w.reshape(R // TILE, TILE, C // TILE, TILE)
    if R and C:
        amax = np.max(np.abs(t), axis=(1, 3))
    else:
        amax = np.zeros((R // TILE, C // TILE), np.float32)
    s = _scale(amax, rule)
    q = _quantize_with(t, s[:, None, :, None]).reshape(R, C)
    return q, s


def quantize_per_tensor(x, rule=SCALE_AMAX):
    """One scale for the whole tensor (the prior practice the pages contrast
    with fine-grained tiles; used only for the naive baseline)."""
    x = _as_f32(x)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    s = _scale(np.float32(amax), rule)
    return _quantize_with(x, s), np.float32(s)


def dequantize_1x128(q, s):
    """float64 values dec(q) * s for 1x128 tiles (exact in float64)."""
    R, C = q.shape
    return decode(q) * np.repeat(s.astype(np.float64), TILE, axis=1)[:, :C]


def dequantize_128x1(q, s):
    R, C = q.shape
    return decode(q) * np.repeat(s.astype(np.float64), TILE, axis=0)[:R, :]


def dequantize_128x128(q, s):
    R, C = q.shape
    full = np.repeat(np.repeat(s.astype(np.float64), TILE, axis=0), TILE, axis=1)
    return decode(q) * full[:R, :C]


def requantize_128x1(q1, s1, rule=SCALE_AMAX):
    """1x128-quantized tensor (q1 [R][C], s1 [R][C/128]) -> 128x1 tiles.

    Source value y = RN32(dec(q1) * s1) in float32, then quantize_128x1(y).
    """
    q1 = np.asarray(q1, dtype=np.uint8)
    R, C = q1.shape
    d = decode(q1).astype(np.float32)                  # exact
    s_exp = np.repeat(np.asarray(s1, np.float32), TILE, axis=1)[:, :C]
    y = (d * s_exp).astype(np.float32)                 # one fp32 rounding
    return quantize_128x1(y, rule)
