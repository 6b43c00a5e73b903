"""E4M3 codec of the oracle (test infrastructure only).

The pages adopt E4M3 -- 4 exponent bits, 3 mantissa bits -- on all tensors
([why-be] hybrid-format paragraph; [thedaegu] Figure 6 passage).  They give
no bit layout, bias or maximum; the reading used here is the OCP 8-bit
floating-point E4M3 ("E4M3FN") encoding:

  * bit 7 = sign, bits 6..3 = exponent field E (bias 7), bits 2..0 = mantissa M;
  * E == 0: subnormal, value (M / 8) * 2**-6;
  * E == 15 and M == 7: NaN (no infinities);
  * otherwise (1 + M / 8) * 2**(E - 7); largest finite magnitude 448 (0x7E).

Encoding is round-to-nearest, ties to the code with an even mantissa, with
saturation to 448 for magnitudes beyond the largest finite value, and the
sign kept (so -0 -> 0x80).

Parity: pinned by tests/test_oracle_codec.py -- a brute-force nearest-code
search in exact integer arithmetic over every finite bf16 pattern, exact
rational checks on random fp32 values, ``torch.float8_e4m3fn`` casts (an
independent library) over the in-range fp32 domain, and hand-derived
points from the definition above.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_table():
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 15 and m == 7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_DECODE = _decode_table()
# Magnitudes of the 127 finite non-negative codes 0x00..0x7E, ascending.
_MAGS = _DECODE[:127].copy()
assert np.all(np.diff(_MAGS) > 0)


def code_magnitudes():
    """The 127 finite non-negative E4M3 magnitudes, ascending (code = index)."""
    return _MAGS.copy()


def decode(q):
    """Value of each E4M3 byte as float64 (exact); NaN for 0x7F / 0xFF."""
    q = np.asarray(q, dtype=np.uint8)
    return _DECODE[q]


def encode(v):
    """Round finite values to E4M3 bytes: nearest, ties to even mantissa,
    saturating at +-448, keeping the sign of zero.

    ``v`` is any float array (float32 in the method); the decision is taken
    exactly in float64, which holds every float32 value and every midpoint
    between adjacent E4M3 magnitudes exactly.
    """
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 oracle: non-finite input is outside the contract")
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(_MAGS, a, side="left")      # first magnitude >= a
    hi = np.minimum(hi, 126)                           # beyond 448: saturate
    lo = np.maximum(hi - 1, 0)
    mid = (_MAGS[lo] + _MAGS[hi]) * 0.5                # exact in float64
    take_hi = a > mid
    tie = a == mid
    # between two adjacent codes exactly one has mantissa LSB (bit 0) == 0
    even_hi = (hi & 1) == 0
    take_hi = take_hi | (tie & even_hi)
    mag_code = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (mag_code | sign).astype(np.uint8)
