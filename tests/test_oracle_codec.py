"""Pins for the oracle's E4M3 codec (CPU only).

The codec is checked against things other than itself:
  * brute force: the nearest of all 127 finite magnitudes, ties to the even
    mantissa, computed in exact integer / rational arithmetic;
  * an independent library: torch's float8_e4m3fn casts (RNE; it returns NaN
    instead of saturating beyond 464, so it is compared below 464 only);
  * points derived by hand from the OCP E4M3 definition.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_all_codes():
    ours = oracle.decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_hand_points():
    d = oracle.decode
    assert d(np.uint8(0x7E)) == 448.0                # 1.75 * 2**8
    assert d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x01)) == 2.0 ** -9             # smallest subnormal
    assert d(np.uint8(0x07)) == 7 * 2.0 ** -9         # largest subnormal
    assert d(np.uint8(0x08)) == 2.0 ** -6             # smallest normal
    assert d(np.uint8(0x38)) == 1.0                   # E = 7, M = 0
    assert d(np.uint8(0x78)) == 256.0                 # E = 15, M = 0
    assert d(np.uint8(0x76)) == 224.0
    assert d(np.uint8(0x77)) == 240.0
    assert np.isnan(d(np.uint8(0x7F)))


def _brute_codes_int(vals_scaled, mags_scaled):
    """argmin_c |v - mag_c| with ties to the even code; integer inputs."""
    d = np.abs(vals_scaled[:, None] - mags_scaled[None, :])
    # lexicographic: distance first, then odd codes lose ties
    key = d * 2 + (np.arange(127)[None, :] & 1)
    return np.argmin(key, axis=1)


def test_encode_brute_force_all_bf16_in_exact_range():
    # every finite bf16 pattern with 2**-20 <= |v| < 2**20: v * 2**27 and every
    # E4M3 magnitude * 2**27 are integers below 2**47, so the distances are exact.
    bits = np.arange(0x10000, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(vals.astype(np.float64))
    sel = np.isfinite(vals) & (a >= 2.0 ** -20) & (a < 2.0 ** 20)
    v = vals[sel]
    vi = (np.abs(v.astype(np.float64)) * 2.0 ** 27).astype(np.int64)
    assert np.array_equal(vi.astype(np.float64), np.abs(v.astype(np.float64)) * 2.0 ** 27)
    mi = (e4m3.code_magnitudes() * 2.0 ** 27).astype(np.int64)
    expect = _brute_codes_int(vi, mi).astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7)
    got = oracle.encode(v)
    assert np.array_equal(got, expect), np.flatnonzero(got != expect)[:10]


def _brute_code_fraction(x):
    fx = Fraction(float(x))
    best = None
    for c in range(127):
        m = Fraction(float(e4m3.code_magnitudes()[c]))
        dist = abs(abs(fx) - m)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    if np.signbit(x):
        code |= 0x80
    return code


def test_encode_brute_force_rational_outside_int_range_and_random_f32():
    rng = np.random.default_rng(7)
    samples = []
    # bf16 values outside the integer-exact window: tiny and huge, both signs
    for e in list(range(-133, -20, 3)) + list(range(20, 128, 5)):
        for m in (0, 1, 37, 127):
            for sgn in (1.0, -1.0):
                samples.append(sgn * (1 + m / 128.0) * 2.0 ** e)
    # random float32 bit patterns across the finite range
    bits = rng.integers(0, 2 ** 32, size=400, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    samples += [float(t) for t in f[np.isfinite(f)]]
    # random float32 values inside (-500, 500) where rounding decisions happen
    samples += [float(t) for t in (rng.standard_normal(400).astype(np.float32) * 100)]
    x = np.array(samples, dtype=np.float32)
    got = oracle.encode(x)
    expect = np.array([_brute_code_fraction(t) for t in x], dtype=np.uint8)
    assert np.array_equal(got, expect)


def test_encode_midpoints_and_neighbours_fraction():
    mags = e4m3.code_magnitudes()
    pts = []
    for i in range(126):
        mid = np.float32((mags[i] + mags[i + 1]) / 2)
        assert float(mid) == (mags[i] + mags[i + 1]) / 2   # midpoints are fp32-exact
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
        pts += [np.float32(mags[i])]
    pts += [np.float32(448.0), np.nextafter(np.float32(448.0), np.float32(1e9)),
            np.float32(463.99997), np.float32(464.0), np.float32(1e30)]
    x = np.array(pts, dtype=np.float32)
    x = np.concatenate([x, -x])
    got = oracle.encode(x)
    expect = np.array([_brute_code_fraction(t) for t in x], dtype=np.uint8)
    assert np.array_equal(got, expect)


def test_encode_matches_torch_cast_below_464():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 464.0)]
    # plus every bf16 pattern below 464
    b = (np.arange(0x10000, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b) & (np.abs(b) < 464.0)]
    x = np.concatenate([f, b, rng.uniform(-463, 463, 1_000_000).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode(x)
    assert np.array_equal(got, ref), (x[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])


def test_encode_hand_points():
    e = lambda v: int(oracle.encode(np.float32(v)))
    assert e(2.0 ** -10) == 0x00        # halfway between 0 and 2**-9 -> even (0)
    assert e(-2.0 ** -10) == 0x80
    assert e(1.5 * 2.0 ** -9) == 0x02   # halfway 2**-9 (M=1) / 2**-8 (M=2) -> M=2
    assert e(432.0) == 0x7E             # halfway 416 (M=5) / 448 (M=6) -> 448
    assert e(232.0) == 0x76             # halfway 224 (M=6) / 240 (M=7) -> 224
    assert e(448.0) == 0x7E
    assert e(460.0) == 0x7E and e(1e6) == 0x7E and e(-1e6) == 0xFE   # saturation
    assert e(-0.0) == 0x80 and e(0.0) == 0x00
    assert e(-1e-30) == 0x80
    assert e(1.0) == 0x38 and e(-1.0) == 0xB8
    assert e(256.0) == 0x78


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        oracle.encode(np.array([1.0, np.nan], dtype=np.float32))
