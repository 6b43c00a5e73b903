"""Pins for the oracle's quantizers (CPU only).

Checked against: an end-to-end brute force in exact rational arithmetic on
small tensors; the closed form "the max-abs element lands on +-448"; the
per-element rounding bound; power-of-two exactness and idempotence;
metamorphic relations; the equivalence of 128x1 tiles with 1x128 tiles of
the transpose and the one-ulp agreement of the two tilings.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import e4m3
from fp8_fine_grained_x1_amd import workloads

F = Fraction
MAGS = [F(float(m)) for m in e4m3.code_magnitudes()]


# ---------------------------------------------------------------- helpers
def rn32(fr):
    """Nearest float32 to a rational (ties to even), subnormals included."""
    if fr == 0:
        return F(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    elif F(2) ** (e + 1) <= a:
        e += 1
    assert F(2) ** e <= a < F(2) ** (e + 1)
    e = max(e, -126)
    ulp = F(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def brute_code(v_frac, negative):
    a = abs(v_frac)
    best = None
    for c in range(127):
        key = (abs(a - MAGS[c]), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] | (0x80 if negative else 0)


def brute_scale(amax, rule):
    if rule == oracle.SCALE_AMAX:
        s = rn32(amax / 448)
    else:
        if amax == 0:
            s = F(0)
        else:
            k = 0
            while F(448) * F(2) ** k < amax:
                k += 1
            while F(448) * F(2) ** (k - 1) >= amax:
                k -= 1
            s = F(2) ** k
    return max(s, F(2) ** -126)


def brute_quant_group(xs, rule):
    """xs: 1-D float32 array of one tile / block. Returns (codes, s)."""
    fx = [F(float(x)) for x in xs]
    amax = max(abs(v) for v in fx)
    s = brute_scale(amax, rule)
    codes = [brute_code(rn32(v / s), bool(np.signbit(x))) for v, x in zip(fx, xs)]
    return np.array(codes, dtype=np.uint8), s


def bf16(x):
    return oracle.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, np.float32)))


def sample_tensor(rows, cols, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if outliers:
        idx = rng.choice(x.size, size=max(1, x.size // 100), replace=False)
        x.flat[idx] *= 50
    return bf16(x)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("rule", [oracle.SCALE_AMAX, oracle.SCALE_POW2])
def test_1x128_brute_force(rule):
    x = sample_tensor(3, 256, seed=1)
    # a tile of tiny (bf16-subnormal and near-FLT_MIN) values, a zero tile with
    # signed zeros, a tile whose max is a power of two times 448
    tiny = bf16(np.random.default_rng(2).standard_normal(128) * 1e-38)
    zeros = np.zeros(128, np.float32)
    zeros[::3] = -0.0
    exact = np.linspace(-1, 1, 128, dtype=np.float32)
    exact[5] = 448.0 * 4
    extra = np.stack([np.concatenate([tiny, zeros]), np.concatenate([exact, -exact])])
    x = np.concatenate([x, bf16(extra)])
    q, s = oracle.quantize_1x128(x, rule)
    for r in range(x.shape[0]):
        for t in range(x.shape[1] // 128):
            codes, sb = brute_quant_group(x[r, 128 * t:128 * (t + 1)], rule)
            assert F(float(s[r, t])) == sb, (r, t)
            assert np.array_equal(q[r, 128 * t:128 * (t + 1)], codes), (r, t)


@pytest.mark.parametrize("rule", [oracle.SCALE_AMAX, oracle.SCALE_POW2])
def test_128x128_brute_force_sampled(rule):
    w = sample_tensor(256, 128, seed=3) * np.float32(0.02)
    q, s = oracle.quantize_128x128(w, rule)
    rng = np.random.default_rng(4)
    for bi in range(2):
        blk = w[128 * bi:128 * (bi + 1), :]
        fx = [F(float(v)) for v in blk.ravel()]
        amax = max(abs(v) for v in fx)
        sb = brute_scale(amax, rule)
        assert F(float(s[bi, 0])) == sb
        for flat in rng.choice(blk.size, size=300, replace=False):
            r, c = divmod(int(flat), 128)
            code = brute_code(rn32(F(float(blk[r, c])) / sb), bool(np.signbit(blk[r, c])))
            assert q[128 * bi + r, c] == code


def test_requant_128x1_brute_force():
    x = sample_tensor(256, 128, seed=5)
    q1, s1 = oracle.quantize_1x128(x)
    q2, s2 = oracle.requantize_128x1(q1, s1)
    dec = oracle.decode(q1)
    for c in (0, 17, 127):
        for g in range(2):
            ys = []
            for r in range(128 * g, 128 * (g + 1)):
                ys.append(rn32(F(float(dec[r, c])) * F(float(s1[r, c // 128]))))
            amax = max(abs(v) for v in ys)
            sb = brute_scale(amax, oracle.SCALE_AMAX)
            assert F(float(s2[g, c])) == sb
            for i, r in enumerate(range(128 * g, 128 * (g + 1))):
                neg = bool(np.signbit(dec[r, c]))
                assert q2[r, c] == brute_code(rn32(ys[i] / sb), neg)


# ---------------------------------------------------------------- closed forms
def test_amax_lands_on_448():
    x = sample_tensor(64, 1024, seed=6)
    q, s = oracle.quantize_1x128(x)
    t = x.reshape(64, 8, 128)
    qt = q.reshape(64, 8, 128)
    arg = np.argmax(np.abs(t), axis=2)
    codes = np.take_along_axis(qt, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((codes & 0x7F) == 0x7E)
    # pow2: the max element's code magnitude lies in [224, 448]
    q2, s2 = oracle.quantize_1x128(x, oracle.SCALE_POW2)
    codes2 = np.take_along_axis(q2.reshape(64, 8, 128), arg[:, :, None], axis=2)[:, :, 0]
    mag = np.abs(oracle.decode(codes2))
    assert np.all((mag >= 224) & (mag <= 448))


def _spacing(v):
    v = np.asarray(v, np.float64)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


@pytest.mark.parametrize("rule", [oracle.SCALE_AMAX, oracle.SCALE_POW2])
def test_rounding_error_bound(rule):
    x = sample_tensor(128, 2048, seed=8)
    q, s = oracle.quantize_1x128(x, rule)
    se = np.repeat(s.astype(np.float64), 128, axis=1)
    xd = x.astype(np.float64)
    deq = oracle.decode(q) * se
    v = np.abs(xd) / se
    bound = (0.5 * _spacing(v * (1 + 2.0 ** -23)) + 2.0 ** -24 * v) * se
    assert np.all(np.abs(xd - deq) <= bound * (1 + 1e-12))


def test_pow2_exactness_and_idempotence():
    x = sample_tensor(64, 512, seed=9)
    q, s = oracle.quantize_1x128(x, oracle.SCALE_POW2)
    assert np.all((s.view(np.uint32) & 0x7FFFFF) == 0)
    amax = np.max(np.abs(x.reshape(64, 4, 128)), axis=2).astype(np.float64)
    sd = s.astype(np.float64)
    assert np.all(448 * sd >= amax) and np.all(224 * sd < amax)
    se = np.repeat(s, 128, axis=1)
    d32 = oracle.decode(q).astype(np.float32) * se
    assert np.array_equal(d32.astype(np.float64),
                          oracle.decode(q) * se.astype(np.float64))   # dec(q)*s exact
    q2, s2 = oracle.quantize_1x128(d32, oracle.SCALE_POW2)
    d2 = oracle.decode(q2) * np.repeat(s2.astype(np.float64), 128, axis=1)
    assert np.array_equal(d2, d32.astype(np.float64))


def test_zero_and_tiny_tiles():
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = -0.0
    x[1, 128] = 2.0 ** -130          # bf16-representable subnormal
    for rule in (oracle.SCALE_AMAX, oracle.SCALE_POW2):
        q, s = oracle.quantize_1x128(x, rule)
        assert np.all(s == np.float32(2.0 ** -126))
        assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80)
        assert q[1, 128] == 0x18                       # 2**-130 / 2**-126 = 2**-4


# ---------------------------------------------------------------- metamorphic
@pytest.mark.parametrize("rule", [oracle.SCALE_AMAX, oracle.SCALE_POW2])
def test_metamorphic(rule):
    x = sample_tensor(32, 512, seed=10)
    q, s = oracle.quantize_1x128(x, rule)
    for k in (-5, 3):
        qk, sk = oracle.quantize_1x128((x * np.float32(2.0 ** k)).astype(np.float32), rule)
        assert np.array_equal(qk, q) and np.array_equal(sk, s * np.float32(2.0 ** k))
    qn, sn = oracle.quantize_1x128(-x, rule)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)
    rng = np.random.default_rng(0)
    perm = rng.permutation(128)
    xp = x.reshape(32, 4, 128)[:, :, perm].reshape(32, 512)
    qp, sp = oracle.quantize_1x128(xp, rule)
    assert np.array_equal(qp, q.reshape(32, 4, 128)[:, :, perm].reshape(32, 512))
    assert np.array_equal(sp, s)


@pytest.mark.parametrize("rule", [oracle.SCALE_AMAX, oracle.SCALE_POW2])
def test_128x1_is_1x128_of_transpose(rule):
    x = sample_tensor(256, 384, seed=12)
    q, s = oracle.quantize_128x1(x, rule)
    qt, st = oracle.quantize_1x128(np.ascontiguousarray(x.T), rule)
    assert np.array_equal(q.T, qt) and np.array_equal(s.T, st)
    qb, sb = oracle.quantize_128x128(x, rule)
    qbt, sbt = oracle.quantize_128x128(np.ascontiguousarray(x.T), rule)
    assert np.array_equal(qb.T, qbt) and np.array_equal(sb.T, sbt)


def _ulp(x_abs, s):
    return s * _spacing(x_abs / s)


def test_1x128_and_128x1_agree_within_one_ulp():
    x = sample_tensor(256, 512, seed=13)
    q1, s1 = oracle.quantize_1x128(x)
    q2, s2 = oracle.quantize_128x1(x)
    d1 = oracle.dequantize_1x128(q1, s1)
    d2 = oracle.dequantize_128x1(q2, s2)
    se1 = np.repeat(s1.astype(np.float64), 128, axis=1)
    se2 = np.repeat(s2.astype(np.float64), 128, axis=0)
    ax = np.abs(x.astype(np.float64))
    tol = np.maximum(_ulp(ax, se1), _ulp(ax, se2)) + 2.0 ** -23 * ax
    assert np.all(np.abs(d1 - d2) <= tol)


def test_block_amax_is_max_of_tile_amax():
    # the 128x128 scale equals the 1x128 rule applied to the largest tile amax
    w = sample_tensor(256, 256, seed=14)
    _, sb = oracle.quantize_128x128(w)
    _, st = oracle.quantize_1x128(w)
    blocks = st.reshape(2, 128, 2, 1).max(axis=(1, 3))
    assert np.array_equal(sb, blocks)        # amax_scale is monotone


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.quantize_1x128(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_128x1(np.zeros((100, 128), np.float32))
    with pytest.raises(TypeError):
        oracle.quantize_1x128(np.zeros((2, 128), np.float64))


def test_division_is_correctly_rounded_on_many_elements():
    # the fp32 quotient RN32(x / s) decides the byte; a reciprocal-multiply or
    # a float64 quotient would change ~5e-4 of the bytes, which this catches.
    x = sample_tensor(64, 4096, seed=15)
    q, s = oracle.quantize_1x128(x)
    rng = np.random.default_rng(16)
    idx = rng.choice(x.size, size=60000, replace=False)
    r, c = np.divmod(idx, x.shape[1])
    quot = np.array([float(rn32(F(float(x[i, j])) / F(float(s[i, j // 128]))))
                     for i, j in zip(r, c)], dtype=np.float32)
    quot = np.where(np.signbit(x[r, c]), -np.abs(quot), np.abs(quot)).astype(np.float32)
    assert np.array_equal(oracle.encode(quot), q[r, c])
