"""The GPU quantizer's division x / s against correctly rounded fp32
division, swept over (x, s) pairs.

Each 1x128 tile has one element that fixes its amax a (a positive finite
bf16 value), so its scale is s = max(RN32(a / 448), 2^-126) (or the
power-of-two rule); the other 127 slots hold bf16 values x with |x| <= a.
Over the tiles of one a, the x run through EVERY bf16 value of magnitude at
most a, both signs and both zeros.  The amax values are every 8th positive
finite bf16 pattern plus the largest one: 4081 scales spread over every
binade, from a = 2^-133 (scale floored at 2^-126) to the largest finite
bf16 value.  That is about 1.3e8 (x, s) pairs, compared byte for byte (and
scale for scale) with the oracle's quantize_1x128, whose quotient is NumPy's
IEEE fp32 division.

The method: derive the scale from the tile's online max-abs, then quantize
the tile with it ([thedaegu], last paragraph on fine-grained quantization;
[why-be], same passage).  The GPU forms the quotient with y = RN(1/s) and
Markstein's FMA correction; this test is the pin that the result is the
correctly rounded quotient on every pair it covers."""

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_x1_amd import tensors as T
from gpu_util import bf16_dev, f32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

MAX_FINITE = 0x7F7F
AMAX_PATTERNS = np.unique(np.concatenate([np.arange(1, MAX_FINITE + 1, 8), [MAX_FINITE]])).astype(np.uint16)


def tiles_for(amax_patterns):
    """Tiles [n][128] of bf16 patterns: slot 0 the amax, slots 1..127 every
    bf16 x with |x| <= amax (zero padding in the last tile of each amax)."""
    out = []
    for ua in amax_patterns:
        pos = np.arange(0, int(ua) + 1, dtype=np.uint32).astype(np.uint16)
        xs = np.concatenate([pos, pos | np.uint16(0x8000)])
        n = -(-len(xs) // 127)
        xs = np.concatenate([xs, np.zeros(n * 127 - len(xs), np.uint16)])
        t = np.empty((n, 128), np.uint16)
        t[:, 0] = ua
        t[:, 1:] = xs.reshape(n, 127)
        out.append(t)
    return np.concatenate(out)


@pytest.mark.parametrize("pow2,rule,stride", [(False, oracle.SCALE_AMAX, 1),
                                              (True, oracle.SCALE_POW2, 4)],
                         ids=["amax", "pow2"])
def test_quotient_sweep_every_x_below_each_amax(pow2, rule, stride):
    pats = AMAX_PATTERNS[::stride]
    pairs = 0
    for c0 in range(0, len(pats), 128):
        bits = tiles_for(pats[c0:c0 + 128])
        # the tile-major layout the oracle returns ([tiles][1] scales)
        q, s = T.quantize_1x128(bf16_dev(bits), pow2=pow2, scale_layout="row_major")
        qo, so = oracle.quantize_1x128(f32(bits), rule)
        qh, sh = host(q), host(s)
        assert np.array_equal(sh, so), c0
        bad = np.flatnonzero(qh != qo)
        if bad.size:
            x = f32(bits).flat[bad[:8]]
            sc = so.flat[bad[:8] // 128]
            raise AssertionError("bytes differ at %d of %d elements, e.g. x=%s s=%s gpu=%s oracle=%s" % (
                bad.size, qh.size, x.tolist(), sc.tolist(), qh.flat[bad[:8]].tolist(),
                qo.flat[bad[:8]].tolist()))
        pairs += bits.size - bits.shape[0]
    say("%s: %d amax values, %d (x, s) pairs, all bytes equal" % (
        "pow2" if pow2 else "amax", len(pats), pairs))
