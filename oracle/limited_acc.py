"""Limited-width fixed-point accumulation of FP8 products.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests to put
the pages' accumulation-error figure beside the measured gap of the naive
per-tensor baseline.  Not part of the product path.

What it models ([hearaon], paragraph on FP8 GEMM accumulation precision
in tensor cores): inside an FP8 MMA the products are brought to a common
exponent by right-shifting their mantissas, with sign fill, according to
the largest exponent; only the highest 14 bits of each shifted product are
kept and lower bits are cut off.  [why-be] and [thedaegu] (limited
accumulation paragraphs) report a maximum relative error of nearly 2% for
K = 4096 in a preliminary test, and [thedaegu] says the effect grows with K.

Readings where the pages are silent:
  * One accumulation step adds ``group`` consecutive products of the dot
    product (default 32, the K extent of one FP8 MMA instruction of the
    architecture the pages name).  With ``align_accumulator`` (default) the
    running sum is one more addend of the step and is aligned with the
    products, which is what makes the error grow with K; without it the
    step's products are summed this way and the group sum is added to an
    FP32 accumulator with round-to-nearest-even.
  * "The highest ``bits`` bits" are counted from the leading one of the
    largest-magnitude addend of the step: with that leading one at 2**L,
    every addend is cut to a multiple of 2**(L - bits + 1).
  * Right-shifting a two's-complement value with sign fill rounds it
    toward minus infinity, so the cut is ``floor``: positive addends lose
    their low bits, negative ones grow by up to one unit of the last kept
    bit.
  * The kept values are added exactly; the step result is rounded to FP32
    (it is exact whenever bits + log2(group + 1) <= 24).

Parity status: pinned by ``tests/test_oracle_limited_acc.py`` (hand-worked
steps that follow the passage, an integer shift-register implementation of
the same description on random FP8 products, the wide-window limit that
reduces to FP32 summation of exact group sums, and the one-sided error of a
floor cut).
"""

import numpy as np

from .e4m3 import decode


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _cut(addends, bits):
    """Cut each row of ``addends`` (float64, exact) to ``bits`` bits below the
    leading one of the row's largest magnitude, rounding toward -inf."""
    mx = np.max(np.abs(addends), axis=-1)
    _, e = np.frexp(np.where(mx > 0, mx, 1.0))  # mx = m * 2**e, m in [0.5, 1): leading one at 2**(e-1)
    quantum = np.ldexp(1.0, (e - bits).astype(np.int64))[..., None]
    return np.floor(addends / quantum) * quantum


def limited_dot(products, group=32, bits=14, align_accumulator=True):
    """Sum the last axis of ``products`` (exact values, float64) with the
    limited-width accumulation described above.  Returns float64 values that
    are FP32 numbers."""
    # kept addends are multiples of one power of two below 2**(lead + 1): a
    # step's float64 sum is exact while bits + log2(group + 1) + 1 <= 53
    assert 1 <= bits <= 40 and group >= 1
    p = np.asarray(products, dtype=np.float64)
    lead, K = p.shape[:-1], p.shape[-1]
    acc = np.zeros(lead, dtype=np.float64)
    for k0 in range(0, K, group):
        chunk = p[..., k0:k0 + group]
        if align_accumulator:
            addends = np.concatenate([acc[..., None], chunk], axis=-1)
            acc = _f32(np.sum(_cut(addends, bits), axis=-1))
        else:
            acc = _f32(acc + np.sum(_cut(chunk, bits), axis=-1))
    return acc


def gemm_limited_per_tensor(qa, s_a, qb, s_b, group=32, bits=14, align_accumulator=True):
    """The naive baseline of the pages' error discussion: E4M3 operands with
    one scale each, the whole K summed in the limited-width accumulator, the
    two scales applied once at the end.  qa [M][K], qb [K][N] (E4M3 codes)."""
    a = decode(np.asarray(qa))
    b = decode(np.asarray(qb))
    prods = a[:, None, :] * b.T[None, :, :]  # exact: 4-bit significands
    acc = limited_dot(prods, group, bits, align_accumulator)
    return (np.float64(s_a) * np.float64(s_b)) * acc
