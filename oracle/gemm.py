"""Block-scaled FP8 GEMMs of the oracle (test infrastructure only).

What the pages fix ([thedaegu] Figure 7(b) passage, [fooled] promotion
paragraph, [hearaon] accumulation-precision paragraph): the FP8 GEMM's inputs
carry one scaling factor per group of K elements (1x128 activation tiles and
128x128 weight blocks), partial sums are promoted into full-precision FP32
accumulators at a fixed interval along K, and the per-group dequantization
scales are applied there.  All three GEMMs of a Linear (Fprop, Dgrad, Wgrad;
Figure 6 passage) run in FP8, and the MoE up-projection consumes activations
quantized to FP8 before dispatch ([hearaon], [thedaegu]).

The oracle computes the exact mathematical value that the method
approximates in FP32:

    C[m, n] = sum_k (dec(qa[m, k]) * sa[m, k // 128]) * (dec(qb[k, n]) * sb(k, n))

with every dequantized operand exact in float64 (a 4-bit significand times a
24-bit scale) and the sum accumulated in float64 by ``numpy.matmul``.  Where
the method's order of summation and its FP32 roundings land is a matter of
tolerance, not of definition.

Readings: B is handled logically as K x N; weight scales are indexed
(k // 128, n // 128); in the per-column mode (Wgrad, both operands in 128x1
tiles along the token dimension) sb is indexed (k // 128, n).  The BF16
output is RNE of the value.

Parity: pinned by tests/test_oracle_gemm.py -- exact rational dot products
on small shapes, the identity-weight special case, K = 128 exactness,
grouped == per-expert dense, Wgrad == the dense product of transposes.
"""

import numpy as np

from .quant import (dequantize_1x128, dequantize_128x128, dequantize_128x1,
                    TILE)
from .e4m3 import decode


def _f64_matmul(a, b):
    return np.matmul(a.astype(np.float64, copy=False), b.astype(np.float64, copy=False))


def gemm_blockscaled(qa, sa, qb, sb):
    """qa uint8 [M][K] with sa [M][K/128] (1x128 tiles);
    qb uint8 [K][N] (logical) with sb [K/128][N/128] (128x128 blocks).
    Returns float64 [M][N]."""
    A = dequantize_1x128(qa, sa)
    B = dequantize_128x128(qb, sb)
    return _f64_matmul(A, B)


def gemm_blockscaled_colscale(qa, sa, qb, sb):
    """As gemm_blockscaled but B carries one scale per (k // 128, n):
    qb uint8 [K][N] with sb [K/128][N] (128x1 tiles along K)."""
    A = dequantize_1x128(qa, sa)
    B = dequantize_128x1(qb, sb)
    return _f64_matmul(A, B)


def grouped_gemm_blockscaled(qa, sa, offsets, qbs, sbs):
    """Experts e = 0..G-1 own rows offsets[e]:offsets[e+1] of qa / the output;
    expert e's weight is qbs[e] [K][N] with block scales sbs[e].
    Returns float64 [M_total][N]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    M = qa.shape[0]
    N = qbs[0].shape[1] if len(qbs) else 0
    out = np.zeros((M, N), dtype=np.float64)
    for e in range(len(qbs)):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = gemm_blockscaled(qa[r0:r1], sa[r0:r1], qbs[e], sbs[e])
    return out


def wgrad(qx, sx, qdy, sdy):
    """Weight gradient dW = X^T . dY from 128x1-quantized operands.

    qx uint8 [T][F] with sx [T/128][F]; qdy uint8 [T][N] with sdy [T/128][N]
    (128 consecutive tokens per scale).  Returns float64 [F][N]."""
    X = dequantize_128x1(qx, sx)
    DY = dequantize_128x1(qdy, sdy)
    return _f64_matmul(X.T, DY)


def gemm_per_tensor(qa, s_a, qb, s_b):
    """Naive baseline: one scale per tensor, C = sA * sB * (dec(qa) @ dec(qb))."""
    return (np.float64(s_a) * np.float64(s_b)) * _f64_matmul(decode(qa), decode(qb))


def bf16_rne_bits(v):
    """Round float64 (or float32) values to bf16, nearest-even, returning
    uint16 bit patterns.  Finite inputs within bf16 range."""
    v = np.asarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    # bf16 keeps 8 significant bits: round the float64 significand at bit 45
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f32 = r.view(np.float64).astype(np.float32)        # exact: <= 8 bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
