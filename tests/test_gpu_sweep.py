"""Seeded sweeps of shapes through every GEMM planner path: dense (256- and
192-column tiles, the 64-row streaming tiles, N = 128), grouped (random
expert sizes, empty experts, 128-row tails) and per-column scales.  Each
case is small enough for the oracle to check the whole output; the shapes
are drawn once from fixed seeds, so a failure names its case."""

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_x1_amd import tensors as T
from fp8_fine_grained_x1_amd import workloads
from gpu_util import DEV, bf16_dev, check_bf16_output, check_gemm, f32, host, say
from test_gpu_gemm import dense_case, grouped_case, rand_bits

pytestmark = pytest.mark.gpu


def _dense_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 700))]))
        N = 128 * int(rng.integers(1, 13))
        K = 128 * int(rng.integers(1, 11))
        out.append((M, N, K, bool(rng.integers(2)), bool(rng.integers(2)),
                    str(rng.choice(["group_major", "row_major"])), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("M,N,K,a_pow2,b_pow2,layout,seed", _dense_shapes(16, 2024))
def test_dense_shape_sweep(M, N, K, a_pow2, b_pow2, layout, seed):
    a = rand_bits(M, K, seed=seed, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=seed + 1, std=0.02)
    dense_case(a, b, a_pow2=a_pow2, b_pow2=b_pow2, scale_layout=layout,
               what="sweep M=%d N=%d K=%d" % (M, N, K))


def _grouped_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.integers(1, 11))
        avg = int(rng.choice([16, 48, 160, 300]))
        counts = rng.poisson(avg, G)
        counts[rng.random(G) < 0.2] = 0
        N = 128 * int(rng.integers(1, 9))
        K = 128 * int(rng.integers(1, 7))
        out.append((tuple(int(c) for c in counts), N, K, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("counts,N,K,seed", _grouped_cases(12, 7))
def test_grouped_shape_sweep(counts, N, K, seed):
    if sum(counts) == 0:
        counts = counts[:-1] + (1,)
    say("grouped sweep counts=%s N=%d K=%d" % (list(counts), N, K))
    grouped_case(list(counts), N=N, K=K, seed=seed % 100000, what="grouped sweep")


def _col_shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 9)),
             bool(rng.integers(2)), int(rng.integers(1 << 30))) for _ in range(n)]


@pytest.mark.parametrize("F,N,Tk,pow2,seed", _col_shapes(6, 11))
def test_column_scale_shape_sweep(F, N, Tk, pow2, seed):
    """Wgrad form: dW[F][N] = X^T dY over Tk tokens, both operands in 128x1
    tiles along the tokens (requantized from 1x128), f32 and bf16 out."""
    rule = oracle.SCALE_POW2 if pow2 else oracle.SCALE_AMAX
    x = rand_bits(Tk, F, seed=seed, outliers=0.01, mult=20)
    dy = rand_bits(Tk, N, seed=seed + 1)
    qx, sx = T.requantize_128x1(*T.quantize_1x128(bf16_dev(x)), pow2=pow2)
    qd, sd = T.requantize_128x1(*T.quantize_1x128(bf16_dev(dy)), pow2=pow2)
    qx1, sx1 = oracle.quantize_1x128(f32(x))
    qd1, sd1 = oracle.quantize_1x128(f32(dy))
    qxo, sxo = oracle.requantize_128x1(qx1, sx1, rule)
    qdo, sdo = oracle.requantize_128x1(qd1, sd1, rule)
    assert np.array_equal(host(qx), qxo.T) and np.array_equal(host(sx), sxo.T)
    assert np.array_equal(host(qd), qdo.T) and np.array_equal(host(sd), sdo.T)
    ref = oracle.wgrad(qxo, sxo, qdo, sdo)
    c32 = host(T.gemm(qx, sx, qd, sd, out_dtype=torch.float32, col_scales=True))
    c16 = host(T.gemm(qx, sx, qd, sd, out_dtype=torch.bfloat16, col_scales=True))
    check_gemm(c32, ref, "column-scale sweep F=%d N=%d T=%d" % (F, N, Tk))
    check_bf16_output(c16, c32, ref)
