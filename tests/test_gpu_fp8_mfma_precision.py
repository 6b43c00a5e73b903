"""What gfx950's FP8 matrix instructions do to a K group's partial sum,
shown through the C ABI: the reason the default GEMM path multiplies on the
BF16 matrix cores (after an exact FP8 -> BF16 conversion) instead of the FP8
ones.

The pages describe Hopper FP8 tensor cores that align the products of an
instruction to the largest exponent and keep only about 14 bits, and the fix
of promoting partial sums to FP32 every 128 elements of K ([hearaon]
accumulation-precision paragraph; [thedaegu] Figure 7(b) passage).  gfx950's
FP8 MFMA has the same kind of limit, but inside every group of 8 consecutive
K products of one instruction: a product 2^-6 next to a product 448 in the
same 8-group is cut off before anything reaches the FP32 accumulator, so no
promotion interval can recover it.  The BF16 MFMA forms every product of two
E4M3 values exactly and adds in FP32, so the default path keeps it.

Operands (scales 1.0; all products exact):
  rows 0..127:   A[r][0] = 448 (E4M3 0x7E); for r >= 1 also A[r][r] = 2^-6
                 (0x08); B = 1.0 (0x38) everywhere.  Row r sums 448 + 2^-6,
                 with the small product at K offset r.
  rows 128..143: A[r][8g] = 448, A[r][8g + 1] = 2^-6 with g = r - 128: the
                 pair in each of the 16 8-groups of the first 128 K.
The exact value 448 + 2^-6 = 448.015625 is an FP32 value (ulp 2^-15 at 448).
"""

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_x1_amd import binding as B
from gpu_util import DEV, host, say

pytestmark = pytest.mark.gpu

BIG, SMALL, ONE = 0x7E, 0x08, 0x38
M, K = 144, 128


def operands(N):
    a = np.zeros((M, K), np.uint8)
    a[:128, 0] = BIG
    for r in range(1, 128):
        a[r, r] = SMALL
    for g in range(16):
        a[128 + g, 8 * g] = BIG
        a[128 + g, 8 * g + 1] = SMALL
    b = np.full((K, N), ONE, np.uint8)                 # logical [K][N]
    return a, b


def run(N, flags, per_tensor=False):
    a, b = operands(N)
    qa = torch.from_numpy(a).to(DEV)
    qb = torch.from_numpy(np.ascontiguousarray(b.T)).to(DEV)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    one = torch.ones(max(M, N), dtype=torch.float32, device=DEV)
    if per_tensor:
        sa_ms = sa_ks = sb_ns = sb_ks = 0
    else:
        sa_ms, sa_ks, sb_ns, sb_ks = 1, M, 1, N // 128
    B.fp8_gemm_blockscaled(M, N, K, qa, K, one, sa_ms, sa_ks, qb, K, one, sb_ns, sb_ks,
                           B.FP8FG_BSCALE_BLOCK128, c, B.FP8FG_F32, N, flags)
    torch.cuda.synchronize()
    return host(c).astype(np.float64)


def expected(N):
    a, b = operands(N)
    ref = oracle.gemm_blockscaled(a, np.ones((M, 1)), b, np.ones((1, N // 128)))
    assert ref[0, 0] == 448.0 and np.all(ref[1:] == 448.015625)
    return ref


PATHS = [
    ("default, 256x256 tiles", 256, B.FP8FG_GEMM_DEFAULT | B.FP8FG_GEMM_TILES_WIDE, False),
    ("default, 64x128 tiles", 256, B.FP8FG_GEMM_DEFAULT | B.FP8FG_GEMM_TILES_NARROW, False),
    ("default, N = 128", 128, B.FP8FG_GEMM_DEFAULT, False),
    ("FP8_MFMA", 256, B.FP8FG_GEMM_FP8_MFMA, False),
    ("E8M0_SCALES, 256-column tiles", 256, B.FP8FG_GEMM_E8M0_SCALES, False),
    ("E8M0_SCALES, 128-column tiles", 128, B.FP8FG_GEMM_E8M0_SCALES, False),
    ("NO_PROMOTION (per-tensor)", 256, B.FP8FG_GEMM_NO_PROMOTION, True),
]


@pytest.mark.parametrize("what,N,flags,per_tensor", PATHS, ids=[p[0] for p in PATHS])
def test_small_product_beside_448_in_one_8_group(what, N, flags, per_tensor):
    ref = expected(N)
    c = run(N, flags, per_tensor)
    assert np.all(c == c[:, :1]), what                    # every column alike
    kept = c[:, 0] == ref[:, 0]
    dropped = c[:, 0] == 448.0
    assert np.all(kept | dropped), (what, c[~(kept | dropped), 0])
    lost = sorted(int(r) for r in np.nonzero(dropped[1:128])[0] + 1)
    lost_groups = sorted(int(r) - 128 for r in np.nonzero(dropped[128:])[0] + 128)
    say("%s: 2^-6 beside 448 lost at K offsets %s; in 8-groups %s" % (what, lost, lost_groups))
    assert c[0, 0] == 448.0
    if flags & (B.FP8FG_GEMM_FP8_MFMA | B.FP8FG_GEMM_E8M0_SCALES | B.FP8FG_GEMM_NO_PROMOTION):
        # lost exactly when it shares the 8-group of the large product ...
        assert lost == list(range(1, 8)), (what, lost)
        # ... in every 8-group of the K range
        assert lost_groups == list(range(16)), (what, lost_groups)
    else:
        # exact products, FP32 sums: nothing lost anywhere
        assert np.array_equal(c, ref), what
