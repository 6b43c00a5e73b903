"""Parity past 32-bit offsets: tensors of more than 4 GiB, where tile bases,
row index times pitch and output offsets need 64 bits.  Inputs are drawn
on the device from seeded generators; sampled rows, columns and blocks
(always including the last ones and ones past the 4 GiB mark) are compared
with the oracle, bit for bit for the quantizers and to the GEMM tolerance
for the GEMMs."""

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_x1_amd import tensors as T
from gpu_util import DEV, check_bf16_output, check_gemm, f32, host, say

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _gen(seed):
    return torch.Generator(device=DEV).manual_seed(seed)


def _bf16(rows, cols, seed, scale=1.0):
    x = torch.randn(rows, cols, device=DEV, generator=_gen(seed))
    x.mul_(scale)
    return x.to(torch.bfloat16)


def _codes(shape, seed):
    """Uniformly random E4M3 codes without the two NaN codes."""
    q = torch.randint(0, 256, shape, dtype=torch.uint8, device=DEV, generator=_gen(seed))
    q.sub_(((q & 0x7F) == 0x7F).to(torch.uint8))
    return q


def _rows_past(nrows, row_bytes, seed, n=12):
    """Sampled row indices: the first, the last, the first row that starts
    past 4 GiB and random ones on both sides of it."""
    first_high = -(-GIB4 // row_bytes)
    assert first_high < nrows
    rng = np.random.default_rng(seed)
    pick = {0, nrows - 1, first_high, first_high - 1}
    pick |= set(rng.integers(0, first_high, n // 2).tolist())
    pick |= set(rng.integers(first_high, nrows, n // 2).tolist())
    return np.array(sorted(pick))


def _bits(t):
    return host(t.contiguous())


def test_1x128_input_past_4gib():
    rows, cols = 278528, 8192   # 4.25 GiB of bf16
    x = _bf16(rows, cols, seed=1)
    q, s = T.quantize_1x128(x)
    torch.cuda.synchronize()
    r = _rows_past(rows, cols * 2, seed=2)
    say("1x128 %dx%d, rows %s" % (rows, cols, r.tolist()))
    idx = torch.from_numpy(r).to(DEV)
    xb = _bits(x.index_select(0, idx))
    qo, so = oracle.quantize_1x128(f32(xb))
    assert np.array_equal(host(q.index_select(0, idx)), qo)
    assert np.array_equal(host(s.index_select(0, idx)), so)


def test_128x1_input_and_output_past_32_bits():
    rows, cols = 557056, 4096   # input 4.25 GiB; output offsets up to 2^31.1
    x = _bf16(rows, cols, seed=3)
    qt, st = T.quantize_128x1(x)
    torch.cuda.synchronize()
    groups = sorted({0, rows // 128 - 1, (GIB4 // (cols * 2)) // 128, 2000})
    say("128x1 %dx%d, row groups %s" % (rows, cols, groups))
    for g in groups:
        blk = _bits(x[g * 128:(g + 1) * 128])
        qo, so = oracle.quantize_128x1(f32(blk))
        assert np.array_equal(host(qt[:, g * 128:(g + 1) * 128]), qo.T), g
        assert np.array_equal(host(st[:, g]), so[0]), g


def test_128x128_input_and_output_past_4gib():
    K, N = 16384, 147456        # 4.5 GiB of bf16 weights, 2.25 GiB of E4M3
    w = _bf16(K, N, seed=4, scale=0.02)
    q, s = T.quantize_block(w)
    torch.cuda.synchronize()
    nbk, nbn = K // 128, N // 128
    blocks = sorted({(0, 0), (nbk - 1, nbn - 1), (nbk - 1, 0), (0, nbn - 1), (77, 1000), (120, 1100)})
    say("128x128 %dx%d, blocks %s" % (K, N, blocks))
    sh = host(s)
    for bk, bn in blocks:
        blk = _bits(w[bk * 128:(bk + 1) * 128, bn * 128:(bn + 1) * 128])
        qo, so = oracle.quantize_128x128(f32(blk))
        assert sh[bk, bn] == so[0, 0], (bk, bn)
        assert np.array_equal(host(q[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]), qo.T), (bk, bn)


def _operands(M, N, K, seed, G=None):
    qa = _codes((M, K), seed)
    # group-major activation scales [K/128][M], used as a [M][K/128] view
    sa = (torch.rand(K // 128, M, device=DEV, generator=_gen(seed + 1)) * 0.01 + 1e-3).t()
    bshape = (N, K) if G is None else (G, N, K)
    qb = _codes(bshape, seed + 2)
    sshape = (K // 128, N // 128) if G is None else (G, K // 128, N // 128)
    sb = torch.rand(*sshape, device=DEV, generator=_gen(seed + 3)) * 0.01 + 1e-3
    return qa, sa, qb, sb


def test_gemm_a_past_4gib():
    M, N, K = 532480, 256, 8192  # A is 4.06 GiB of E4M3
    qa, sa, qb, sb = _operands(M, N, K, seed=10)
    c32 = T.gemm(qa, sa, qb, sb, out_dtype=torch.float32)
    c16 = T.gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    r = _rows_past(M, K, seed=11)
    say("dense GEMM %dx%dx%d, rows %s" % (M, N, K, r.tolist()))
    idx = torch.from_numpy(r).to(DEV)
    ref = oracle.gemm_blockscaled(host(qa.index_select(0, idx)), host(sa.index_select(0, idx)),
                                  host(qb).T, host(sb))
    h32 = host(c32.index_select(0, idx))
    check_gemm(h32, ref, "dense past 4 GiB")
    check_bf16_output(host(c16.index_select(0, idx)), h32, ref)


def test_grouped_gemm_experts_past_4gib():
    # three experts, the last one starting past the 4 GiB mark of A
    M, N, K, G = 532480, 256, 8192, 3
    offsets = [0, 100000, 530000, M]
    qa, sa, qb, sb = _operands(M, N, K, seed=20, G=G)
    off = torch.tensor(offsets, dtype=torch.int32, device=DEV)
    c32 = T.grouped_gemm(qa, sa, off, qb, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = np.array(sorted(set(_rows_past(M, K, seed=21).tolist()) | {99999, 100000, 529999, 530000}))
    say("grouped GEMM G=%d, rows %s" % (G, r.tolist()))
    idx = torch.from_numpy(r).to(DEV)
    qar, sar, h32 = host(qa.index_select(0, idx)), host(sa.index_select(0, idx)), host(c32.index_select(0, idx))
    qbh, sbh = host(qb), host(sb)
    e_of = np.searchsorted(np.array(offsets), r, side="right") - 1
    for e in range(G):
        m = e_of == e
        ref = oracle.gemm_blockscaled(qar[m], sar[m], qbh[e].T, sbh[e])
        check_gemm(h32[m], ref, "grouped past 4 GiB, expert %d" % e)
