"""GPU parity of the block-scaled GEMMs against the CPU oracle.

The quantized operands are checked bit for bit first; the FP32 result must
satisfy rel_frob <= 1e-5 and max_rel <= 1e-3 (|ref| > 1e-2 rms) against the
oracle's float64 value; the BF16 result must equal RNE of the same kernel's
FP32 result and lie within one bf16 ulp of RNE(oracle).  Full-size
workloads are checked on sampled rows x sampled 128-column blocks that the
oracle computes exactly; the small cases span several tiles and ragged
tails and are checked entirely."""

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_x1_amd import binding as B
from fp8_fine_grained_x1_amd import tensors as T
from fp8_fine_grained_x1_amd import workloads
from gpu_util import (DEV, bf16_dev, check_bf16_output, check_fp8_path, check_gemm, f32, f32_dev,
                      fp8_mfma_bound, host, say, workload)

pytestmark = pytest.mark.gpu


def rand_bits(rows, cols, seed, std=1.0, outliers=0.0, mult=1.0, uniform=False):
    rng = np.random.default_rng(seed)
    if uniform:
        x = (rng.random((rows, cols), dtype=np.float32) * 2 - 1).astype(np.float32)
    else:
        x = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    if outliers:
        x.flat[rng.choice(x.size, size=max(1, int(outliers * x.size)), replace=False)] *= np.float32(mult)
    return workloads.f32_to_bf16_bits(x)


def dense_case(a_bits, b_bits, a_pow2=False, b_pow2=False, what="", scale_layout="group_major"):
    """Quantize on the GPU, check bytes, run both output types, compare."""
    ra = oracle.SCALE_POW2 if a_pow2 else oracle.SCALE_AMAX
    rb = oracle.SCALE_POW2 if b_pow2 else oracle.SCALE_AMAX
    qa, sa = T.quantize_1x128(bf16_dev(a_bits), pow2=a_pow2, scale_layout=scale_layout)
    qb, sb = T.quantize_block(bf16_dev(b_bits), pow2=b_pow2, transpose=True)
    qao, sao = oracle.quantize_1x128(f32(a_bits), ra)
    qbo, sbo = oracle.quantize_128x128(f32(b_bits), rb)
    assert np.array_equal(host(qa), qao) and np.array_equal(host(sa), sao)
    assert np.array_equal(host(qb), qbo.T) and np.array_equal(host(sb), sbo)
    ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
    # both tile shapes of the exact path and the automatic choice, each
    # against the oracle; from N = 256 on they agree bit for bit (at N = 128
    # the 256-row choice promotes separate group sums)
    outs = {}
    for choice in ("wide", "narrow", None):
        h32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, tiles=choice))
        h16 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16, tiles=choice))
        check_gemm(h32, ref, "%s (%s tiles)" % (what, choice or "chosen"))
        check_bf16_output(h16, h32, ref)
        outs[choice] = (h32, h16)
    if qb.shape[0] >= 256:
        for choice in ("narrow", None):
            assert np.array_equal(outs[choice][0], outs["wide"][0]), choice
            assert np.array_equal(outs[choice][1], outs["wide"][1]), choice
    return outs[None][0], ref


@pytest.mark.parametrize("scale_layout", ["group_major", "row_major"])
def test_workload1_full(scale_layout):
    w = workload(1)
    dense_case(w["A"], w["B"], what="workload 1", scale_layout=scale_layout)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (300, 384, 640), (129, 256, 256),
                                   (64, 1024, 1152), (513, 640, 384)])
def test_dense_ragged(M, N, K):
    a = rand_bits(M, K, seed=M + K, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=N + K, std=0.02)
    dense_case(a, b, what="M=%d N=%d K=%d" % (M, N, K))


def test_dense_pow2_both_operands_k128_fidelity():
    # with power-of-two scales and K = 128 the oracle value is exact; the gap is
    # the matrix core's internal summation plus one FP32 promotion
    a = rand_bits(256, 128, seed=1, outliers=0.01, mult=50)
    b = rand_bits(128, 256, seed=2, std=0.02)
    h32, ref = dense_case(a, b, a_pow2=True, b_pow2=True, what="K=128 pow2")
    err = np.abs(h32 - ref) / np.maximum(np.abs(ref), 1e-30)
    say("K=128 pow2: max rel err %.3e (median %.3e)" % (err.max(), np.median(err)))


def test_identity_weights_bit_exact():
    M, K = 200, 384
    a = rand_bits(M, K, seed=4, outliers=0.01, mult=50)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    eye = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    qb, sb = T.quantize_block(eye, pow2=True, transpose=True)
    qao, sao = oracle.quantize_1x128(f32(a))
    expect = (oracle.decode(qao).astype(np.float32) * np.repeat(sao, 128, axis=1)).astype(np.float32)
    for choice in ("wide", "narrow"):
        c32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, tiles=choice))
        assert np.array_equal(c32, expect), choice


def _extreme_rows(M, K, seed):
    """A [M][K] whose rows mix zero groups, groups 1e-25 / 1e-30 below their
    neighbours, rising and falling scales, and rows tiny throughout."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = K // 128
    f = np.ones((M, g), dtype=np.float32)
    f[0:32, 0] = 0.0
    f[32:64, 3] = 0.0
    f[64:96, 2] = 1e-25
    f[96:128, 5] = 1e-30
    f[128:160, :] = np.logspace(-30, 0, g)
    f[160:192, :] = np.logspace(0, -20, g)
    f[192:224, :] = 1e-36
    f[224:256, ::2] = 0.0
    return x * np.repeat(f, 128, axis=1)


def _check_rows(c, ref):
    c = np.asarray(c, np.float64)
    assert np.all(np.isfinite(c))
    for r in range(ref.shape[0]):
        nr = np.linalg.norm(ref[r])
        if nr == 0:
            assert np.all(c[r] == 0), r
            continue
        err = np.linalg.norm(c[r] - ref[r]) / nr
        assert err <= 1e-5, (r, err)


@pytest.mark.parametrize("N", [512, 384])
def test_extreme_group_scales_per_row(N):
    """Every row must match the oracle to 1e-5 relative to its own norm,
    however its group scales vary (N = 512 runs the 256-column kernel,
    N = 384 the 128-column one)."""
    M, K = 256, 1024
    x = _extreme_rows(M, K, 31)
    w = (np.random.default_rng(32).standard_normal((K, N)) * 0.02).astype(np.float32)
    qa, sa = T.quantize_1x128(f32_dev(x))
    qb, sb = T.quantize_block(f32_dev(w))
    qao, sao = oracle.quantize_1x128(x)
    qbo, sbo = oracle.quantize_128x128(w)
    assert np.array_equal(host(qa), qao) and np.array_equal(host(sa), sao)
    c = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, tiles="wide"))
    _check_rows(c, oracle.gemm_blockscaled(qao, sao, qbo, sbo))


def test_extreme_group_scales_per_row_streaming():
    """The same rows through the weight-streaming kernel (dense calls of at
    most 64 rows), on 256- and 128-column tiles."""
    M, K = 256, 1024
    x = _extreme_rows(M, K, 35)
    qa, sa = T.quantize_1x128(f32_dev(x))
    qao, sao = oracle.quantize_1x128(x)
    for N in (512, 384):
        w = (np.random.default_rng(36 + N).standard_normal((K, N)) * 0.02).astype(np.float32)
        qb, sb = T.quantize_block(f32_dev(w))
        qbo, sbo = oracle.quantize_128x128(w)
        for r0 in range(0, M, 64):
            c = host(T.gemm(qa[r0:r0 + 64], sa[r0:r0 + 64], qb, sb, out_dtype=torch.float32))
            _check_rows(c, oracle.gemm_blockscaled(qao[r0:r0 + 64], sao[r0:r0 + 64], qbo, sbo))


def test_extreme_group_scales_per_row_column_scales():
    """The same rows through the per-column-scale (wgrad) layout."""
    M, K, N = 256, 1024, 256
    a = _extreme_rows(M, K, 33)
    x = np.ascontiguousarray(a.T)                     # X [T=K][F=M]
    dy = np.random.default_rng(34).standard_normal((K, N)).astype(np.float32)
    qx, sx = T.quantize_128x1(f32_dev(x))
    qd, sd = T.quantize_128x1(f32_dev(dy))
    qxo, sxo = oracle.quantize_128x1(x)
    qdo, sdo = oracle.quantize_128x1(dy)
    assert np.array_equal(host(qx), qxo.T) and np.array_equal(host(sx), sxo.T)
    c = host(T.gemm(qx, sx, qd, sd, out_dtype=torch.float32, col_scales=True))
    _check_rows(c, oracle.wgrad(qxo, sxo, qdo, sdo))


def test_strided_output_and_guard_bands():
    M, N, K = 130, 256, 384
    a = rand_bits(M, K, seed=8)
    b = rand_bits(K, N, seed=9, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    qb, sb = T.quantize_block(bf16_dev(b))
    for choice in ("wide", "narrow"):
        strided_output_case(qa, sa, qb, sb, a, b, M, N, choice)


def strided_output_case(qa, sa, qb, sb, a, b, M, N, choice):
    cbuf = torch.full((M + 2, N + 64), 12345.0, dtype=torch.float32, device=DEV)
    c = cbuf[1:M + 1, 32:32 + N]
    T.gemm(qa, sa, qb, sb, out=c, tiles=choice)
    hb = host(cbuf)
    mask = np.ones_like(hb, dtype=bool)
    mask[1:M + 1, 32:32 + N] = False
    assert np.all(hb[mask] == 12345.0)
    ref = oracle.gemm_blockscaled(*oracle.quantize_1x128(f32(a)), *oracle.quantize_128x128(f32(b)))
    check_gemm(hb[1:M + 1, 32:32 + N], ref, "strided, %s tiles" % choice)


def unaligned_out(run, M, N, dt):
    """run(out) into an [M][N + 1] buffer (odd row pitch: the kernels' scalar
    store path) and into a contiguous [M][N] one (vector stores): the same
    values bit for bit, and the extra column untouched."""
    buf = torch.full((M, N + 1), 7.0, dtype=dt, device=DEV)
    run(buf[:, :N])
    dense = torch.empty((M, N), dtype=dt, device=DEV)
    run(dense)
    hb = host(buf)
    assert np.array_equal(hb[:, :N], host(dense))
    assert np.array_equal(hb[:, N], host(torch.full((M,), 7.0, dtype=dt, device=DEV)))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_unaligned_output_rows_every_kernel(dt):
    # every GEMM kernel picks its store width from the output's alignment
    # once per tile; this drives the unaligned (scalar) stores of each one
    M, N, K = 130, 256, 384
    a = rand_bits(M, K, seed=91)
    b = rand_bits(K, N, seed=92, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    qb, sb = T.quantize_block(bf16_dev(b))
    for choice in ("wide", "narrow"):
        unaligned_out(lambda o: T.gemm(qa, sa, qb, sb, out=o, tiles=choice), M, N, dt)
    pa, psa = T.quantize_1x128(bf16_dev(a), pow2=True)
    pb, psb = T.quantize_block(bf16_dev(b), pow2=True)
    unaligned_out(lambda o: T.gemm(pa, psa, pb, psb, out=o, e8m0_scales=True), M, N, dt)
    unaligned_out(lambda o: T.gemm(qa, sa, qb, sb, out=o, fp8_mfma=True), M, N, dt)
    # column scales (the wgrad layout)
    x = rand_bits(K, M + 126, seed=93)
    dy = rand_bits(K, N, seed=94)
    qx, sx = T.quantize_128x1(bf16_dev(x))
    qd, sd = T.quantize_128x1(bf16_dev(dy))
    unaligned_out(lambda o: T.gemm(qx, sx, qd, sd, out=o, col_scales=True), M + 126, N, dt)
    # grouped: 256-row tiles, 128-row expert tails and an empty expert
    counts = np.array([300, 0, 129, 37])
    offs = torch.from_numpy(workloads.moe_offsets(counts).astype(np.int32)).to(DEV)
    G, Mg = len(counts), int(counts.sum())
    ag = rand_bits(Mg, K, seed=95)
    qg, sg = T.quantize_1x128(bf16_dev(ag), pow2=True)
    qbg = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    sbg = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        q, s_ = T.quantize_block(bf16_dev(rand_bits(K, N, seed=96 + e, std=0.02)))
        qbg[e].copy_(q)
        sbg[e].copy_(s_)
    for choice in ("wide", "narrow"):
        unaligned_out(lambda o: T.grouped_gemm(qg, sg, offs, qbg, sbg, out=o, tiles=choice), Mg, N, dt)


@pytest.mark.parametrize("M,N,K", [(256, 128, 256), (384, 512, 640)])
def test_column_scales(M, N, K):
    # Wgrad layout: both operands 128x1-quantized along K (the token axis)
    x = rand_bits(K, M, seed=M + 1)        # X [T=K][F=M]
    dy = rand_bits(K, N, seed=N + 2)       # dY [T=K][N]
    qx, sx = T.quantize_128x1(bf16_dev(x))      # [M][K], [M][K/128]
    qd, sd = T.quantize_128x1(bf16_dev(dy))     # [N][K], [N][K/128]
    c32 = host(T.gemm(qx, sx, qd, sd, out_dtype=torch.float32, col_scales=True))
    qxo, sxo = oracle.quantize_128x1(f32(x))
    qdo, sdo = oracle.quantize_128x1(f32(dy))
    assert np.array_equal(host(qx), qxo.T) and np.array_equal(host(sd), sdo.T)
    check_gemm(c32, oracle.wgrad(qxo, sxo, qdo, sdo), "colscale")


def test_no_promotion_per_tensor():
    # the naive baseline: per-tensor scales, whole-K accumulation in the FP8
    # matrix core.  Its error is bounded by the FP8 MFMA's 8-product groups.
    M, N, K = 128, 256, 1024
    a = rand_bits(M, K, seed=21, uniform=True)
    b = rand_bits(K, N, seed=22, uniform=True)
    qao, s_a = oracle.quantize_per_tensor(f32(a))
    qbo, s_b = oracle.quantize_per_tensor(f32(b))
    qa = torch.from_numpy(qao).to(DEV)
    qb = torch.from_numpy(np.ascontiguousarray(qbo.T)).to(DEV)
    sa = torch.tensor([s_a], dtype=torch.float32, device=DEV)
    sb = torch.tensor([s_b], dtype=torch.float32, device=DEV)
    c32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, no_promotion=True)).astype(np.float64)
    ref = oracle.gemm_per_tensor(qao, s_a, qbo, s_b)
    bound = fp8_mfma_bound(qao, s_a, qbo, s_b, promote=False)
    check_fp8_path(c32, ref, bound, "no-promotion")


def test_fp8_mfma_flag_within_group_bound():
    # promoted FP8-MFMA path: each K group's partial sum from the FP8 MFMA
    M, N, K = 64, 256, 640
    a = rand_bits(M, K, seed=23, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=24, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    qb, sb = T.quantize_block(bf16_dev(b))
    c32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, fp8_mfma=True)).astype(np.float64)
    qao, sao = oracle.quantize_1x128(f32(a))
    qbo, sbo = oracle.quantize_128x128(f32(b))
    ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
    bound = fp8_mfma_bound(qao, sao, qbo, np.repeat(sbo, 128, axis=1))
    check_fp8_path(c32, ref, bound, "fp8-mfma promoted")


@pytest.mark.parametrize("N", [128, 384])
def test_e8m0_scales_equal_promoted_fp8_mfma_for_pow2(N):
    """E8M0 path on 128-column tiles (N not a multiple of 256) with
    power-of-two scales: the instruction applies the scales exactly, so the
    result equals the promoted FP8-MFMA path bit for bit (acc + sa sb P
    rounded once either way), and both stay within the FP8 MFMA's
    group-truncation bound of the oracle."""
    M, K = 200, 640
    a = rand_bits(M, K, seed=70, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=71, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a), pow2=True)
    qb, sb = T.quantize_block(bf16_dev(b), pow2=True)
    for dt in (torch.float32, torch.bfloat16):
        mx = T.gemm(qa, sa, qb, sb, out_dtype=dt, e8m0_scales=True)
        pr = T.gemm(qa, sa, qb, sb, out_dtype=dt, fp8_mfma=True)
        assert torch.equal(mx, pr)
    c32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, e8m0_scales=True)).astype(np.float64)
    qao, sao = oracle.quantize_1x128(f32(a), oracle.SCALE_POW2)
    qbo, sbo = oracle.quantize_128x128(f32(b), oracle.SCALE_POW2)
    ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
    bound = fp8_mfma_bound(qao, sao, qbo, np.repeat(sbo, 128, axis=1))
    check_fp8_path(c32, ref, bound, "e8m0 N=%d" % N)


def test_e8m0_scales_any_scale_within_bound():
    """Scales that are not powers of two: the instruction takes their powers
    of two and the rest multiplies the partial sum, so the result is still
    the block-scaled product within the FP8 MFMA bound."""
    M, N, K = 96, 256, 512
    a = rand_bits(M, K, seed=72, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=73, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    qb, sb = T.quantize_block(bf16_dev(b))
    c32 = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, e8m0_scales=True)).astype(np.float64)
    qao, sao = oracle.quantize_1x128(f32(a))
    qbo, sbo = oracle.quantize_128x128(f32(b))
    ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
    bound = fp8_mfma_bound(qao, sao, qbo, np.repeat(sbo, 128, axis=1))
    check_fp8_path(c32, ref, bound, "e8m0 amax scales")


def test_e8m0_scales_column_scales_and_grouped():
    # per-column (wgrad) scales, power of two: equal to the promoted FP8 path
    T_, F, Nn = 512, 256, 384
    x = rand_bits(T_, F, seed=74)
    dy = rand_bits(T_, Nn, seed=75)
    qx, sx = T.quantize_128x1(bf16_dev(x), pow2=True)
    qd, sd = T.quantize_128x1(bf16_dev(dy), pow2=True)
    mx = T.gemm(qx, sx, qd, sd, out_dtype=torch.float32, col_scales=True, e8m0_scales=True)
    pr = T.gemm(qx, sx, qd, sd, out_dtype=torch.float32, col_scales=True, fp8_mfma=True)
    assert torch.equal(mx, pr)
    # grouped, ragged and empty experts, 128-column tiles: equal to the
    # promoted FP8 path
    counts = np.array([0, 37, 300, 1, 0, 129])
    off = workloads.moe_offsets(counts)
    M, N, K = int(counts.sum()), 384, 384
    a = rand_bits(M, K, seed=76)
    qa, sa = T.quantize_1x128(bf16_dev(a), pow2=True)
    qb = torch.empty((len(counts), N, K), dtype=torch.uint8, device=DEV)
    sb = torch.empty((len(counts), K // 128, N // 128), dtype=torch.float32, device=DEV)
    for e in range(len(counts)):
        q, s_ = T.quantize_block(bf16_dev(rand_bits(K, N, seed=77 + e, std=0.02)), pow2=True)
        qb[e].copy_(q)
        sb[e].copy_(s_)
    offs = torch.from_numpy(off.astype(np.int32)).to(DEV)
    gm = T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32, flags=B.FP8FG_GEMM_E8M0_SCALES)
    gp = T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32, flags=B.FP8FG_GEMM_FP8_MFMA)
    assert torch.equal(gm, gp)


def e8m0_wide_check(qao, sao, qbo, sbo, what, offsets=None, qbs=None, sbs=None):
    """E8M0 path on 256-column tiles (N a multiple of 256): FP32 result
    within the FP8 MFMA bound of the oracle for the scales as given, BF16
    result = RNE of the FP32 one.  Operands come from the oracle's arrays."""
    qa = torch.from_numpy(np.ascontiguousarray(qao)).to(DEV)
    sa = f32_dev(sao)
    if offsets is None:
        qb = torch.from_numpy(np.ascontiguousarray(qbo.T)).to(DEV)
        sb = f32_dev(sbo)
        run = lambda dt: T.gemm(qa, sa, qb, sb, out_dtype=dt, e8m0_scales=True)
        ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
        bound = fp8_mfma_bound(qao, sao, qbo, np.repeat(sbo, 128, axis=1))
    else:
        qb = torch.from_numpy(np.stack([np.ascontiguousarray(q.T) for q in qbs])).to(DEV)
        sb = f32_dev(np.stack(sbs))
        offs = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
        run = lambda dt: T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=dt, flags=B.FP8FG_GEMM_E8M0_SCALES)
        ref = oracle.grouped_gemm_blockscaled(qao, sao, offsets, qbs, sbs)
        bound = np.zeros_like(ref)
        for e in range(len(qbs)):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 > r0:
                bound[r0:r1] = fp8_mfma_bound(qao[r0:r1], sao[r0:r1], qbs[e], np.repeat(sbs[e], 128, axis=1))
    c32 = host(run(torch.float32)).astype(np.float64)
    c16 = host(run(torch.bfloat16))
    check_fp8_path(c32, ref, bound, what)
    assert np.array_equal(c16, oracle.bf16_rne_bits(c32.astype(np.float32)))
    return c32


@pytest.mark.parametrize("M,N,K", [(200, 256, 640), (300, 512, 1024), (64, 256, 128)])
def test_e8m0_wide_tiles_pow2_within_bound(M, N, K):
    # an odd number of K groups (the last one alone), an even number, and a
    # single group; ragged row tiles
    a = rand_bits(M, K, seed=80 + M, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=81 + N, std=0.02)
    qao, sao = oracle.quantize_1x128(f32(a), oracle.SCALE_POW2)
    qbo, sbo = oracle.quantize_128x128(f32(b), oracle.SCALE_POW2)
    e8m0_wide_check(qao, sao, qbo, sbo, "e8m0 wide pow2 %dx%dx%d" % (M, N, K))


def test_e8m0_wide_tiles_mixed_scales_within_bound():
    """Power-of-two scales with some made general part way along K: the rows
    of one 32-row tile from group 3 on, one B block's scale in group 5.  The
    waves holding them leave the chained form for the general one at the
    next pair of groups; the others stay chained.  The oracle takes the same
    scales."""
    M, N, K = 256, 512, 1024
    a = rand_bits(M, K, seed=90, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=91, std=0.02)
    qao, sao = oracle.quantize_1x128(f32(a), oracle.SCALE_POW2)
    qbo, sbo = oracle.quantize_128x128(f32(b), oracle.SCALE_POW2)
    sao = sao.astype(np.float32).copy()
    sbo = sbo.astype(np.float32).copy()
    sao[32:64, 3:] *= np.float32(1.5)
    sao[200, 0] *= np.float32(0.75)
    sbo[5, 2] *= np.float32(1.25)
    e8m0_wide_check(qao, sao, qbo, sbo, "e8m0 wide mixed scales")


@pytest.mark.parametrize("M,N,K", [(160, 256, 768), (100, 512, 640), (64, 256, 128)])
def test_e8m0_wide_tiles_amax_scales_within_bound(M, N, K):
    # every group rescales the accumulator: an even and an odd number of K
    # groups, and a single one
    a = rand_bits(M, K, seed=92 + K, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=93 + N, std=0.02)
    qao, sao = oracle.quantize_1x128(f32(a))
    qbo, sbo = oracle.quantize_128x128(f32(b))
    e8m0_wide_check(qao, sao, qbo, sbo, "e8m0 wide amax scales %dx%dx%d" % (M, N, K))


def test_e8m0_wide_tiles_grouped_ragged_and_empty_experts():
    counts = np.array([0, 37, 300, 1, 0, 129, 256])
    off = workloads.moe_offsets(counts)
    M, N, K = int(counts.sum()), 256, 384
    qao, sao = oracle.quantize_1x128(f32(rand_bits(M, K, seed=94)), oracle.SCALE_POW2)
    qbs, sbs = zip(*[oracle.quantize_128x128(f32(rand_bits(K, N, seed=95 + e, std=0.02)), oracle.SCALE_POW2)
                     for e in range(len(counts))])
    e8m0_wide_check(qao, sao, None, None, "e8m0 wide grouped", offsets=off, qbs=qbs, sbs=sbs)


@pytest.mark.parametrize("path", ["wide", "narrow", "n128", "e8m0", "e8m0_n128", "fp8_mfma",
                                  "no_promotion", "col_scales", "grouped"])
def test_empty_contraction_writes_zeros(path):
    """K = 0 (no K groups): every kernel writes C = 0 over the whole output,
    the empty sum of the oracle, and nothing past it."""
    M = 200
    N = 128 if path in ("n128", "e8m0_n128") else 256
    dummy = torch.zeros(64, dtype=torch.uint8, device=DEV)          # operands: never read
    one = torch.ones(1, dtype=torch.float32, device=DEV)            # scales, broadcast
    cbuf = torch.full((M + 1, N), 7.0, dtype=torch.float32, device=DEV)
    c = cbuf[:M]
    flags = {"e8m0": B.FP8FG_GEMM_E8M0_SCALES, "e8m0_n128": B.FP8FG_GEMM_E8M0_SCALES,
             "fp8_mfma": B.FP8FG_GEMM_FP8_MFMA, "no_promotion": B.FP8FG_GEMM_NO_PROMOTION}.get(path, 0)
    mode = B.FP8FG_BSCALE_COL if path == "col_scales" else B.FP8FG_BSCALE_BLOCK128
    flags |= T.tile_flags(path if path in ("wide", "narrow") else None)
    if path == "grouped":
        offs = torch.tensor([0, 0, 150, 150, M], dtype=torch.int32, device=DEV)
        B.fp8_grouped_gemm_blockscaled(4, offs, M, N, 0, dummy, 0, one, 0, 0, dummy, 0, 0, one, 0, 0,
                                       0, c, B.FP8FG_F32, N, flags)
    else:
        B.fp8_gemm_blockscaled(M, N, 0, dummy, 0, one, 0, 0, dummy, 0, one, 0, 0, mode, c,
                               B.FP8FG_F32, N, flags)
    h = host(cbuf)
    ref = oracle.gemm_blockscaled(np.zeros((M, 0), np.uint8), np.zeros((M, 0)), np.zeros((0, N), np.uint8),
                                  np.zeros((0, N // 128)))
    assert np.array_equal(h[:M], ref) and np.all(h[:M] == 0.0)
    assert np.all(h[M] == 7.0)


# ---------------------------------------------------------------- grouped
def grouped_case(counts, N, K, seed, what):
    counts = np.asarray(counts, np.int64)
    G, M = len(counts), int(counts.sum())
    off = workloads.moe_offsets(counts)
    a = rand_bits(M, K, seed=seed)
    ws = [rand_bits(K, N, seed=seed + 1 + e, std=0.02) for e in range(G)]
    qa, sa = T.quantize_1x128(bf16_dev(a), pow2=True)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    sb = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        q, s = T.quantize_block(bf16_dev(ws[e]))
        qb[e].copy_(q)
        sb[e].copy_(s)
    offs = torch.from_numpy(off.astype(np.int32)).to(DEV)
    c32 = host(T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32))
    c16 = host(T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.bfloat16))
    qao, sao = oracle.quantize_1x128(f32(a), oracle.SCALE_POW2)
    qbs, sbs = zip(*[oracle.quantize_128x128(f32(w)) for w in ws])
    ref = oracle.grouped_gemm_blockscaled(qao, sao, off, qbs, sbs)
    check_gemm(c32, ref, what)
    check_bf16_output(c16, c32, ref)
    if N >= 256:
        # both tile shapes of the exact path give the same bits
        for choice in ("wide", "narrow"):
            assert np.array_equal(host(T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32,
                                                      tiles=choice)), c32), choice
    return qa, sa, offs, qb, sb, c32


def test_grouped_ragged_and_empty_experts():
    grouped_case([0, 5, 130, 0, 257, 1, 128], N=256, K=384, seed=30, what="grouped ragged")


@pytest.mark.parametrize("N", [256, 384])
def test_grouped_streaming_ragged_and_empty_experts(N):
    # at most 64 rows per expert on average: the weight-streaming kernel, with
    # experts of 0, 1, 64 (one full tile), 65 and 130 rows (ragged second and
    # third tiles)
    grouped_case([0, 5, 64, 65, 1, 0, 130, 33], N=N, K=640, seed=50, what="grouped streaming N=%d" % N)


@pytest.mark.parametrize("N", [512, 384])
def test_streaming_kernel_bitwise_equals_tiled_kernel(N):
    """Rows computed by the weight-streaming kernel (a dense call of 64 rows,
    a grouped call of 40) equal, bit for bit, the same rows of a 300-row
    dense call on the 256-row tiles."""
    M, K = 300, 768
    a = rand_bits(M, K, seed=60, outliers=0.01, mult=50)
    b = rand_bits(K, N, seed=61, std=0.02)
    qa, sa = T.quantize_1x128(bf16_dev(a))
    qb, sb = T.quantize_block(bf16_dev(b))
    for dt in (torch.float32, torch.bfloat16):
        big = T.gemm(qa, sa, qb, sb, out_dtype=dt, tiles="wide")
        small = T.gemm(qa[100:164], sa[100:164], qb, sb, out_dtype=dt)
        assert torch.equal(big[100:164], small)
        offs = torch.tensor([0, 40], dtype=torch.int32, device=DEV)
        grp = T.grouped_gemm(qa[7:47], sa[7:47], offs, qb.unsqueeze(0), sb.unsqueeze(0), out_dtype=dt)
        assert torch.equal(big[7:47], grp)


def test_grouped_256_experts():
    # a DeepSeek-V3-sized expert count: 2048 tokens over 256 experts (a few
    # rows each, many empty); both tile shapes, every expert's rows checked
    rng = np.random.default_rng(57)
    counts = rng.multinomial(2048, np.full(256, 1 / 256))
    counts[rng.choice(256, 40, replace=False)] = 0
    say("256 experts: %d empty, at most %d rows" % (int(np.sum(counts == 0)), int(counts.max())))
    grouped_case(counts, N=256, K=256, seed=58, what="grouped G=256")


def test_grouped_single_expert_equals_dense():
    qa, sa, offs, qb, sb, c32 = grouped_case([300], N=384, K=512, seed=40, what="grouped G=1")
    dense = host(T.gemm(qa, sa, qb[0], sb[0], out_dtype=torch.float32))
    assert np.array_equal(c32, dense)


def test_grouped_all_rows_in_last_expert():
    grouped_case([0, 0, 0, 200], N=128, K=256, seed=50, what="grouped last")


# ---------------------------------------------------------------- full size
def sample_rows(M, seed, n=40):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(M, size=min(n, M), replace=False).tolist())
    pick |= {0, M - 1, min(127, M - 1), min(128, M - 1)}
    return np.array(sorted(pick))


def sample_blocks(N, seed):
    # first, last and a random 128-column block, plus blocks 31..33: with
    # M = 4096 and N = 7168 the dense kernel switches from 256- to 192-column
    # tiles at column 4096, and block 33 straddles two 192-column tiles
    rng = np.random.default_rng(seed + 1000)
    nb = N // 128
    return sorted({0, nb - 1, int(rng.integers(nb))} | {b for b in (31, 32, 33) if b < nb})


def dense_full_size(w, pow2_a=False):
    d = workload(w)
    a_bits, b_bits = d["A"], d["B"]
    M, K = a_bits.shape
    N = b_bits.shape[1]
    say("workload %d: M=%d N=%d K=%d" % (w, M, N, K))
    qa, sa = T.quantize_1x128(bf16_dev(a_bits), pow2=pow2_a)
    qb, sb = T.quantize_block(bf16_dev(b_bits))
    # the tiles bench.py's launch takes (chosen from the shape) ...
    c32 = T.gemm(qa, sa, qb, sb, out_dtype=torch.float32)
    c16 = T.gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16)
    # ... equal, over the whole output, those of both forced choices
    for choice in ("wide", "narrow"):
        assert torch.equal(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, tiles=choice), c32), choice
    rows = sample_rows(M, w)
    qao, sao = oracle.quantize_1x128(f32(a_bits[rows]))
    idx = torch.from_numpy(rows).to(DEV)
    h32 = host(c32.index_select(0, idx))
    h16 = host(c16.index_select(0, idx))
    for blk in sample_blocks(N, w):
        cols = slice(blk * 128, (blk + 1) * 128)
        qbo, sbo = oracle.quantize_128x128(f32(b_bits[:, cols]))
        ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
        check_gemm(h32[:, cols], ref, "workload %d block %d" % (w, blk))
        check_bf16_output(h16[:, cols], h32[:, cols], ref)
    return qa, sa, qb, sb


def test_workload2_full_size_sampled():
    dense_full_size(2)


@pytest.mark.parametrize("pow2", [True, False], ids=["pow2", "amax"])
def test_workload2_e8m0_full_size_sampled(pow2):
    """The E8M0-scale path at 4096 x 7168 x 7168 in the launch the bench
    times (group-major activation scales, 256 x 256 tiles, bf16 and f32
    out): sampled rows x 128-column blocks against the oracle, held to the
    FP8-path levels and the group-truncation bound."""
    d = workload(2)
    a_bits, b_bits = d["A"], d["B"]
    M, K = a_bits.shape
    N = b_bits.shape[1]
    rule = oracle.SCALE_POW2 if pow2 else oracle.SCALE_AMAX
    qa, sa = T.quantize_1x128(bf16_dev(a_bits), pow2=pow2)
    qb, sb = T.quantize_block(bf16_dev(b_bits), pow2=pow2)
    c32 = T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, e8m0_scales=True)
    c16 = T.gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16, e8m0_scales=True)
    rows = sample_rows(M, 202, n=12)
    idx = torch.from_numpy(rows).to(DEV)
    qao, sao = oracle.quantize_1x128(f32(a_bits[rows]), rule)
    assert np.array_equal(host(qa.index_select(0, idx)), qao)
    h32 = host(c32.index_select(0, idx)).astype(np.float64)
    h16 = host(c16.index_select(0, idx))
    assert np.array_equal(h16, oracle.bf16_rne_bits(h32.astype(np.float32)))
    for blk in sample_blocks(N, 2):
        cols = slice(blk * 128, (blk + 1) * 128)
        qbo, sbo = oracle.quantize_128x128(f32(b_bits[:, cols]), rule)
        ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
        bound = fp8_mfma_bound(qao, sao, qbo, np.repeat(sbo, 128, axis=1))
        check_fp8_path(h32[:, cols], ref, bound, "workload 2 E8M0 %s block %d" % (
            "pow2" if pow2 else "amax", blk))


def test_workload3_full_size_sampled_and_naive_gap():
    """Long K (16384, 128 promotions per output).  Besides the parity of the
    default path, the error gap the pages' accumulation passages are about
    ([why-be] / [thedaegu] "nearly 2%" passages; [hearaon] accumulation
    precision): the naive baseline (per-tensor scales, the whole K summed in
    the FP8 matrix core, no promotion) against the fine-grained path, each
    compared with the exact product of its own E4M3 operands (accumulation
    error alone) and with the unquantized product (accumulation plus
    quantization error)."""
    dense_full_size(3)
    d = workload(3)
    a, b = f32(d["A"]), f32(d["B"])
    rows = sample_rows(a.shape[0], 33, n=24)
    cols = slice(0, 256)
    qao, s_a = oracle.quantize_per_tensor(a)
    qbo, s_b = oracle.quantize_per_tensor(b)
    qa = torch.from_numpy(qao).to(DEV)
    qb = torch.from_numpy(np.ascontiguousarray(qbo.T)).to(DEV)
    sa = torch.tensor([s_a], dtype=torch.float32, device=DEV)
    sb = torch.tensor([s_b], dtype=torch.float32, device=DEV)
    naive = host(T.gemm(qa, sa, qb, sb, out_dtype=torch.float32, no_promotion=True))[rows][:, cols]
    naive = naive.astype(np.float64)
    # the naive path is the FP8 MFMA's whole-K accumulation: within the
    # group-truncation bound on a sub-block (the bound needs every product)
    sub_r, sub_c = rows[:6], slice(0, 64)
    bound = fp8_mfma_bound(qao[sub_r], s_a, qbo[:, sub_c], s_b, promote=False)
    ref_sub = oracle.gemm_per_tensor(qao[sub_r], s_a, qbo[:, sub_c], s_b)
    assert np.all(np.abs(naive[:6, :64] - ref_sub) <= bound)
    naive_own = oracle.gemm_per_tensor(qao[rows], s_a, qbo[:, cols], s_b)
    # the fine-grained path and the exact product of its own operands
    qfa, sfa = T.quantize_1x128(bf16_dev(d["A"]))
    qfb, sfb = T.quantize_block(bf16_dev(d["B"]))
    fine = host(T.gemm(qfa, sfa, qfb, sfb, out_dtype=torch.float32))[rows][:, cols].astype(np.float64)
    qfao, sfao = oracle.quantize_1x128(a[rows])
    qfbo, sfbo = oracle.quantize_128x128(b[:, cols])
    fine_own = oracle.gemm_blockscaled(qfao, sfao, qfbo, sfbo)
    truth = a[rows].astype(np.float64) @ b[:, cols].astype(np.float64)
    acc_naive = oracle.rel_frob(naive, naive_own)
    acc_fine = oracle.rel_frob(fine, fine_own)
    tot_naive = oracle.rel_frob(naive, truth)
    tot_fine = oracle.rel_frob(fine, truth)
    say("K=16384, accumulation error (vs the exact product of the same E4M3 operands): "
        "fine-grained rel_frob=%.3e max_rel=%.3e; naive rel_frob=%.3e max_rel=%.3e" % (
            acc_fine, oracle.max_rel(fine, fine_own), acc_naive, oracle.max_rel(naive, naive_own)))
    say("K=16384, total error (vs the unquantized product): fine-grained rel_frob=%.3e max_rel=%.3e; "
        "naive rel_frob=%.3e max_rel=%.3e" % (tot_fine, oracle.max_rel(fine, truth), tot_naive,
                                             oracle.max_rel(naive, truth)))
    # Promotion of exact partial sums leaves FP32 rounding only; whole-K FP8
    # accumulation adds the instruction's in-group truncation (7.1 times the
    # fine-grained path's error when measured).  Against the unquantized
    # product both are dominated by E4M3 rounding of U(-1,1) operands (about
    # 3.5e-2), where per-tile scales come out slightly ahead of one
    # per-tensor scale (3.51e-2 against 3.58e-2).
    assert acc_fine <= 1e-5
    assert acc_naive >= 3.0 * acc_fine, (acc_naive, acc_fine)
    assert tot_fine <= tot_naive, (tot_fine, tot_naive)
    # context: the same per-tensor operands through the emulated 14-bit
    # tensor-core accumulation the pages describe, on an 8 x 64 sub-block,
    # against the exact product of the same E4M3 operands
    er, ec = rows[:8], slice(0, 64)
    for kk in (4096, 16384):
        qa_k, qb_k = qao[er][:, :kk], qbo[:kk, ec]
        exact = oracle.gemm_per_tensor(qa_k, s_a, qb_k, s_b)
        emu = oracle.gemm_limited_per_tensor(qa_k, s_a, qb_k, s_b)
        say("K=%d per-tensor E4M3, emulated 14-bit accumulation vs exact: rel_frob=%.3e max_rel=%.3e" % (
            kk, oracle.rel_frob(emu, exact), oracle.max_rel(emu, exact)))


def test_workload6_dgrad_full_size_sampled():
    # dX = dY . W^T: dY quantized 1x128 along N (the contraction), W block-
    # quantized without the transpose ([K][N] is K-major for this product:
    # its rows are the output columns), its block scales read transposed
    d = workload(6)
    dy_bits, w_bits = d["dY"], d["W"]
    M, N = dy_bits.shape
    K = w_bits.shape[0]
    say("workload 6: dX[%d][%d] = dY[%d][%d] . W^T, W[%d][%d]" % (M, K, M, N, K, N))
    qd, sd = T.quantize_1x128(bf16_dev(dy_bits))
    qw, sw = T.quantize_block(bf16_dev(w_bits), transpose=False)      # [K][N], [K/128][N/128]
    c32 = T.gemm(qd, sd, qw, sw.t(), out_dtype=torch.float32)           # [M][K]
    c16 = T.gemm(qd, sd, qw, sw.t(), out_dtype=torch.bfloat16)
    rows = sample_rows(M, 6)
    qdo, sdo = oracle.quantize_1x128(f32(dy_bits[rows]))
    idx = torch.from_numpy(rows).to(DEV)
    h32 = host(c32.index_select(0, idx))
    h16 = host(c16.index_select(0, idx))
    for blk in sample_blocks(K, 6):
        cols = slice(blk * 128, (blk + 1) * 128)
        # the oracle's B operand is W^T [N][K]; its 128x128 blocks are those of W
        qbo, sbo = oracle.quantize_128x128(f32(w_bits[cols, :]).T)
        ref = oracle.gemm_blockscaled(qdo, sdo, qbo, sbo)
        check_gemm(h32[:, cols], ref, "workload 6 block %d" % blk)
        check_bf16_output(h16[:, cols], h32[:, cols], ref)


def grouped_full_size(w):
    d = workload(w)
    a_bits, w_bits, counts, off = d["A"], d["W"], d["counts"], d["offsets"]
    G, K, N = w_bits.shape
    M = a_bits.shape[0]
    say("workload %d: G=%d M=%d N=%d K=%d counts=%s" % (w, G, M, N, K, counts.tolist()))
    qa, sa = T.quantize_1x128(bf16_dev(a_bits), pow2=True)
    qb = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    sb = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device=DEV)
    for e in range(G):
        q, s = T.quantize_block(bf16_dev(w_bits[e]))
        qb[e].copy_(q)
        sb[e].copy_(s)
    offs = torch.from_numpy(off.astype(np.int32)).to(DEV)
    c32 = T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32)
    c16 = T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.bfloat16)
    # the other tile shape of the exact path gives the same bits
    other = "narrow" if M > 64 * G else "wide"
    assert torch.equal(T.grouped_gemm(qa, sa, offs, qb, sb, out_dtype=torch.float32, tiles=other), c32)
    rng = np.random.default_rng(44)
    for e in range(G):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        rows = np.array(sorted({r0, r1 - 1} | set(rng.integers(r0, r1, size=6).tolist())))
        idx = torch.from_numpy(rows).to(DEV)
        h32 = host(c32.index_select(0, idx))
        h16 = host(c16.index_select(0, idx))
        qao, sao = oracle.quantize_1x128(f32(a_bits[rows]), oracle.SCALE_POW2)
        for blk in sample_blocks(N, e):
            cols = slice(blk * 128, (blk + 1) * 128)
            qbo, sbo = oracle.quantize_128x128(f32(w_bits[e][:, cols]))
            ref = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
            check_gemm(h32[:, cols], ref, "workload %d expert %d block %d" % (w, e, blk))
            check_bf16_output(h16[:, cols], h32[:, cols], ref)


def test_workload4_grouped_full_size_sampled():
    grouped_full_size(4)


def test_workload7_grouped_down_projection_full_size_sampled():
    grouped_full_size(7)


def test_workload8_grouped_decode_full_size_sampled():
    grouped_full_size(8)


def test_workload5_wgrad_full_size_sampled():
    d = workload(5)
    x_bits, dy_bits = d["X"], d["dY"]
    Tn, Fn = x_bits.shape
    N = dy_bits.shape[1]
    say("workload 5: T=%d F=%d N=%d" % (Tn, Fn, N))
    qx1, sx1 = T.quantize_1x128(bf16_dev(x_bits))
    qd1, sd1 = T.quantize_1x128(bf16_dev(dy_bits))
    qxt, sxt = T.requantize_128x1(qx1, sx1)        # [F][T], [F][T/128]
    qdt, sdt = T.requantize_128x1(qd1, sd1)        # [N][T], [N][T/128]
    dw = T.gemm(qxt, sxt, qdt, sdt, out_dtype=torch.float32, col_scales=True)   # [F][N]
    # oracle: dY fully (its 128x1 tiles span every token), X on sampled slabs
    qd1o, sd1o = oracle.quantize_1x128(f32(dy_bits))
    qdo, sdo = oracle.requantize_128x1(qd1o, sd1o)
    rng = np.random.default_rng(55)
    for slab in sorted({0, Fn // 128 - 1, int(rng.integers(Fn // 128))}):
        fs = slice(slab * 128, (slab + 1) * 128)
        qx1o, sx1o = oracle.quantize_1x128(f32(x_bits[:, fs]))
        qxo, sxo = oracle.requantize_128x1(qx1o, sx1o)
        assert np.array_equal(host(qxt[fs]), qxo.T)
        f_pick = np.array(sorted({0, 127} | set(rng.integers(0, 128, size=10).tolist())))
        ref = oracle.wgrad(qxo[:, f_pick], sxo[:, f_pick], qdo, sdo)
        idx = torch.from_numpy(slab * 128 + f_pick).to(DEV)
        check_gemm(host(dw.index_select(0, idx)), ref, "workload 5 slab %d" % slab)
