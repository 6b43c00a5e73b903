"""Shared plumbing for the GPU parity tests: moving seeded inputs to the
device, caching the large workloads, and the GEMM tolerance check."""

import functools
import os
import sys

import numpy as np
import torch

import oracle
from fp8_fine_grained_x1_amd import workloads

DEV = "cuda:0"

# GEMM tolerances on the FP32 result (relative Frobenius; max relative error
# over entries with |ref| > 1e-2 * rms(ref)).
TOL_FROB = 1e-5
TOL_MAXREL = 1e-3

# The FP8-MFMA paths (flags FP8_MFMA, E8M0_SCALES, NO_PROMOTION) cannot
# meet TOL_FROB: the matrix instruction cuts small products off inside
# 8-product groups (tests/test_gpu_fp8_mfma_precision.py).  They are held to
# the measured level of that loss instead -- across every FP8-path test at
# most rel_frob 6.8e-5, max_rel 2.9e-2, and 0.17 of the per-element
# group-truncation bound (fp8_mfma_bound) -- with some margin.
FP8_PATH_FROB = 1e-4
FP8_PATH_MAXREL = 5e-2
FP8_PATH_BOUND_FRAC = 0.25


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32(bits):
    return oracle.bf16_bits_to_f32(bits)


@functools.lru_cache(maxsize=None)
def workload(w):
    """Host inputs of a workload (generated once per test session)."""
    say("generating workload %d inputs" % w)
    return workloads.workload_inputs(w)


def check_gemm(c32, ref, what=""):
    """Tolerances on an FP32 GEMM result against the oracle's float64 value."""
    c = np.asarray(c32, dtype=np.float64)
    fro = oracle.rel_frob(c, ref)
    mr = oracle.max_rel(c, ref)
    say("%s rel_frob=%.3e max_rel=%.3e" % (what, fro, mr))
    assert fro <= TOL_FROB, (what, fro)
    assert mr <= TOL_MAXREL, (what, mr)
    return fro, mr


def check_fp8_path(c32, ref, bound, what=""):
    """An FP8-MFMA path's FP32 result: every element within half of the
    group-truncation bound, relative Frobenius and max relative error within
    the FP8 path levels.  Returns (rel_frob, max_rel, max err/bound)."""
    c = np.asarray(c32, dtype=np.float64)
    err = np.abs(c - ref)
    frac = float(np.max(err / bound)) if err.size else 0.0
    fro = oracle.rel_frob(c, ref)
    mr = oracle.max_rel(c, ref)
    say("%s rel_frob=%.3e max_rel=%.3e max err/bound=%.3f" % (what, fro, mr, frac))
    assert frac <= FP8_PATH_BOUND_FRAC, (what, frac)
    assert fro <= FP8_PATH_FROB, (what, fro)
    assert mr <= FP8_PATH_MAXREL, (what, mr)
    return fro, mr, frac


def check_bf16_output(c16_bits, c32, ref):
    """BF16 output == RNE of the same kernel's FP32 result, bit for bit, and
    within one bf16 ulp of RNE(oracle) wherever |ref| > 1e-2 * rms(ref) (the
    entries the max-relative criterion covers; tinier entries carry only
    absolute error and may cross zero)."""
    assert np.array_equal(c16_bits, oracle.bf16_rne_bits(np.asarray(c32, np.float32)))
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    mask = np.abs(ref) > 1e-2 * rms
    r16 = oracle.bf16_rne_bits(ref).astype(np.int32)[mask]
    a = c16_bits.astype(np.int32)[mask]
    assert np.all((a >> 15) == (r16 >> 15))
    assert np.all(np.abs(a - r16) <= 1), int(np.sum(np.abs(a - r16) > 1))


def fp8_mfma_bound(qa, sa_rows, qb, sb_cols, promote=True):
    """Error bound for results whose K-group partial sums come from gfx950's
    FP8 MFMA.  That datapath adds each group of 8 consecutive K products
    keeping about 14 bits below the largest of them (measured on the GPU by
    probing single instructions), then accumulates the 8-product sums in
    FP32.  Bound per output element, conservatively:
        sum over groups g of s_g * 2^(floor(log2 max_{k in g} |p_k|) - 9)
        + 2^-20 * sum_k s_k |p_k|
    where p_k = dec(a_k) dec(b_k) and s the scale product of k's K group
    (promote) or the per-tensor scale product (no promotion).
    qa: [M][K] codes, qb: [K][N] codes (logical), sa_rows: [M][K/128] (or a
    scalar), sb_cols: [K/128][N] (or a scalar)."""
    import oracle
    da = np.abs(oracle.decode(qa))
    db = np.abs(oracle.decode(qb))
    M, K = da.shape
    N = db.shape[1]
    prod = da[:, None, :] * db.T[None, :, :]               # [M][N][K]
    if promote:
        s = (np.repeat(np.asarray(sa_rows, np.float64), 128, axis=1)[:, None, :] *
             np.repeat(np.asarray(sb_cols, np.float64), 128, axis=0).T[None, :, :])
    else:
        s = np.float64(sa_rows) * np.float64(sb_cols)
    g = prod.reshape(M, N, K // 8, 8).max(axis=3)
    with np.errstate(divide="ignore"):
        e = np.where(g > 0, np.floor(np.log2(np.where(g > 0, g, 1.0))) - 9, -np.inf)
    sg = s.reshape(M, N, K // 8, 8)[..., 0] if promote else s
    trunc = np.sum(sg * np.exp2(e), axis=2)
    fp32 = 2.0 ** -20 * np.sum(s * prod, axis=2)
    return trunc + fp32
