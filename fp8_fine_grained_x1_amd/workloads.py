"""Seeded synthetic inputs for the workloads.

This module only draws random numbers and stores them as bf16 bit patterns;
it holds none of the method's arithmetic (no scales, no FP8, no GEMM).  Both
the HIP path (tests, bench) and the CPU oracle take their inputs from here.

Recipe (identical for every consumer):
  * one ``numpy.random.default_rng(seed)`` per tensor role, with
    seed = 100 * (workload - 1) + t, t = 0 for A / X, 1 for B / W / dY,
    2 for the outlier positions, 3 for the MoE token counts;
  * samples are drawn in float32 (normal: ``standard_normal`` * std;
    uniform on (-1, 1): 2 * ``random`` - 1), outliers are applied in float32
    (exactly round(frac * numel) distinct positions, uniform without
    replacement, multiplied by the factor), then each value is rounded to
    bf16 with round-to-nearest-even;
  * MoE token counts: multinomial(total, p_k proportional to k**-1.2,
    k = 1..G), expert 0 taking rank 1 (Zipf workloads), or with equal p_k
    (the decode workload).

Arrays are returned as uint16 bf16 bit patterns, row-major, in the logical
orientation of the problem: A [M][K], B [K][N], W [G][K][N], X [T][F],
dY [T][N] (workload 5) or [M][N] (workload 6).
"""

import numpy as np

# Workload table: what each of the five workloads is.
WORKLOADS = {
    1: dict(name="tiny block-scaled FP8 GEMM",
            M=128, N=256, K=512,
            a=dict(dist="normal", std=1.0, outlier_frac=0.01, outlier_mult=50.0),
            b=dict(dist="normal", std=0.02)),
    2: dict(name="dense forward GEMM",
            M=4096, N=7168, K=7168,
            a=dict(dist="normal", std=1.0, outlier_frac=0.001, outlier_mult=100.0),
            b=dict(dist="normal", std=0.02)),
    3: dict(name="long-K accumulation stress",
            M=1024, N=4096, K=16384,
            a=dict(dist="uniform"), b=dict(dist="uniform")),
    4: dict(name="MoE grouped up-projection",
            M=16384, N=4096, K=7168, G=8, zipf=1.2,
            a=dict(dist="normal", std=1.0),
            b=dict(dist="normal", std=0.02)),
    5: dict(name="backward weight-gradient GEMM",
            T=8192, F=7168, N=4096,
            a=dict(dist="normal", std=1.0),      # X  [T][F]
            b=dict(dist="normal", std=1.0)),     # dY [T][N]
    # dX [M][K] = dY [M][N] . W^T of the dense forward layer's shape
    6: dict(name="backward input-gradient GEMM",
            M=4096, N=7168, K=7168,
            a=dict(dist="normal", std=1.0, outlier_frac=0.001, outlier_mult=100.0),  # dY [M][N]
            b=dict(dist="normal", std=0.02)),                                         # W [K][N]
    7: dict(name="MoE grouped down-projection",
            M=16384, N=7168, K=4096, G=8, zipf=1.2,
            a=dict(dist="normal", std=1.0),
            b=dict(dist="normal", std=0.02)),
    # few tokens per expert: the weights dominate the bytes moved
    8: dict(name="MoE grouped up-projection, decode",
            M=512, N=4096, K=7168, G=16, zipf=None,
            a=dict(dist="normal", std=1.0),
            b=dict(dist="normal", std=0.02)),
}


def seed_for(workload, role):
    """role: 0 = A/X, 1 = B/W/dY, 2 = outlier positions, 3 = token counts."""
    return 100 * (workload - 1) + role


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest-even) and return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def draw_f32(shape, spec, seed, outlier_seed=None):
    """float32 samples for one tensor, outliers applied."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    if spec["dist"] == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        std = np.float32(spec.get("std", 1.0))
        if std != np.float32(1.0):
            x *= std
    elif spec["dist"] == "uniform":
        x = rng.random(n, dtype=np.float32)
        x *= np.float32(2.0)
        x -= np.float32(1.0)
    else:
        raise ValueError(spec["dist"])
    frac = spec.get("outlier_frac", 0.0)
    if frac:
        k = int(round(frac * n))
        orng = np.random.default_rng(outlier_seed)
        pos = orng.choice(n, size=k, replace=False)
        x[pos] *= np.float32(spec["outlier_mult"])
    return x.reshape(shape)


def draw_bf16(shape, spec, seed, outlier_seed=None):
    return f32_to_bf16_bits(draw_f32(shape, spec, seed, outlier_seed))


def moe_token_counts(workload=4):
    w = WORKLOADS[workload]
    G, total, alpha = w["G"], w["M"], w["zipf"]
    if alpha is None:
        p = np.full(G, 1.0 / G)
    else:
        p = np.arange(1, G + 1, dtype=np.float64) ** (-alpha)
        p /= p.sum()
    rng = np.random.default_rng(seed_for(workload, 3))
    return rng.multinomial(total, p).astype(np.int64)


def moe_offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    np.cumsum(counts, out=off[1:])
    return off


def workload_inputs(workload):
    """All inputs of one workload as bf16 bit arrays (dict of numpy arrays)."""
    w = WORKLOADS[workload]
    out = {}
    if workload in (1, 2, 3):
        out["A"] = draw_bf16((w["M"], w["K"]), w["a"], seed_for(workload, 0),
                             seed_for(workload, 2))
        out["B"] = draw_bf16((w["K"], w["N"]), w["b"], seed_for(workload, 1))
    elif workload in (4, 7, 8):
        out["A"] = draw_bf16((w["M"], w["K"]), w["a"], seed_for(workload, 0))
        out["W"] = draw_bf16((w["G"], w["K"], w["N"]), w["b"], seed_for(workload, 1))
        out["counts"] = moe_token_counts(workload)
        out["offsets"] = moe_offsets(out["counts"])
    elif workload == 5:
        out["X"] = draw_bf16((w["T"], w["F"]), w["a"], seed_for(workload, 0))
        out["dY"] = draw_bf16((w["T"], w["N"]), w["b"], seed_for(workload, 1))
    elif workload == 6:
        out["dY"] = draw_bf16((w["M"], w["N"]), w["a"], seed_for(workload, 0),
                              seed_for(workload, 2))
        out["W"] = draw_bf16((w["K"], w["N"]), w["b"], seed_for(workload, 1))
    else:
        raise ValueError(workload)
    return out
