"""Error metrics used to compare a GEMM result with the oracle (test
infrastructure only).

rel_frob = ||C - R||_F / ||R||_F.
max_rel  = max |C - R| / |R| over the entries with |R| > 1e-2 * rms(R).
"""

import numpy as np


def rel_frob(c, ref):
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(c - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)


def max_rel(c, ref, floor=1e-2):
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    mask = np.abs(ref) > floor * rms
    if not np.any(mask):
        return 0.0
    return float(np.max(np.abs(c[mask] - ref[mask]) / np.abs(ref[mask])))
