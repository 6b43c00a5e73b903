"""Writes tests/golden/workload1.json: SHA-256 digests of the tiny
workload's inputs and of the oracle's outputs for it, plus the MoE token
counts.  Calls only the input generators and oracle/.

Run from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from fp8_fine_grained_x1_amd import workloads  # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def golden():
    w = workloads.workload_inputs(1)
    a = oracle.bf16_bits_to_f32(w["A"])
    b = oracle.bf16_bits_to_f32(w["B"])
    qa, sa = oracle.quantize_1x128(a)
    qb, sb = oracle.quantize_128x128(b)
    c = oracle.gemm_blockscaled(qa, sa, qb, sb)
    return {
        "source": "tests/golden/make_golden.py (input generators + oracle only)",
        "A_bf16": sha(w["A"]), "B_bf16": sha(w["B"]),
        "qa": sha(qa), "sa": sha(sa), "qb": sha(qb), "sb": sha(sb),
        "C_bf16": sha(oracle.bf16_rne_bits(c)),
        "moe_counts": [int(x) for x in workloads.moe_token_counts(4)],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload1.json")
    with open(out, "w") as f:
        json.dump(golden(), f, indent=1)
        f.write("\n")
    print(open(out).read())
