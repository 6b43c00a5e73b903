"""The seeded input generators (CPU only): determinism, the outlier recipe,
the MoE token counts and bf16 rounding."""

import json
import os

import numpy as np
import torch

from fp8_fine_grained_x1_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload1.json")


def test_workload1_matches_recorded_digests():
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    g = json.load(open(GOLDEN))
    now = make_golden.golden()
    for k in ("A_bf16", "B_bf16", "qa", "sa", "qb", "sb", "C_bf16", "moe_counts"):
        assert now[k] == g[k], k


def test_determinism_and_shapes():
    a1 = workloads.workload_inputs(1)
    a2 = workloads.workload_inputs(1)
    assert np.array_equal(a1["A"], a2["A"]) and np.array_equal(a1["B"], a2["B"])
    assert a1["A"].shape == (128, 512) and a1["B"].shape == (512, 256)
    assert a1["A"].dtype == np.uint16


def test_outlier_recipe():
    spec = workloads.WORKLOADS[1]["a"]
    base = workloads.draw_f32((128, 512), dict(spec, outlier_frac=0.0), 0)
    with_out = workloads.draw_f32((128, 512), spec, 0, 2)
    changed = np.flatnonzero(base.ravel() != with_out.ravel())
    assert len(changed) == round(0.01 * 128 * 512) == 655
    assert np.allclose(with_out.ravel()[changed], base.ravel()[changed] * 50)


def test_moe_counts():
    c = workloads.moe_token_counts(4)
    assert c.sum() == 16384 and len(c) == 8
    assert np.all(np.diff(c) <= 0)            # Zipf(1.2) ranks, expert 0 largest
    p = np.arange(1, 9) ** -1.2
    p /= p.sum()
    assert np.all(np.abs(c - 16384 * p) < 6 * np.sqrt(16384 * p))
    off = workloads.moe_offsets(c)
    assert off[0] == 0 and off[-1] == 16384


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(x), ref)
