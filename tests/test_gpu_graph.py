"""The hot path under HIP graph capture: quantize A (1x128 tiles), quantize
B (128x128 blocks), the block-scaled GEMM and a grouped GEMM with
device-side expert offsets are captured once and replayed on new inputs.
Nothing in these calls synchronizes with the host or allocates, so every
replay must equal the eager calls on the same inputs bit for bit.  Eager
work and synchronizations run between the replays."""

import numpy as np
import pytest
import torch

from fp8_fine_grained_x1_amd import tensors as T
from fp8_fine_grained_x1_amd import workloads
from gpu_util import DEV, bf16_dev, say

pytestmark = pytest.mark.gpu

M, N, K = 384, 512, 640
COUNTS = np.array([200, 0, 57, 127])   # one 256-row tile, an empty expert, two tails


def bits(rows, cols, seed, std):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols), dtype=np.float32) * std).view(np.uint32) >> 16


def step(x, w, xg, offs, wg):
    qa, sa = T.quantize_1x128(x)
    qb, sb = T.quantize_block(w)
    c = T.gemm(qa, sa, qb, sb)
    qg, sg = T.quantize_1x128(xg, pow2=True)
    qbg = torch.stack([T.quantize_block(wg[e])[0] for e in range(wg.shape[0])])
    sbg = torch.stack([T.quantize_block(wg[e])[1] for e in range(wg.shape[0])])
    cg = T.grouped_gemm(qg, sg, offs, qbg, sbg, out_dtype=torch.float32)
    return c, cg


def test_step_replays_in_a_graph():
    Mg, G = int(COUNTS.sum()), len(COUNTS)
    offs = torch.from_numpy(workloads.moe_offsets(COUNTS).astype(np.int32)).to(DEV)
    x = bf16_dev(bits(M, K, 1, 1.0).astype(np.uint16))
    w = bf16_dev(bits(K, N, 2, 0.02).astype(np.uint16))
    xg = bf16_dev(bits(Mg, K, 3, 1.0).astype(np.uint16))
    wg = torch.stack([bf16_dev(bits(K, N, 4 + e, 0.02).astype(np.uint16)) for e in range(G)])

    side = torch.cuda.Stream()                  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(x, w, xg, offs, wg)                # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        c_g, cg_g = step(x, w, xg, offs, wg)

    for rep in range(4):
        x.copy_(bf16_dev(bits(M, K, 100 + rep, 1.0).astype(np.uint16)))
        w.copy_(bf16_dev(bits(K, N, 200 + rep, 0.02).astype(np.uint16)))
        xg.copy_(bf16_dev(bits(Mg, K, 300 + rep, 1.0).astype(np.uint16)))
        for e in range(G):
            wg[e].copy_(bf16_dev(bits(K, N, 400 + 10 * rep + e, 0.02).astype(np.uint16)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        c_e, cg_e = step(x, w, xg, offs, wg)    # eager, same inputs
        torch.cuda.synchronize()
        say("replay %d: max |c| %.3f" % (rep, float(c_g.float().abs().max())))
        assert torch.equal(c_g, c_e), rep
        assert torch.equal(cg_g, cg_e), rep
        assert float(c_g.float().abs().max()) > 0.0
