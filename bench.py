"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = one pass of the dense forward path over the 4096 x 7168 x 7168
workload (bf16 activations ~N(0,1) with 0.1% x100 outliers, bf16 weights
~N(0, 0.02)):
  1. fp8_quantize_rowtile  -- activations A [4096][7168] -> E4M3 1x128 tiles
                              (scales stored group-major, [K/128][M])
  2. fp8_quantize_block    -- weights B [7168][7168] -> E4M3 128x128 blocks,
                              written transposed (K contiguous)
  3. fp8_gemm_blockscaled  -- C = A . B, FP32 promotion every 128 of K, bf16 out
Inputs are resident in HBM before the timed region; several input/output
sets are rotated so that the 256 MB Infinity Cache cannot hold a step's
working set from one step to the next.

Printed: one JSON line.  `value` is whole-step throughput in GEMM TFLOP/s
(2 M N K per step / wall time per step, quantizers included).  Per-kernel
times come from HIP events recorded on the launch stream around every
launch inside the timed region; `roofline` is the GEMM's (the dominant
kernel): algorithmic 2 M N K flops per GEMM call / its mean time, against
the dense peak of the matrix instruction it runs (BF16: the FP8 operands are
converted exactly to BF16 in registers, because the FP8 matrix instruction
truncates inside its 8-product groups).  On this shape one GEMM call is two
back-to-back launches of the same kernel, on 256- and on 192-column tiles
(4096 and 3072 of the 7168 columns); the events bracket both.
`hbm_copy_context` times a plain 1 GiB device copy in the same run: the HBM
rate a pure stream reaches here, beside which the quantizers' fractions of
the published 8 TB/s are to be read.

    python bench.py [--gpus 1] [--steps 100] [--warmup 200]
    python bench.py --copy-calibration   # plain 1 GiB device copy, for the
                                         # HBM-counter scale factor
    python bench.py --kernel gemm|e8m0   # one GEMM kernel alone on the same
                                         # operands, for counter profiles
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense BF16 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_blockscaled_dense_4096x7168x7168_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_x1_amd", "csrc", "gemm.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # ~80 ms of untimed warmup: the clocks take tens of milliseconds to settle
    # after the setup, and the first steps run up to 12% slower
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--sets", type=int, default=4, help="rotated input/output sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel", choices=["gemm", "e8m0"],
                   help="run only this GEMM on the workload's operands (default path, or the "
                        "E8M0-scale path on power-of-two operands), --steps times after "
                        "--warmup, and print its mean time (for counter profiles)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of 1 GiB (counter calibration)")
    return p.parse_args()


def gemm_source_sha():
    return hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()


def traffic_from_profile():
    """HBM bytes per GEMM call (both launches) from the committed rocprofv3
    PMC summary, or None when absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256") != gemm_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_gemm_call"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(a_bits, b_bits):
    """The oracle on one full step of the same workload (quantization of A
    and B, FP64 block-scaled GEMM, bf16 rounding), timed on the host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    M, K = a_bits.shape
    N = b_bits.shape[1]
    reps = 0
    t0 = time.perf_counter()
    while True:   # whole steps, until about 10 s of CPU work (at most 3)
        qa, sa = oracle.quantize_1x128(oracle.bf16_bits_to_f32(a_bits))
        qb, sb = oracle.quantize_128x128(oracle.bf16_bits_to_f32(b_bits))
        c = oracle.gemm_blockscaled(qa, sa, qb, sb)
        oracle.bf16_rne_bits(c)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps == 3:
            break
    return {
        "value": round(2.0 * M * N * K * reps / dt / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "%d full step(s) (%dx%dx%d): 1x128 quantization of A, 128x128 quantization "
                  "of B, FP64 GEMM with per-group scaling, bf16 rounding; %.1f s in total, "
                  "host %s, %d logical CPUs" % (reps, M, N, K, dt, platform.processor() or
                                                platform.machine(), os.cpu_count() or 0),
    }


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)


def kernel_only(args, M, N, K, st, stream, B):
    """One GEMM kernel alone, repeated: the default path on the step's amax
    operands, or the E8M0-scale path on power-of-two operands."""
    import torch
    G = K // 128
    pow2 = args.kernel == "e8m0"
    rule = B.FP8FG_SCALE_POW2 if pow2 else B.FP8FG_SCALE_AMAX
    B.fp8_quantize_rowtile(st["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128, rule,
                           st["qa"], K, st["sa"], 1, M, stream)
    B.fp8_quantize_block(st["b"], B.FP8FG_BF16, K, N, N, rule, 1, st["qb"], K, st["sb"], N // 128, 1,
                         stream)
    flags = B.FP8FG_GEMM_E8M0_SCALES if pow2 else B.FP8FG_GEMM_DEFAULT

    def gemm():
        B.fp8_gemm_blockscaled(M, N, K, st["qa"], K, st["sa"], 1, M, st["qb"], K, st["sb"], 1,
                               N // 128, B.FP8FG_BSCALE_BLOCK128, st["c"], B.FP8FG_BF16, N, flags,
                               stream)

    for _ in range(args.warmup):
        gemm()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        gemm()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"kernel": args.kernel, "ms": round(ms, 4),
                      "TFLOP/s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the quantizers and GEMMs shard by rows / experts with no exchange).  "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp8_fine_grained_x1_amd import binding, workloads

    binding.lib()   # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = workloads.WORKLOADS[2]
    M, N, K = wl["M"], wl["N"], wl["K"]
    G = K // 128
    d = workloads.workload_inputs(2)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    a0, b0 = to_dev(d["A"]), to_dev(d["B"])
    sets = []
    for i in range(args.sets):
        a = a0 if i == 0 else a0.clone()
        b = b0 if i == 0 else b0.clone()
        sets.append(dict(
            a=a, b=b,
            qa=torch.empty((M, K), dtype=torch.uint8, device=dev),
            sa=torch.empty((G, M), dtype=torch.float32, device=dev),    # group-major
            qb=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sb=torch.empty((G, N // 128), dtype=torch.float32, device=dev),
            c=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)
    B = binding

    if args.kernel:
        kernel_only(args, M, N, K, sets[0], stream, B)
        return

    def step(st, ev=None):
        if ev is not None:
            ev[0].record(stream)
        # sa(m, g) = sa[g * M + m]
        B.fp8_quantize_rowtile(st["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128,
                               B.FP8FG_SCALE_AMAX, st["qa"], K, st["sa"], 1, M, stream)
        if ev is not None:
            ev[1].record(stream)
        B.fp8_quantize_block(st["b"], B.FP8FG_BF16, K, N, N, B.FP8FG_SCALE_AMAX, 1, st["qb"], K,
                             st["sb"], N // 128, 1, stream)
        if ev is not None:
            ev[2].record(stream)
        B.fp8_gemm_blockscaled(M, N, K, st["qa"], K, st["sa"], 1, M, st["qb"], K,
                               st["sb"], 1, N // 128, B.FP8FG_BSCALE_BLOCK128, st["c"],
                               B.FP8FG_BF16, N, B.FP8FG_GEMM_DEFAULT, stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)], events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps

    # Quantizer variants outside the step (same activations): the backward-pass
    # 128x1 requantization of the FP8 activations (output transposed) and the
    # power-of-two 1x128 rule.
    st0 = sets[0]
    q2 = torch.empty((K, M), dtype=torch.uint8, device=dev)
    s2 = torch.empty((M // 128, K), dtype=torch.float32, device=dev)      # group-major
    qp = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sp = torch.empty((G, M), dtype=torch.float32, device=dev)

    def requant():
        B.fp8_quantize_rowtile(st0["qa"], B.FP8FG_E4M3, M, K, K, st0["sa"], 1, M,
                               B.FP8FG_TILE_128x1, B.FP8FG_SCALE_AMAX, q2, M, s2, 1, K, stream)

    def pow2():
        B.fp8_quantize_rowtile(st0["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128,
                               B.FP8FG_SCALE_POW2, qp, K, sp, 1, M, stream)

    def timed(fn, reps=20, warm_s=0.1):
        # After the host-side setup of a workload the GPU has idled for
        # seconds, and its clock needs tens of milliseconds of load to come
        # back: run the call for warm_s of wall time before timing it.
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record(stream)
            fn()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]))

    rq_ms = timed(requant)
    p2_ms = timed(pow2)

    # The E8M0-scale path (FP8 MFMA dequantizing with power-of-two scales) on
    # the same operands quantized with the power-of-two rule.
    qa2 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa2 = torch.empty((G, M), dtype=torch.float32, device=dev)
    qb2 = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sb2 = torch.empty((G, N // 128), dtype=torch.float32, device=dev)
    c2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    B.fp8_quantize_rowtile(st0["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128,
                           B.FP8FG_SCALE_POW2, qa2, K, sa2, 1, M, stream)
    B.fp8_quantize_block(st0["b"], B.FP8FG_BF16, K, N, N, B.FP8FG_SCALE_POW2, 1, qb2, K,
                         sb2, N // 128, 1, stream)

    def e8m0_gemm():
        B.fp8_gemm_blockscaled(M, N, K, qa2, K, sa2, 1, M, qb2, K, sb2, 1, N // 128,
                               B.FP8FG_BSCALE_BLOCK128, c2, B.FP8FG_BF16, N,
                               B.FP8FG_GEMM_E8M0_SCALES, stream)

    mx_ms = timed(e8m0_gemm)
    del qa2, sa2, qb2, sb2, c2

    # The same path on the step's own operands (amax scales, as the workload
    # states): the scales' mantissas are applied in FP32.
    def e8m0_gemm_amax():
        B.fp8_gemm_blockscaled(M, N, K, st0["qa"], K, st0["sa"], 1, M, st0["qb"], K, st0["sb"], 1,
                               N // 128, B.FP8FG_BSCALE_BLOCK128, st0["c"], B.FP8FG_BF16, N,
                               B.FP8FG_GEMM_E8M0_SCALES, stream)

    mxa_ms = timed(e8m0_gemm_amax)

    # Dgrad of a layer of the same shape, dX [M][K] = dY [M][N] . W^T: dY
    # quantized 1x128 along N, W [K][N] block-quantized without the transpose
    # (its rows, the output columns, are then contraction-contiguous).
    d6 = workloads.workload_inputs(6)
    dy6, w6 = to_dev(d6["dY"]), to_dev(d6["W"])
    qdy6 = torch.empty((M, N), dtype=torch.uint8, device=dev)
    sdy6 = torch.empty((N // 128, M), dtype=torch.float32, device=dev)       # group-major
    qw6 = torch.empty((K, N), dtype=torch.uint8, device=dev)
    sw6 = torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev)
    c6 = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    B.fp8_quantize_rowtile(dy6, B.FP8FG_BF16, M, N, N, None, 0, 0, B.FP8FG_TILE_1x128,
                           B.FP8FG_SCALE_AMAX, qdy6, N, sdy6, 1, M, stream)
    B.fp8_quantize_block(w6, B.FP8FG_BF16, K, N, N, B.FP8FG_SCALE_AMAX, 0, qw6, N,
                         sw6, N // 128, 1, stream)
    del dy6, w6

    def dgrad():
        B.fp8_gemm_blockscaled(M, K, N, qdy6, N, sdy6, 1, M, qw6, N, sw6, N // 128, 1,
                               B.FP8FG_BSCALE_BLOCK128, c6, B.FP8FG_BF16, K, B.FP8FG_GEMM_DEFAULT,
                               stream)

    dg_ms = timed(dgrad)
    del qdy6, sdy6, qw6, sw6, c6

    def grouped_setup(w):
        """FP8 operands of a grouped workload: 1x128 power-of-two activation
        scales (group-major), per-expert 128x128 weight blocks, transposed."""
        dw = workloads.workload_inputs(w)
        spec = workloads.WORKLOADS[w]
        Gx, Mx, Nx, Kx = spec["G"], spec["M"], spec["N"], spec["K"]
        ax = to_dev(dw["A"])
        o = dict(G=Gx, M=Mx, N=Nx, K=Kx,
                 qa=torch.empty((Mx, Kx), dtype=torch.uint8, device=dev),
                 sa=torch.empty((Kx // 128, Mx), dtype=torch.float32, device=dev),
                 qb=torch.empty((Gx, Nx, Kx), dtype=torch.uint8, device=dev),
                 sb=torch.empty((Gx, Kx // 128, Nx // 128), dtype=torch.float32, device=dev),
                 c=torch.empty((Mx, Nx), dtype=torch.bfloat16, device=dev),
                 off=torch.from_numpy(dw["offsets"].astype(np.int32)).to(dev),
                 counts=dw["counts"].tolist())
        B.fp8_quantize_rowtile(ax, B.FP8FG_BF16, Mx, Kx, Kx, None, 0, 0, B.FP8FG_TILE_1x128,
                               B.FP8FG_SCALE_POW2, o["qa"], Kx, o["sa"], 1, Mx, stream)
        for e in range(Gx):
            we = to_dev(dw["W"][e])
            B.fp8_quantize_block(we, B.FP8FG_BF16, Kx, Nx, Nx, B.FP8FG_SCALE_AMAX, 1, o["qb"][e], Kx,
                                 o["sb"][e], Nx // 128, 1, stream)
        torch.cuda.synchronize()
        return o

    def grouped(o):
        B.fp8_grouped_gemm_blockscaled(o["G"], o["off"], o["M"], o["N"], o["K"], o["qa"], o["K"],
                                       o["sa"], 1, o["M"], o["qb"], o["K"], o["N"] * o["K"], o["sb"],
                                       1, o["N"] // 128, (o["K"] // 128) * (o["N"] // 128), o["c"],
                                       B.FP8FG_BF16, o["N"], B.FP8FG_GEMM_DEFAULT, stream)

    g4 = grouped_setup(4)
    up_ms = timed(lambda: grouped(g4))
    up_flops = 2.0 * g4["M"] * g4["N"] * g4["K"]
    del g4
    g7 = grouped_setup(7)
    dn_ms = timed(lambda: grouped(g7))
    dn_flops = 2.0 * g7["M"] * g7["N"] * g7["K"]
    del g7
    g8 = grouped_setup(8)
    dc_ms = timed(lambda: grouped(g8))
    dc_flops = 2.0 * g8["M"] * g8["N"] * g8["K"]
    # algorithmic bytes of the decode call: every expert's weights and block
    # scales once, the activations and their scales once, the bf16 output once
    dc_bytes = (g8["G"] * g8["N"] * g8["K"] + g8["G"] * (g8["K"] // 128) * (g8["N"] // 128) * 4
                + g8["M"] * g8["K"] + g8["M"] * (g8["K"] // 128) * 4 + g8["M"] * g8["N"] * 2)
    dc_desc = "G=%d, %d tokens (%d-%d per expert), K=%d -> N=%d" % (
        g8["G"], g8["M"], min(g8["counts"]), max(g8["counts"]), g8["K"], g8["N"])
    del g8
    # Long-K dense GEMM (1024 x 4096 x 16384: 128 promotions per output).
    from fp8_fine_grained_x1_amd import tensors as T
    w3 = workloads.WORKLOADS[3]
    d3 = workloads.workload_inputs(3)
    qa3, sa3 = T.quantize_1x128(to_dev(d3["A"]))
    qb3, sb3 = T.quantize_block(to_dev(d3["B"]))
    c3 = torch.empty((w3["M"], w3["N"]), dtype=torch.bfloat16, device=dev)
    lk_ms = timed(lambda: T.gemm(qa3, sa3, qb3, sb3, out=c3))
    lk_flops = 2.0 * w3["M"] * w3["N"] * w3["K"]
    del d3, qa3, sa3, qb3, sb3, c3
    # Weight gradient dW [F][N] = X^T dY over T = 8192 tokens: X and dY
    # quantized 1x128, requantized to 128x1 tiles (transposed, per-column
    # scales along the token axis), FP32 out.
    w5 = workloads.WORKLOADS[5]
    d5 = workloads.workload_inputs(5)
    qx5, sx5 = T.requantize_128x1(*T.quantize_1x128(to_dev(d5["X"])))
    qd5, sd5 = T.requantize_128x1(*T.quantize_1x128(to_dev(d5["dY"])))
    c5 = torch.empty((w5["F"], w5["N"]), dtype=torch.float32, device=dev)
    wg_ms = timed(lambda: T.gemm(qx5, sx5, qd5, sd5, out=c5, col_scales=True))
    wg_flops = 2.0 * w5["F"] * w5["N"] * w5["T"]
    del d5, qx5, sx5, qd5, sd5, c5

    # Context for the HBM fractions: a plain 1 GiB device-to-device copy (the
    # runtime's copy kernel) in the same run, read + write bytes per time.
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    cp_dst = torch.empty_like(cp_src)
    cp_ms = timed(lambda: cp_dst.copy_(cp_src), reps=10)
    del cp_src, cp_dst

    qa_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    qb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    gemm_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    flops = 2.0 * M * N * K
    # algorithmic bytes: read the bf16 input once, write the e4m3 bytes and the scales once
    bytes_qa = M * K * (2 + 1) + M * G * 4
    bytes_qb = K * N * (2 + 1) + G * (N // 128) * 4
    bytes_rq = M * K * (1 + 1) + M * G * 4 + (M // 128) * K * 4
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    def tflops(nflops, ms):
        return nflops / (ms * 1e-3) / 1e12

    out = {
        "metric": "block-scaled FP8 GEMM TFLOPS (% FP8 MFMA peak); quantize GB/s (% HBM)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 operands, bf16 MFMA (exact conversion), fp32 accumulate",
        "data": "synthetic: seeded bf16 A ~N(0,1) with 0.1% x100 outliers, B ~N(0,0.02)",
        "config": {"workload": "dense forward GEMM 4096x7168x7168, 1x128 activation tiles, "
                               "128x128 weight blocks, bf16 out (quantize A + quantize B + GEMM)",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "kernels": {
            "fp8_quantize_rowtile_1x128": {
                "ms": round(qa_ms, 4), "GB/s": round(gbs(bytes_qa, qa_ms), 1),
                "frac_hbm": round(gbs(bytes_qa, qa_ms) / PEAK_HBM_GBS, 3)},
            "fp8_quantize_block_128x128": {
                "ms": round(qb_ms, 4), "GB/s": round(gbs(bytes_qb, qb_ms), 1),
                "frac_hbm": round(gbs(bytes_qb, qb_ms) / PEAK_HBM_GBS, 3)},
            "fp8_quantize_rowtile_128x1_requant (outside the step)": {
                "ms": round(rq_ms, 4), "GB/s": round(gbs(bytes_rq, rq_ms), 1),
                "frac_hbm": round(gbs(bytes_rq, rq_ms) / PEAK_HBM_GBS, 3)},
            "fp8_quantize_rowtile_1x128_pow2 (outside the step)": {
                "ms": round(p2_ms, 4), "GB/s": round(gbs(bytes_qa, p2_ms), 1),
                "frac_hbm": round(gbs(bytes_qa, p2_ms) / PEAK_HBM_GBS, 3)},
            "fp8_gemm_blockscaled": {
                "ms": round(gemm_ms, 4), "TFLOP/s": round(gemm_tflops, 1),
                "frac_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4)},
            "fp8_gemm_blockscaled E8M0_SCALES (FP8 MFMA dequantizing; pow2 scales), "
            "4096x7168x7168 (outside the step)": {
                "ms": round(mx_ms, 4), "TFLOP/s": round(tflops(flops, mx_ms), 1),
                "frac_fp8_peak": round(tflops(flops, mx_ms) / PEAK_FP8_TFLOPS, 4)},
            "fp8_gemm_blockscaled E8M0_SCALES (FP8 MFMA dequantizing; amax scales, the step's "
            "operands), 4096x7168x7168 (outside the step)": {
                "ms": round(mxa_ms, 4), "TFLOP/s": round(tflops(flops, mxa_ms), 1),
                "frac_fp8_peak": round(tflops(flops, mxa_ms) / PEAK_FP8_TFLOPS, 4)},
            "fp8_gemm_blockscaled dgrad dX = dY.W^T, 4096x7168x7168 (outside the step)": {
                "ms": round(dg_ms, 4), "TFLOP/s": round(tflops(flops, dg_ms), 1),
                "frac_bf16_peak": round(tflops(flops, dg_ms) / PEAK_BF16_TFLOPS, 4)},
            "fp8_gemm_blockscaled long K 1024x4096x16384 (outside the step)": {
                "ms": round(lk_ms, 4), "TFLOP/s": round(tflops(lk_flops, lk_ms), 1),
                "frac_bf16_peak": round(tflops(lk_flops, lk_ms) / PEAK_BF16_TFLOPS, 4)},
            "fp8_gemm_blockscaled wgrad dW = X^T.dY 7168x4096, 8192 tokens, 128x1 column scales, "
            "f32 out (outside the step)": {
                "ms": round(wg_ms, 4), "TFLOP/s": round(tflops(wg_flops, wg_ms), 1),
                "frac_bf16_peak": round(tflops(wg_flops, wg_ms) / PEAK_BF16_TFLOPS, 4)},
            "fp8_grouped_gemm_blockscaled MoE up-projection G=8, 16384 tokens, K=7168 -> N=4096, "
            "pow2 activation scales (outside the step)": {
                "ms": round(up_ms, 4), "TFLOP/s": round(tflops(up_flops, up_ms), 1),
                "frac_bf16_peak": round(tflops(up_flops, up_ms) / PEAK_BF16_TFLOPS, 4)},
            "fp8_grouped_gemm_blockscaled MoE down-projection G=8, 16384 tokens, K=4096 -> N=7168, "
            "pow2 activation scales (outside the step)": {
                "ms": round(dn_ms, 4), "TFLOP/s": round(tflops(dn_flops, dn_ms), 1),
                "frac_bf16_peak": round(tflops(dn_flops, dn_ms) / PEAK_BF16_TFLOPS, 4)},
            "fp8_grouped_gemm_blockscaled MoE decode %s (outside the step)" % dc_desc: {
                "ms": round(dc_ms, 4), "GB/s": round(gbs(dc_bytes, dc_ms), 1),
                "frac_hbm": round(gbs(dc_bytes, dc_ms) / PEAK_HBM_GBS, 3),
                "TFLOP/s": round(tflops(dc_flops, dc_ms), 1)},
        },
        "hbm_copy_context": {
            "1 GiB device copy GB/s (read + write)": round(gbs(2 * (1 << 30), cp_ms), 1),
            "frac_hbm": round(gbs(2 * (1 << 30), cp_ms) / PEAK_HBM_GBS, 3)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile()},
        "context": "the pages report no throughput; their only figure is ~2% max relative error "
                   "of un-promoted FP8 accumulation at K=4096 on Hopper",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d["A"], d["B"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
