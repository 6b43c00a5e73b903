"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = one pass of the dense forward path over the 4096 x 7168 x 7168
workload (bf16 activations with 0.1% x100 outliers, bf16 weights ~N(0, 0.02)):
  1. fp8_quantize_rowtile  -- activations A [4096][7168] -> E4M3 1x128 tiles
  2. fp8_quantize_block    -- weights B [7168][7168] -> E4M3 128x128 blocks,
                              written transposed (K contiguous)
  3. fp8_gemm_blockscaled  -- C = A . B, FP32 promotion every 128 of K, bf16 out
Inputs are resident in HBM before the timed region; several input/output
sets are rotated so that the 256 MB Infinity Cache cannot hold a step's
working set from one step to the next.

Printed: one JSON line.  `value` is whole-step throughput in GEMM TFLOP/s
(2 M N K per step / wall time per step, quantizers included); per-kernel
figures come from HIP events recorded on the launch stream around every
launch inside the timed region.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_blockscaled_dense_4096x7168x7168_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_x1_amd", "csrc", "gemm.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="rotated input/output sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=1024)
    p.add_argument("--cpu-cols", type=int, default=2048)
    return p.parse_args()


def gemm_source_sha():
    return hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()


def traffic_from_profile():
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary,
    or None when absent or taken on a different kernel source."""
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
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(a_bits, b_bits, rows, cols):
    """The oracle on a bounded sample: rows x cols of the output with the full
    K, including the quantization of exactly the operand parts it needs."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    K = a_bits.shape[1]
    t0 = time.perf_counter()
    qa, sa = oracle.quantize_1x128(oracle.bf16_bits_to_f32(a_bits[:rows]))
    qb, sb = oracle.quantize_128x128(oracle.bf16_bits_to_f32(b_bits[:, :cols]))
    c = oracle.gemm_blockscaled(qa, sa, qb, sb)
    oracle.bf16_rne_bits(c)
    dt = time.perf_counter() - t0
    return {
        "value": 2.0 * rows * cols * K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "output rows 0..%d x cols 0..%d at K=%d: 1x128 quantization of those A rows, "
                  "128x128 quantization of those B columns, FP64 GEMM, bf16 rounding; %.1f s"
                  % (rows - 1, cols - 1, K, dt),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the quantizers and GEMMs shard by rows / experts with no exchange; "
              "see the design notes).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp8_fine_grained_x1_amd import binding, tensors, workloads

    binding.lib()   # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = workloads.WORKLOADS[2]
    M, N, K = wl["M"], wl["N"], wl["K"]
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
            sa=torch.empty((M, K // 128), dtype=torch.float32, device=dev),
            qb=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sb=torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev),
            c=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream(dev)
    B = binding

    def step(st, ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.fp8_quantize_rowtile(st["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128,
                               B.FP8FG_SCALE_AMAX, st["qa"], K, st["sa"], K // 128, 1, stream)
        if ev is not None:
            ev[1].record(stream)
        B.fp8_quantize_block(st["b"], B.FP8FG_BF16, K, N, N, B.FP8FG_SCALE_AMAX, 1, st["qb"], K,
                             st["sb"], N // 128, 1, stream)
        if ev is not None:
            ev[2].record(stream)
        B.fp8_gemm_blockscaled(M, N, K, st["qa"], K, st["sa"], K // 128, 1, st["qb"], K,
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
    qa_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    qb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    gemm_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    flops = 2.0 * M * N * K
    bytes_qa = M * K * (2 + 1) + M * (K // 128) * 4
    bytes_qb = K * N * (2 + 1) + (K // 128) * (N // 128) * 4
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    traffic = traffic_from_profile()

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
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic: seeded bf16 A ~N(0,1) with 0.1% x100 outliers, B ~N(0,0.02)",
        "config": {"workload": "dense forward GEMM 4096x7168x7168, 1x128 activation tiles, "
                               "128x128 weight blocks, bf16 out",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "kernels": {
            "fp8_quantize_rowtile_1x128": {"ms": round(qa_ms, 4),
                                           "GB/s": round(bytes_qa / (qa_ms * 1e-3) / 1e9, 1),
                                           "frac_hbm": round(bytes_qa / (qa_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)},
            "fp8_quantize_block_128x128": {"ms": round(qb_ms, 4),
                                           "GB/s": round(bytes_qb / (qb_ms * 1e-3) / 1e9, 1),
                                           "frac_hbm": round(bytes_qb / (qb_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)},
            "fp8_gemm_blockscaled": {"ms": round(gemm_ms, 4), "TFLOP/s": round(gemm_tflops, 1),
                                     "frac_mfma": round(gemm_tflops / PEAK_FP8_TFLOPS, 3)},
        },
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic},
        "context": "the pages report no throughput; their only figure is ~2% max relative error "
                   "of un-promoted FP8 accumulation at K=4096 on Hopper",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d["A"], d["B"], args.cpu_rows, args.cpu_cols)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
