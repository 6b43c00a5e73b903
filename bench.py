"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = one pass of the dense forward path over the 4096 x 7168 x 7168
workload (bf16 activations ~N(0,1) with 0.1% x100 outliers, bf16 weights
~N(0, 0.02)):
  1. fp8_quantize_rowtile  -- activations A [4096][7168] -> E4M3 1x128 tiles
                              (scales stored group-major, [K/128][M])
  2. fp8_quantize_block    -- weights B [7168][7168] -> E4M3 128x128 blocks,
                              written transposed (K contiguous)
  3. fp8_gemm_blockscaled  -- C = A . B, FP32 promotion every 128 of K, bf16 out
Inputs are resident in HBM before the timed region; four input/output sets
(1.2 GB) are rotated so that the 256 MB Infinity Cache cannot hold a step's
working set from one step to the next.  Before the --warmup steps the step
runs for --settle-ms of wall time (reported as clock_settle_ms): after the
host-side setup the GPU has idled, and its clock needs tens of milliseconds
of load to reach its steady state.

Printed: one JSON line.  `value` is whole-step throughput in GEMM TFLOP/s
(2 M N K per step / wall time per step, quantizers included).  Per-kernel
times come from HIP events recorded on the launch stream around every
launch inside the timed region.  `roofline` is the GEMM's (the dominant
kernel): algorithmic 2 M N K flops per GEMM call / its mean time, against
the dense FP8 MFMA peak that the metric names.  The default path runs its
products on the BF16 matrix cores (the FP8 operands are converted exactly
to BF16 in registers, because gfx950's FP8 matrix instruction truncates
inside its 8-product groups), so its ceiling is the BF16 peak, half the FP8
one; `frac_bf16_peak` states the fraction against that ceiling.  On this
shape one GEMM call is two back-to-back launches of the same kernel, on
256- and on 192-column tiles (4096 and 3072 of the 7168 columns); the
events bracket both.

Entries outside the step (other workloads, other scale rules and paths)
each rotate at least 1 GiB of operand and output sets, and run for 100 ms
before 20 timed calls.  The quantizers, in the step and outside it, also
carry a back-to-back figure (one event pair around 40 calls over >= 1 GiB
of rotated sets): an event pair around every launch adds its dispatch gap,
about 3 us, to a kernel of about 20 us.  `hbm_copy_context` times a plain 1 GiB device copy
and torch's own bf16 -> E4M3 cast of the step's activations in the same run:
the HBM rates a pure stream and a stream with the 1x128 quantizer's
read/write mix reach here, beside which the quantizers' fractions of the
published 8 TB/s are to be read;
`vendor_gemm_context` times the vendor library's FP8 GEMM (per-tensor and
row/column scales, no per-K-group promotion) and BF16 GEMM on the dense
forward shape, beside which the GEMM's fraction of the FP8 peak is to be
read.

    python bench.py [--gpus 1] [--steps 100] [--warmup 200] [--settle-ms 500]
    python bench.py --copy-calibration   # plain 1 GiB device copy, for the
                                         # HBM-counter scale factor
    python bench.py --kernel NAME        # one kernel alone on the workload's
                                         # operands, for counter profiles
"""

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense BF16 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
ROTATE_BYTES = 1 << 30       # operand sets rotated by every entry outside the step

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_blockscaled_dense_4096x7168x7168_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_x1_amd", "csrc", "gemm.hip")

KERNELS = ["gemm", "e8m0", "quant1x128", "quant128x128", "requant128x1"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--settle-ms", type=float, default=500.0,
                   help="wall time of steps run before the warmup steps (clock settling)")
    p.add_argument("--sets", type=int, default=4, help="rotated input/output sets of the step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the step (no entries outside it)")
    p.add_argument("--kernel", choices=KERNELS,
                   help="run only this kernel on the workload's operands (the GEMM's default "
                        "path, the E8M0-scale path on power-of-two operands, or one quantizer), "
                        "rotating >= 1 GiB of operand sets, --steps times after --warmup, and "
                        "print its mean time (for counter profiles)")
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


def progress(msg):
    """One line on stderr as each part of the run ends."""
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


def nbytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts)


def n_sets(set_bytes):
    """Operand sets needed to rotate at least 1 GiB."""
    return max(2, math.ceil(ROTATE_BYTES / max(set_bytes, 1)))


def clones(d, n):
    """n sets: d itself and n - 1 deep copies of its tensors."""
    out = [d]
    for _ in range(n - 1):
        out.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in d.items()})
    return out


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
    from fp8_fine_grained_x1_amd import tensors as T

    binding.lib()   # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B = binding

    wl = workloads.WORKLOADS[2]
    M, N, K = wl["M"], wl["N"], wl["K"]
    G = K // 128
    d = workloads.workload_inputs(2)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    a0, b0 = to_dev(d["A"]), to_dev(d["B"])
    stream = torch.cuda.current_stream(dev)

    def new_step_set(a, b):
        return dict(
            a=a, b=b,
            qa=torch.empty((M, K), dtype=torch.uint8, device=dev),
            sa=torch.empty((G, M), dtype=torch.float32, device=dev),    # group-major
            qb=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sb=torch.empty((G, N // 128), dtype=torch.float32, device=dev),
            c=torch.empty((M, N), dtype=torch.bfloat16, device=dev))

    def quant_a(st, rule=B.FP8FG_SCALE_AMAX):
        # sa(m, g) = sa[g * M + m]
        B.fp8_quantize_rowtile(st["a"], B.FP8FG_BF16, M, K, K, None, 0, 0, B.FP8FG_TILE_1x128,
                               rule, st["qa"], K, st["sa"], 1, M, stream)

    def quant_b(st, rule=B.FP8FG_SCALE_AMAX):
        B.fp8_quantize_block(st["b"], B.FP8FG_BF16, K, N, N, rule, 1, st["qb"], K,
                             st["sb"], N // 128, 1, stream)

    def gemm(st, flags=B.FP8FG_GEMM_DEFAULT, c=None):
        B.fp8_gemm_blockscaled(M, N, K, st["qa"], K, st["sa"], 1, M, st["qb"], K,
                               st["sb"], 1, N // 128, B.FP8FG_BSCALE_BLOCK128,
                               st["c"] if c is None else c,
                               B.FP8FG_BF16 if c is None or c.dtype == torch.bfloat16 else B.FP8FG_F32,
                               N, flags, stream)

    def requant(st):
        B.fp8_quantize_rowtile(st["qa"], B.FP8FG_E4M3, M, K, K, st["sa"], 1, M,
                               B.FP8FG_TILE_128x1, B.FP8FG_SCALE_AMAX, st["q2"], M, st["s2"], 1, K,
                               stream)

    def timed_batch(fns, reps=40, warm_s=0.1):
        """Mean time per call of reps back-to-back calls cycling over fns,
        one HIP event pair around the batch: for short kernels, where an
        event pair around every launch adds its dispatch gap."""
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < warm_s:
            for _ in range(8):
                fns[i % len(fns)]()
                i += 1
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fns[r % len(fns)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def timed(fns, reps=20, warm_s=0.1):
        """Mean HIP-event time of one call, cycling over the operand sets of
        fns; the calls first run for warm_s of wall time (clock settling)."""
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < warm_s:
            for _ in range(4):
                fns[i % len(fns)]()
                i += 1
            torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            fns[r % len(fns)]()
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(reps)]))

    if args.kernel:
        kernel_only(args, locals())
        return

    sets = [new_step_set(a0 if i == 0 else a0.clone(), b0 if i == 0 else b0.clone())
            for i in range(args.sets)]

    def step(st, ev=None):
        if ev is not None:
            ev[0].record(stream)
        quant_a(st)
        if ev is not None:
            ev[1].record(stream)
        quant_b(st)
        if ev is not None:
            ev[2].record(stream)
        gemm(st)
        if ev is not None:
            ev[3].record(stream)

    # clock settling, then the warmup steps as given, then the timed steps
    t_settle = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(sets[i % len(sets)])
            i += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
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
    progress("step timed: %.4f ms per step after %.0f ms of clock settling" % (ms_step, settle_ms))

    qa_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    qb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    gemm_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    flops = 2.0 * M * N * K
    # algorithmic bytes: read the bf16 input once, write the e4m3 bytes and the scales once
    bytes_qa = M * K * (2 + 1) + M * G * 4
    bytes_qb = K * N * (2 + 1) + G * (N // 128) * 4
    bytes_rq = M * K * (1 + 1) + M * G * 4 + (M // 128) * K * 4
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12

    def gbs(nb, ms):
        return nb / (ms * 1e-3) / 1e9

    def tflops(nf, ms):
        return nf / (ms * 1e-3) / 1e12

    def q_entry(nb, ms, sets_n, b2b_ms=None):
        e = {"ms": round(ms, 4), "GB/s": round(gbs(nb, ms), 1),
             "frac_hbm": round(gbs(nb, ms) / PEAK_HBM_GBS, 3), "rotated_sets": sets_n}
        if b2b_ms is not None:
            e.update(back_to_back_ms=round(b2b_ms, 4), back_to_back_frac_hbm=round(gbs(nb, b2b_ms) / PEAK_HBM_GBS, 3))
        return e

    def g_entry(nf, ms, sets_n, peak=PEAK_BF16_TFLOPS, **extra):
        e = {"ms": round(ms, 4), "TFLOP/s": round(tflops(nf, ms), 1),
             "frac_fp8_peak": round(tflops(nf, ms) / PEAK_FP8_TFLOPS, 4)}
        if peak == PEAK_BF16_TFLOPS:
            e["frac_bf16_peak"] = round(tflops(nf, ms) / PEAK_BF16_TFLOPS, 4)
        e["rotated_sets"] = sets_n
        e.update(extra)
        return e

    # The step's quantizers again, back to back (one event pair around 40
    # calls, >= 1 GiB of rotated sets): their HIP-event times in the step
    # include the dispatch gap that an event pair around every launch adds.
    qa_sets = clones(dict(a=a0, qa=sets[0]["qa"], sa=sets[0]["sa"]),
                     n_sets(nbytes(a0, sets[0]["qa"], sets[0]["sa"])))
    qa_b2b = timed_batch([lambda s=s: quant_a(s) for s in qa_sets])
    del qa_sets
    qb_sets = clones(dict(b=b0, qb=sets[0]["qb"], sb=sets[0]["sb"]),
                     n_sets(nbytes(b0, sets[0]["qb"], sets[0]["sb"])))
    qb_b2b = timed_batch([lambda s=s: quant_b(s) for s in qb_sets])
    del qb_sets
    progress("step quantizers timed back to back")

    kernels = {
        "fp8_quantize_rowtile_1x128": {
            "ms": round(qa_ms, 4), "GB/s": round(gbs(bytes_qa, qa_ms), 1),
            "frac_hbm": round(gbs(bytes_qa, qa_ms) / PEAK_HBM_GBS, 3),
            "back_to_back_ms": round(qa_b2b, 4),
            "back_to_back_frac_hbm": round(gbs(bytes_qa, qa_b2b) / PEAK_HBM_GBS, 3)},
        "fp8_quantize_block_128x128": {
            "ms": round(qb_ms, 4), "GB/s": round(gbs(bytes_qb, qb_ms), 1),
            "frac_hbm": round(gbs(bytes_qb, qb_ms) / PEAK_HBM_GBS, 3),
            "back_to_back_ms": round(qb_b2b, 4),
            "back_to_back_frac_hbm": round(gbs(bytes_qb, qb_b2b) / PEAK_HBM_GBS, 3)},
        "fp8_gemm_blockscaled": {
            "ms": round(gemm_ms, 4), "TFLOP/s": round(gemm_tflops, 1),
            "frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "frac_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4)},
    }
    extra = {}
    if not args.no_extra:
        extra = outside_step(locals())
        kernels.update(extra.pop("kernels"))

    out = {
        "metric": "block-scaled FP8 GEMM TFLOPS (% FP8 MFMA peak); quantize GB/s (% HBM)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_ms": round(settle_ms, 1),
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 operands, bf16 MFMA (exact conversion), fp32 accumulate",
        "data": "synthetic: seeded bf16 A ~N(0,1) with 0.1% x100 outliers, B ~N(0,0.02)",
        "config": {"workload": "dense forward GEMM 4096x7168x7168, 1x128 activation tiles, "
                               "128x128 weight blocks, bf16 out (quantize A + quantize B + GEMM)",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "kernels": kernels,
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic_from_profile(),
                     "frac_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "ceiling_frac_of_fp8_peak": PEAK_BF16_TFLOPS / PEAK_FP8_TFLOPS,
                     "note": "the default path multiplies on the BF16 matrix cores (exact "
                             "products); traffic is HBM bytes per GEMM call from the committed "
                             "counter profile of the same kernel source (null otherwise)"},
        "context": "the pages report no throughput; their only figure is ~2% max relative error "
                   "of un-promoted FP8 accumulation at K=4096 on Hopper",
    }
    out.update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d["A"], d["B"])
        progress("cpu baseline done")
    print(json.dumps(out), flush=True)


def outside_step(env):
    """Entries outside the step, each on >= 1 GiB of rotated operand sets;
    returns {"kernels": {...}, "hbm_copy_context": ..., "error_context": ...}."""
    import numpy as np
    import torch

    from fp8_fine_grained_x1_amd import binding as B
    from fp8_fine_grained_x1_amd import tensors as T
    from fp8_fine_grained_x1_amd import workloads

    dev, stream, M, N, K, G = env["dev"], env["stream"], env["M"], env["N"], env["K"], env["G"]
    to_dev, timed, gemm, requant = env["to_dev"], env["timed"], env["gemm"], env["requant"]
    quant_a, quant_b, new_step_set = env["quant_a"], env["quant_b"], env["new_step_set"]
    gbs, tflops, q_entry, g_entry = env["gbs"], env["tflops"], env["q_entry"], env["g_entry"]
    st0 = env["sets"][0]
    flops, bytes_qa, bytes_rq = env["flops"], env["bytes_qa"], env["bytes_rq"]
    kernels = {}

    def rel_err(c, ref):
        """rel_frob and max_rel (|ref| > 1e-2 rms(ref)) in float64 on the GPU."""
        c = c.to(torch.float64)
        ref = ref.to(torch.float64)
        fro = float(torch.linalg.norm(c - ref) / torch.linalg.norm(ref))
        mask = ref.abs() > 1e-2 * torch.sqrt(torch.mean(ref * ref))
        mr = float(((c - ref).abs()[mask] / ref.abs()[mask]).max())
        return fro, mr

    # ---- 128x1 requantization of the step's FP8 activations (transposed out)
    base = dict(qa=st0["qa"].clone(), sa=st0["sa"].clone(),
                q2=torch.empty((K, M), dtype=torch.uint8, device=dev),
                s2=torch.empty((M // 128, K), dtype=torch.float32, device=dev))
    rs = clones(base, n_sets(nbytes(*base.values())))
    ms = timed([lambda s=s: requant(s) for s in rs])
    b2b = env["timed_batch"]([lambda s=s: requant(s) for s in rs])
    kernels["fp8_quantize_rowtile_128x1_requant (outside the step)"] = q_entry(bytes_rq, ms, len(rs), b2b)
    progress("requant 128x1 timed")
    del rs, base

    # ---- power-of-two 1x128 rule on the step's activations
    base = dict(a=st0["a"], qa=torch.empty((M, K), dtype=torch.uint8, device=dev),
                sa=torch.empty((G, M), dtype=torch.float32, device=dev))
    ps = clones(base, n_sets(nbytes(*base.values())))
    ms = timed([lambda s=s: quant_a(s, B.FP8FG_SCALE_POW2) for s in ps])
    b2b = env["timed_batch"]([lambda s=s: quant_a(s, B.FP8FG_SCALE_POW2) for s in ps])
    kernels["fp8_quantize_rowtile_1x128_pow2 (outside the step)"] = q_entry(bytes_qa, ms, len(ps), b2b)
    progress("pow2 1x128 timed")
    del ps, base

    # ---- E8M0-scale path (FP8 MFMA dequantizing): power-of-two operands, and
    # the step's own amax operands; error against the exact default path's
    # FP32 result on the same operands (which matches the oracle to ~1e-7)
    for label, rule in (("pow2 scales", B.FP8FG_SCALE_POW2), ("amax scales, the step's operands",
                                                                B.FP8FG_SCALE_AMAX)):
        base = new_step_set(st0["a"], st0["b"])
        quant_a(base, rule)
        quant_b(base, rule)
        del base["a"], base["b"]
        c_mx = torch.empty((M, N), dtype=torch.float32, device=dev)
        c_ex = torch.empty((M, N), dtype=torch.float32, device=dev)
        gemm(base, B.FP8FG_GEMM_E8M0_SCALES, c_mx)
        gemm(base, B.FP8FG_GEMM_DEFAULT, c_ex)
        fro, mr = rel_err(c_mx, c_ex)
        del c_mx, c_ex
        gs = clones(base, n_sets(nbytes(*base.values())))
        ms = timed([lambda s=s: gemm(s, B.FP8FG_GEMM_E8M0_SCALES) for s in gs])
        kernels["fp8_gemm_blockscaled E8M0_SCALES (FP8 MFMA dequantizing; %s), 4096x7168x7168 "
                "(outside the step)" % label] = g_entry(
            flops, ms, len(gs), peak=PEAK_FP8_TFLOPS,
            rel_frob_vs_exact_path=float("%.3e" % fro), max_rel_vs_exact_path=float("%.3e" % mr))
        progress("E8M0 GEMM (%s) timed" % label)
        del gs, base

    # ---- Dgrad dX [M][K] = dY [M][N] . W^T of a layer of the same shape: dY
    # quantized 1x128 along N, W [K][N] block-quantized without the transpose
    d6 = workloads.workload_inputs(6)
    dy6, w6 = to_dev(d6["dY"]), to_dev(d6["W"])
    base = dict(qd=torch.empty((M, N), dtype=torch.uint8, device=dev),
                sd=torch.empty((N // 128, M), dtype=torch.float32, device=dev),
                qw=torch.empty((K, N), dtype=torch.uint8, device=dev),
                sw=torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev),
                c=torch.empty((M, K), dtype=torch.bfloat16, device=dev))
    B.fp8_quantize_rowtile(dy6, B.FP8FG_BF16, M, N, N, None, 0, 0, B.FP8FG_TILE_1x128,
                           B.FP8FG_SCALE_AMAX, base["qd"], N, base["sd"], 1, M, stream)
    B.fp8_quantize_block(w6, B.FP8FG_BF16, K, N, N, B.FP8FG_SCALE_AMAX, 0, base["qw"], N,
                         base["sw"], N // 128, 1, stream)
    del dy6, w6, d6

    def dgrad(s):
        B.fp8_gemm_blockscaled(M, K, N, s["qd"], N, s["sd"], 1, M, s["qw"], N, s["sw"], N // 128, 1,
                               B.FP8FG_BSCALE_BLOCK128, s["c"], B.FP8FG_BF16, K,
                               B.FP8FG_GEMM_DEFAULT, stream)

    gs = clones(base, n_sets(nbytes(*base.values())))
    ms = timed([lambda s=s: dgrad(s) for s in gs])
    kernels["fp8_gemm_blockscaled dgrad dX = dY.W^T, 4096x7168x7168 (outside the step)"] = g_entry(
        flops, ms, len(gs))
    progress("dgrad timed")
    del gs, base

    # ---- grouped GEMMs (MoE): power-of-two 1x128 activation scales
    # (group-major), per-expert 128x128 weight blocks, transposed
    def grouped_setup(w):
        dw = workloads.workload_inputs(w)
        spec = workloads.WORKLOADS[w]
        Gx, Mx, Nx, Kx = spec["G"], spec["M"], spec["N"], spec["K"]
        ax = to_dev(dw["A"])
        o = dict(qa=torch.empty((Mx, Kx), dtype=torch.uint8, device=dev),
                 sa=torch.empty((Kx // 128, Mx), dtype=torch.float32, device=dev),
                 qb=torch.empty((Gx, Nx, Kx), dtype=torch.uint8, device=dev),
                 sb=torch.empty((Gx, Kx // 128, Nx // 128), dtype=torch.float32, device=dev),
                 c=torch.empty((Mx, Nx), dtype=torch.bfloat16, device=dev),
                 off=torch.from_numpy(dw["offsets"].astype(np.int32)).to(dev))
        B.fp8_quantize_rowtile(ax, B.FP8FG_BF16, Mx, Kx, Kx, None, 0, 0, B.FP8FG_TILE_1x128,
                               B.FP8FG_SCALE_POW2, o["qa"], Kx, o["sa"], 1, Mx, stream)
        for e in range(Gx):
            we = to_dev(dw["W"][e])
            B.fp8_quantize_block(we, B.FP8FG_BF16, Kx, Nx, Nx, B.FP8FG_SCALE_AMAX, 1, o["qb"][e], Kx,
                                 o["sb"][e], Nx // 128, 1, stream)
        torch.cuda.synchronize()
        meta = dict(G=Gx, M=Mx, N=Nx, K=Kx, counts=dw["counts"].tolist())
        return o, meta

    def grouped(o, m):
        B.fp8_grouped_gemm_blockscaled(m["G"], o["off"], m["M"], m["N"], m["K"], o["qa"], m["K"],
                                       o["sa"], 1, m["M"], o["qb"], m["K"], m["N"] * m["K"], o["sb"],
                                       1, m["N"] // 128, (m["K"] // 128) * (m["N"] // 128), o["c"],
                                       B.FP8FG_BF16, m["N"], B.FP8FG_GEMM_DEFAULT, stream)

    for w, label in ((4, "MoE up-projection G=8, 16384 tokens, K=7168 -> N=4096, pow2 activation "
                         "scales"),
                     (7, "MoE down-projection G=8, 16384 tokens, K=4096 -> N=7168, pow2 activation "
                         "scales"),
                     (8, None)):
        o, m = grouped_setup(w)
        gs = clones(o, n_sets(nbytes(*o.values())))
        ms = timed([lambda s=s: grouped(s, m) for s in gs])
        nf = 2.0 * m["M"] * m["N"] * m["K"]
        if label is not None:
            kernels["fp8_grouped_gemm_blockscaled %s (outside the step)" % label] = g_entry(nf, ms, len(gs))
        else:
            # algorithmic bytes of the decode call: every expert's weights and
            # block scales once, the activations and their scales once, the
            # bf16 output once
            nb = (m["G"] * m["N"] * m["K"] + m["G"] * (m["K"] // 128) * (m["N"] // 128) * 4
                  + m["M"] * m["K"] + m["M"] * (m["K"] // 128) * 4 + m["M"] * m["N"] * 2)
            desc = "G=%d, %d tokens (%d-%d per expert), K=%d -> N=%d" % (
                m["G"], m["M"], min(m["counts"]), max(m["counts"]), m["K"], m["N"])
            e = q_entry(nb, ms, len(gs))
            e["TFLOP/s"] = round(tflops(nf, ms), 1)
            kernels["fp8_grouped_gemm_blockscaled MoE decode %s (outside the step)" % desc] = e
        progress("grouped workload %d timed" % w)
        del gs, o

    # ---- long-K dense GEMM (1024 x 4096 x 16384: 128 promotions per output)
    w3 = workloads.WORKLOADS[3]
    d3 = workloads.workload_inputs(3)
    a3, b3 = to_dev(d3["A"]), to_dev(d3["B"])
    qa3, sa3 = T.quantize_1x128(a3)
    qb3, sb3 = T.quantize_block(b3)
    base = dict(qa=qa3, sa=sa3, qb=qb3, sb=sb3,
                c=torch.empty((w3["M"], w3["N"]), dtype=torch.bfloat16, device=dev))
    gs = clones(base, n_sets(nbytes(*base.values())))
    ms = timed([lambda s=s: T.gemm(s["qa"], s["sa"], s["qb"], s["sb"], out=s["c"]) for s in gs])
    kernels["fp8_gemm_blockscaled long K 1024x4096x16384 (outside the step)"] = g_entry(
        2.0 * w3["M"] * w3["N"] * w3["K"], ms, len(gs))
    del gs
    progress("long K timed")
    error_context = long_k_error_gap(a3, b3, qa3, sa3, qb3, sb3, rel_err)
    progress("long-K error gap measured")
    del base, qa3, sa3, qb3, sb3, a3, b3, d3

    # ---- weight gradient dW [F][N] = X^T dY over T = 8192 tokens: X and dY
    # quantized 1x128, requantized to 128x1 tiles (transposed, per-column
    # scales along the token axis), FP32 out
    w5 = workloads.WORKLOADS[5]
    d5 = workloads.workload_inputs(5)
    qx5, sx5 = T.requantize_128x1(*T.quantize_1x128(to_dev(d5["X"])))
    qd5, sd5 = T.requantize_128x1(*T.quantize_1x128(to_dev(d5["dY"])))
    base = dict(qx=qx5, sx=sx5, qd=qd5, sd=sd5,
                c=torch.empty((w5["F"], w5["N"]), dtype=torch.float32, device=dev))
    gs = clones(base, n_sets(nbytes(*base.values())))
    ms = timed([lambda s=s: T.gemm(s["qx"], s["sx"], s["qd"], s["sd"], out=s["c"], col_scales=True)
                for s in gs])
    kernels["fp8_gemm_blockscaled wgrad dW = X^T.dY 7168x4096, 8192 tokens, 128x1 column scales, "
            "f32 out (outside the step)"] = g_entry(2.0 * w5["F"] * w5["N"] * w5["T"], ms, len(gs))
    progress("wgrad timed")
    del gs, base, qx5, sx5, qd5, sd5, d5

    # ---- context: a plain 1 GiB device-to-device copy (the runtime's copy
    # kernel), read + write bytes per time
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    cp_dst = torch.empty_like(cp_src)
    cp_ms = timed([lambda: cp_dst.copy_(cp_src)], reps=10)
    del cp_src, cp_dst
    # ... and torch's own cast of the step's activations to E4M3 (2 bytes in,
    # 1 out per element, no maxima or scales): a stream with the 1x128
    # quantizer's read/write mix
    cast_base = dict(a=st0["a"], o=torch.empty(st0["a"].shape, dtype=torch.float8_e4m3fn, device=dev))
    cast_sets = clones(cast_base, n_sets(nbytes(*cast_base.values())))
    cast_ms = env["timed_batch"]([lambda s=s: s["o"].copy_(s["a"]) for s in cast_sets])
    cast_bytes = st0["a"].numel() * 3
    del cast_sets, cast_base
    progress("copy context timed")
    vendor = vendor_gemm_context(timed, nbytes, n_sets, tflops)
    progress("vendor GEMM context timed")
    return {
        "kernels": kernels,
        "hbm_copy_context": {
            "1 GiB device copy GB/s (read + write)": round(gbs(2 * (1 << 30), cp_ms), 1),
            "frac_hbm": round(gbs(2 * (1 << 30), cp_ms) / PEAK_HBM_GBS, 3),
            "torch bf16 -> float8_e4m3fn cast of the 4096x7168 activations GB/s (back to back)":
                round(gbs(cast_bytes, cast_ms), 1),
            "cast_frac_hbm": round(gbs(cast_bytes, cast_ms) / PEAK_HBM_GBS, 3)},
        "vendor_gemm_context": vendor,
        "error_context": error_context,
    }


def vendor_gemm_context(timed, nbytes, n_sets, tflops):
    """The vendor library (hipBLASLt through torch) on the dense forward
    shape 4096 x 7168 x 7168, same run, rotated operand sets: its FP8 GEMM
    with one scale per tensor and with one scale per row of A and column of
    B (no per-K-group scaling, accumulated inside the FP8 matrix core over
    the whole K), and its BF16 GEMM.  They show what the matrix cores deliver
    on this shape under the chip's power limit; none of them is the method
    (the first two are the un-promoted kind of accumulation whose error the
    method removes)."""
    import torch
    dev = torch.device("cuda:0")
    M, N, K = 4096, 7168, 7168
    g = torch.Generator(device=dev).manual_seed(5)
    a = torch.randn(M, K, generator=g, device=dev).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, generator=g, device=dev) * 9.0).to(torch.float8_e4m3fn)
    out = {}
    flops = 2.0 * M * N * K
    try:
        base = dict(a=a, b=b, c=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
        sets = [base] + [{k: v.clone() for k, v in base.items()}
                         for _ in range(n_sets(nbytes(*base.values())) - 1)]
        one = torch.ones((), device=dev)
        ra, rb = torch.ones((M, 1), device=dev), torch.ones((1, N), device=dev)
        ms = timed([lambda s=s: torch._scaled_mm(s["a"], s["b"].t(), scale_a=one, scale_b=one,
                                                 out_dtype=torch.bfloat16, out=s["c"]) for s in sets])
        out["fp8 per-tensor scales, TFLOP/s"] = round(tflops(flops, ms), 1)
        ms = timed([lambda s=s: torch._scaled_mm(s["a"], s["b"].t(), scale_a=ra, scale_b=rb,
                                                 out_dtype=torch.bfloat16, out=s["c"]) for s in sets])
        out["fp8 row/column scales, TFLOP/s"] = round(tflops(flops, ms), 1)
        del sets, base
    except (RuntimeError, TypeError) as e:  # no FP8 GEMM in this torch build
        out["fp8"] = "unavailable: %s" % str(e)[:120]
    del a, b
    a = torch.randn(M, K, generator=g, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, generator=g, device=dev, dtype=torch.bfloat16)
    base = dict(a=a, b=b, c=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    sets = [base] + [{k: v.clone() for k, v in base.items()}
                     for _ in range(n_sets(nbytes(*base.values())) - 1)]
    ms = timed([lambda s=s: torch.matmul(s["a"], s["b"], out=s["c"]) for s in sets])
    out["bf16, TFLOP/s"] = round(tflops(flops, ms), 1)
    out["fp8 peak TFLOP/s"] = PEAK_FP8_TFLOPS
    return out


def long_k_error_gap(a3, b3, qa3, sa3, qb3, sb3, rel_err):
    """Long-K workload (1024 x 4096 x 16384, U(-1,1)): the fine-grained path
    (1x128 / 128x128 scales, exact partial sums promoted every 128 of K) and
    the naive baseline (per-tensor scales, the whole K summed in the FP8
    matrix core, no promotion) against the unquantized product, and the
    naive path against the exact product of its own E4M3 operands (its
    accumulation error alone).  64 sampled rows, all 4096 columns, float64
    references on the GPU.  The per-tensor operands are prepared here, as a
    harness would (scale = tensor amax / 448, E4M3 by torch's cast)."""
    import torch

    from fp8_fine_grained_x1_amd import binding as B
    from fp8_fine_grained_x1_amd import tensors as T

    M, Kx = a3.shape
    N = b3.shape[1]
    rows = torch.linspace(0, M - 1, 64, device=a3.device).round().long()
    af, bf = a3.float(), b3.float()
    s_a = (af.abs().max() / 448.0).reshape(1)
    s_b = (bf.abs().max() / 448.0).reshape(1)
    qa_n = (af / s_a).to(torch.float8_e4m3fn).view(torch.uint8)
    qb_n = (bf / s_b).t().contiguous().to(torch.float8_e4m3fn).view(torch.uint8)   # [N][K]
    naive = T.gemm(qa_n, s_a, qb_n, s_b, out_dtype=torch.float32, no_promotion=True)[rows]
    fine = T.gemm(qa3, sa3, qb3, sb3, out_dtype=torch.float32)[rows]
    truth = a3[rows].double() @ b3.double()
    own = ((qa_n[rows].view(torch.float8_e4m3fn).double() * s_a.double()) @
           (qb_n.view(torch.float8_e4m3fn).double().t().contiguous() * s_b.double()))
    f_fro, f_mr = rel_err(fine, truth)
    n_fro, n_mr = rel_err(naive, truth)
    a_fro, a_mr = rel_err(naive, own)
    torch.cuda.synchronize()
    return {
        "workload": "long-K 1024x4096x16384, U(-1,1); 64 sampled rows x 4096 columns",
        "fine_grained_vs_unquantized": {"rel_frob": float("%.4e" % f_fro), "max_rel": float("%.4e" % f_mr)},
        "naive_per_tensor_no_promotion_vs_unquantized": {"rel_frob": float("%.4e" % n_fro),
                                                         "max_rel": float("%.4e" % n_mr)},
        "naive_accumulation_vs_exact_product_of_its_operands": {"rel_frob": float("%.4e" % a_fro),
                                                               "max_rel": float("%.4e" % a_mr)},
        "pages_context": "~2% max relative error of limited-width FP8 accumulation at K=4096 "
                         "(Hopper, preliminary test; no inputs given)",
    }


def kernel_only(args, env):
    """One kernel alone, repeated over >= 1 GiB of rotated operand sets: the
    GEMM's default path on the step's amax operands, the E8M0-scale path on
    power-of-two operands, or one of the step's quantizers."""
    import numpy as np
    import torch

    from fp8_fine_grained_x1_amd import binding as B

    M, N, K = env["M"], env["N"], env["K"]
    a0, b0 = env["a0"], env["b0"]
    new_step_set, quant_a, quant_b = env["new_step_set"], env["quant_a"], env["quant_b"]
    gemm, requant, stream = env["gemm"], env["requant"], env["stream"]
    k = args.kernel
    if k in ("gemm", "e8m0"):
        rule = B.FP8FG_SCALE_POW2 if k == "e8m0" else B.FP8FG_SCALE_AMAX
        base = new_step_set(a0, b0)
        quant_a(base, rule)
        quant_b(base, rule)
        del base["a"], base["b"]
        flags = B.FP8FG_GEMM_E8M0_SCALES if k == "e8m0" else B.FP8FG_GEMM_DEFAULT
        sets = clones(base, n_sets(nbytes(*base.values())))
        fn = lambda s: gemm(s, flags)
        work = 2.0 * M * N * K
    elif k == "quant1x128":
        base = new_step_set(a0, b0)
        del base["b"], base["qb"], base["sb"], base["c"]
        sets = clones(base, n_sets(nbytes(*base.values())))
        fn = quant_a
        work = M * K * 3 + M * (K // 128) * 4
    elif k == "quant128x128":
        base = new_step_set(a0, b0)
        del base["a"], base["qa"], base["sa"], base["c"]
        sets = clones(base, n_sets(nbytes(*base.values())))
        fn = quant_b
        work = K * N * 3 + (K // 128) * (N // 128) * 4
    else:
        base = new_step_set(a0, b0)
        quant_a(base)
        base = dict(qa=base["qa"], sa=base["sa"],
                    q2=torch.empty((K, M), dtype=torch.uint8, device=env["dev"]),
                    s2=torch.empty((M // 128, K), dtype=torch.float32, device=env["dev"]))
        sets = clones(base, n_sets(nbytes(*base.values())))
        fn = requant
        work = M * K * 2 + M * (K // 128) * 4 + (M // 128) * K * 4
    for i in range(args.warmup):
        fn(sets[i % len(sets)])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        fn(sets[i % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    rate = ({"TFLOP/s": round(work / (ms * 1e-3) / 1e12, 1)} if k in ("gemm", "e8m0")
            else {"GB/s": round(work / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": work})
    print(json.dumps(dict(kernel=k, ms=round(ms, 4), rotated_sets=len(sets), **rate)), flush=True)


if __name__ == "__main__":
    main()
