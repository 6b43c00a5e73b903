"""Fine-grained FP8 quantization and block-scaled FP8 GEMM for MI355X (gfx950).

The compute lives in the HIP library ``libfp8fg.so`` (sources under
``csrc/``, C interface in ``include/fp8fg.h``); ``binding`` marshals
arguments to it and ``workloads`` draws the seeded synthetic inputs.
"""
