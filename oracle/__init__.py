"""CPU oracle for fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library under
``fp8_fine_grained_x1_amd/csrc`` and imports nothing from it.

What it computes follows the DeepSeek-V3 FP8 text as it appears on the pages
(page keys as in the list below; no page has section numbers, so passages are
named by their subject, and by the figure or appendix they mention):

* [why-be]   why-be.why-be.co.kr (untitled): online max-abs per 1x128
  activation tile / 128x128 weight block, E4M3 on all tensors, the 1x128 ->
  128x1 conversion for the backward pass and integral power-of-two scales.
* [thedaegu] thedaegu.com, "OMG! The most effective Deepseek Ever!": scaling
  the max-abs onto the largest FP8 value, exponent sharing within small
  groups, promotion of partial sums to FP32 (Figure 7(b) passage), the three
  FP8 GEMMs of a Linear (Figure 6 passage).
* [hearaon]  hearaon.co.kr (untitled): limited-width tensor-core
  accumulation; quantizing activations before the MoE up-projection.
* [fooled]   xn--jj0bz6z98ct0a29q.com, "Don't Be Fooled By Deepseek Chatgpt":
  the mixed-precision framework and promotion to CUDA cores.

Readings of places where the pages are silent (all fixed here, mirrored
by the HIP path):
  * FP8 format: OCP E4M3FN (bias 7, max finite 448, no infinity, NaN =
    S.1111.111); rounding is round-to-nearest-even with saturation.
  * scale s = RN32(amax / 448) is the dequantization multiplier; the
    quantized value is E4M3(RN32(x / s)) -- two roundings, fp32 division
    correctly rounded.
  * s is floored at 2**-126 so all-zero tiles give s = 2**-126 and zero bytes.
  * power-of-two rule: s = max(2**ceil(log2(amax / 448)), 2**-126).
  * signed zeros are kept (-0 encodes as 0x80).

Parity status: every public function here is pinned by tests under
``tests/test_oracle_*.py`` (brute force, closed forms, exact rational
arithmetic, an independent library cast); see the header of each module.
"""

from .e4m3 import (E4M3_MAX, decode, encode, code_magnitudes)
from .quant import (bf16_bits_to_f32, amax_scale, pow2_scale,
                    quantize_1x128, quantize_128x128, quantize_128x1,
                    quantize_per_tensor, requantize_128x1,
                    dequantize_1x128, dequantize_128x128, dequantize_128x1,
                    SCALE_AMAX, SCALE_POW2)
from .gemm import (gemm_blockscaled, gemm_blockscaled_colscale,
                   grouped_gemm_blockscaled, wgrad, gemm_per_tensor,
                   bf16_rne_bits, bf16_bits_to_f64)
from .metrics import rel_frob, max_rel
from .limited_acc import limited_dot, gemm_limited_per_tensor

__all__ = [
    "E4M3_MAX", "decode", "encode", "code_magnitudes",
    "bf16_bits_to_f32", "amax_scale", "pow2_scale",
    "quantize_1x128", "quantize_128x128", "quantize_128x1",
    "quantize_per_tensor", "requantize_128x1",
    "dequantize_1x128", "dequantize_128x128", "dequantize_128x1",
    "SCALE_AMAX", "SCALE_POW2",
    "gemm_blockscaled", "gemm_blockscaled_colscale",
    "grouped_gemm_blockscaled", "wgrad", "gemm_per_tensor",
    "limited_dot", "gemm_limited_per_tensor",
    "bf16_rne_bits", "bf16_bits_to_f64", "rel_frob", "max_rel",
]
