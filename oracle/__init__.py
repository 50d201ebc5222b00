"""CPU oracle for the Jet-RL mixed-granularity FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or execute anything in this package.  The product path (the HIP
library and its Python binding in ``quantized_rl_amd``) never calls it, and
this package never imports the product: the two share no code.

What it computes, and where the pages define it (Jet-RL, arXiv 2601.14243;
page "paper.rainbus.top/paper/2601.14243", sections "FP8 量化 (E4M3 格式)",
"Per-group / Per-block 量化粒度", "核心方法" and "方法步骤详情"):

* ``e4m3``   -- the OCP E4M3FN codec (4 exponent bits, 3 mantissa bits, largest
  finite value 448) and the cast written as a bracket around X / S_X, read as a
  round-to-nearest-even, saturating cast.
* ``quant``  -- S = max|X| / 448 in fp32; 1x128 groups for activations and
  gradients, 128x128 blocks for weights; the fused RMSNorm + 1x128 quantiser;
  and the requantisation of a saved 1x128 FP8 tensor into 128x1 groups along
  the token dimension, stored transposed.
* ``norm``   -- the gradients of the RMSNorm (dx, dgamma) in fp64, and their
  acceptance check.
* ``swiglu`` -- SiLU(gate) * up of the gate+up projection's output, quantised
  1x128 for the down projection (the fused quantisation of "核心方法"; SiLU with
  a correctly rounded fp32 exponential).
* ``layout`` -- the rollout-packed byte order of the weight codes (a
  permutation the library defines for its rollout FProp; no arithmetic).
* ``gemm``   -- the three block-scaled GEMMs (FProp Y = X W^T, DGrad
  dX = dY W, WGrad dW = dY^T X) as their plain definition on dequantised values
  in fp64, the bf16 rounding of the result, and the acceptance check.

Every floating-point step of the quantisers is one IEEE-754 binary32 operation
with round-to-nearest-even, written with numpy float32 arithmetic, in the
order the definition states.  The GEMMs are plain fp64 matrix products.

Pins: ``tests/test_oracle_*.py`` check each function against closed forms,
invariants, hand-derived golden cases (``tests/golden``), library routines,
brute force and exact rational arithmetic.  ``rmsnorm_quant`` and
``swiglu_quant`` follow readings of the pages (no formula is printed for the
RMSNorm or for SiLU), and are pinned bit for bit to exact evaluations of those
readings.  The RMSNorm backward (``norm``) follows from calculus on the forward
reading; it is pinned against central finite differences of the forward,
torch's autograd of rms_norm in float64 and a closed-form identity for
sum_k x_k dx_k.
"""

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_table
from .quant import (
    bf16_bits_to_f32,
    quant_act_1x128,
    quant_act_1x128_f32,
    rmsnorm_f32,
    rmsnorm_rstd_f32,
    quant_weight_128x128,
    rmsnorm_quant,
    requant_transpose_128x1,
    pairwise_sum_f32,
)
from .norm import check_rmsnorm_backward, rmsnorm_backward_ref
from .swiglu import exp_rn32, silu_f32, swiglu_f32, swiglu_quant
from .layout import pack_weight_rollout
from .gemm import (
    dequant_groups,
    dequant_blocks,
    gemm_fprop_ref,
    gemm_dgrad_ref,
    gemm_wgrad_ref,
    gemm_fprop_ref_at,
    gemm_dgrad_ref_at,
    gemm_wgrad_ref_at,
    f64_to_bf16_bits,
    bf16_ulp,
    check_gemm,
    check_gemm_f32,
)

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_table",
    "bf16_bits_to_f32", "quant_act_1x128", "quant_act_1x128_f32", "rmsnorm_f32", "rmsnorm_rstd_f32", "rmsnorm_backward_ref", "check_rmsnorm_backward", "quant_weight_128x128", "rmsnorm_quant",
    "requant_transpose_128x1", "pairwise_sum_f32",
    "dequant_groups", "dequant_blocks", "gemm_fprop_ref", "gemm_dgrad_ref", "gemm_wgrad_ref",
    "gemm_fprop_ref_at", "gemm_dgrad_ref_at", "gemm_wgrad_ref_at",
    "f64_to_bf16_bits", "bf16_ulp", "check_gemm", "check_gemm_f32",
    "exp_rn32", "silu_f32", "swiglu_f32", "swiglu_quant",
    "pack_weight_rollout",
]
