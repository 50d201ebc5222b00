"""MI355X (gfx950) FP8 linear layer of Jet-RL's unified FP8 precision flow.

The compute path is the C-ABI library ``libjetfp8.so`` (hand-written HIP for
gfx950, declared in ``include/jetfp8.h``); this package holds its build script
(``build``), a thin ctypes binding (``_lib``) whose functions carry the same
names as the C entry points, and the seeded input generators (``synth``).
The library is loaded on first use; nothing here falls back to another path.
"""

from ._lib import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    JetFP8Error,
    gemm_dgrad,
    gemm_fprop,
    gemm_fprop_packed,
    gemm_fprop_quant,
    gemm_fprop_splitk,
    gemm_fprop_splitk_noalloc,
    gemm_fprop_swiglu_quant,
    gemm_fprop_splitk_workspace_bytes,
    gemm_wgrad,
    gemm_wgrad_f32,
    pack_weight_rollout,
    quantize_act_1x128,
    quantize_weight_128x128,
    requant_transpose_128x1,
    rmsnorm_backward,
    rmsnorm_backward_workspace_bytes,
    rmsnorm_quant,
    rmsnorm_quant_rstd,
    swiglu_quant,
)
