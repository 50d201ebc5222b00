"""SwiGLU + 1x128 quantisation of the down projection's input (oracle; test
infrastructure only).

Where the pages stand: the summary page (paper.rainbus.top/paper/2601.14243)
says the quantisation of the forward and backward passes is fused into the
neighbouring kernels to cut its overhead (section "核心方法"), and that the
training forward quantises exactly as the inference engine does ("方法步骤详情"
step 2).  The models it trains (Qwen3, Llama) feed their MLP down projection
with SwiGLU(gate, up) = SiLU(gate) * up, which the 1x128 quantiser then turns
into FP8; the pages define neither SiLU nor the layout of the fused gate+up
output.  Readings (every step one IEEE-754 binary32 operation, round to
nearest even):

* the gate+up projection's output y [M, 2I] (bf16) holds gate in columns
  0 .. I-1 and up in columns I .. 2I-1;
* E = the fp32 value nearest to e^(-g) (correctly rounded; +inf past the fp32
  range), d = fl32(1 + E), silu(g) = fl32(g / d) (a true division);
* h = fl32(silu(g) * u), quantised 1x128 exactly as quant_act_1x128 does for an
  fp32 input (no bf16 rounding of h in between).

The gate values are bf16, so e^(-g) is only ever needed at 65536 arguments;
tests/test_oracle_swiglu.py checks ``exp_rn32`` against a 60-digit evaluation on
every one of them.
"""

import numpy as np

from .quant import bf16_bits_to_f32, quant_act_1x128_f32

_ONE = np.float32(1.0)


def exp_rn32(x):
    """The fp32 value nearest to e^x for float32 x: numpy's fp64 exp (within an
    ulp) rounded once to fp32, which is the correctly rounded result wherever
    e^x is at least 2^-51 (relatively) away from an fp32 rounding midpoint --
    every bf16 argument included."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        return np.exp(x.astype(np.float64)).astype(np.float32)


def silu_f32(g):
    """silu(g) = fl32(g / fl32(1 + E)), E = exp_rn32(-g); g float32."""
    g = np.asarray(g, dtype=np.float32)
    e = exp_rn32(-g)
    d = (_ONE + e).astype(np.float32)
    return (g / d).astype(np.float32)


def swiglu_f32(y_bf16):
    """h = fl32(silu(gate) * up) [M, I] from the gate+up output y [M, 2I] (bf16 bits)."""
    y = bf16_bits_to_f32(y_bf16)
    if y.ndim != 2 or y.shape[1] % 256:
        raise ValueError("expected y [M, 2I] with I a multiple of 128")
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite input is outside the contract")
    i = y.shape[1] // 2
    with np.errstate(over="ignore"):  # an overflowing h is rejected by the quantiser
        return (silu_f32(y[:, :i]) * y[:, i:]).astype(np.float32)


def swiglu_quant(y_bf16):
    """SwiGLU of the gate+up output followed by the 1x128 quantiser.

    y_bf16: uint16 [M, 2I], I % 128 == 0.
    Returns (q uint8 [M, I], s float32 [I // 128, M])."""
    return quant_act_1x128_f32(swiglu_f32(y_bf16))
