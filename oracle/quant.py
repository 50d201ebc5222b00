"""Quantisers of the Jet-RL FP8 linear layer (oracle; test infrastructure only).

Definitions followed (page paper.rainbus.top/paper/2601.14243):

* section "FP8 量化 (E4M3 格式)": scale S_X = max(|X|) / 448, quantised value
  [X / S_X] (cast to E4M3);
* section "Per-group / Per-block 量化粒度" and "方法步骤详情" step 1: activations
  and gradients use 1x128 per-group scaling (128 consecutive elements along a
  row), weights use 128x128 per-block scaling;
* "方法步骤详情" steps 3-4 and "技术新颖性": the forward pass saves the FP8
  activation in 1x128 groups; the backward pass needs 128x1 groups (along the
  token dimension) for the weight-gradient GEMM, so the saved tensor is
  requantised;
* "方法步骤详情" step 5: a fused RMSNorm kernel precedes quantisation.

Readings where the pages are silent (each is one numpy float32 operation, i.e.
one IEEE-754 binary32 operation rounded to nearest even):

* S = fl32(amax / 448) is a true division; S = 1 when that quotient is 0, i.e.
  when amax == 0 or amax <= 448 * 2^-150 (a nonzero amax so small that the fp32
  quotient underflows to zero, which only requantised or RMSNorm'ed fp32 values
  can reach); every code of such a group is then e4m3(x), a signed zero;
* q = e4m3(fl32(x / S)) -- the quotient is rounded to fp32, then cast;
* requantisation dequantises in fp32, v = fl32(decode(q) * S), then applies the
  same rule down each 128-token column;
* RMSNorm: y = fl32(fl32(x * inv) * gamma) with inv = fl32(1 / fl32(sqrt(d))),
  d = fl32(fl32(ss / K) + eps), ss = the pairwise-tree fp32 sum of x*x (adjacent
  pairs added level by level, an odd last element carried up unchanged); y is
  quantised without any intermediate bf16 rounding.

Layouts: bf16 tensors are uint16 bit patterns.  A 1x128-grouped tensor Q[R, C]
carries scales S[C // 128, R] (group-major: S[g, r] scales row r's g-th group).
A 128x128-blocked weight Q[N, K] carries S[N // 128, K // 128].  The 128x1
requantised tensor is stored transposed: Qt[K, M] with St[M // 128, K].
"""

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode

GROUP = 128
_F448 = np.float32(448.0)
_ONE = np.float32(1.0)


def bf16_bits_to_f32(u):
    """bf16 bit patterns (uint16) -> float32, exact."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_from_amax(amax):
    """S = amax / 448 in fp32 (true division); S = 1 where that quotient is zero
    (amax == 0, or an amax that underflows when divided by 448)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / _F448).astype(np.float32)
    return np.where(s == np.float32(0.0), _ONE, s).astype(np.float32)


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")


def quant_act_1x128(x_bf16):
    """1x128 per-group quantisation of an activation or gradient.

    x_bf16: uint16 [R, C] (bf16 bits), C % 128 == 0.
    Returns (q uint8 [R, C], s float32 [C // 128, R]).
    """
    x = bf16_bits_to_f32(x_bf16)
    return quant_act_1x128_f32(x)


def quant_act_1x128_f32(x):
    """Same as quant_act_1x128, on an fp32 input (used by rmsnorm_quant)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % GROUP:
        raise ValueError("expected [R, C] with C a multiple of 128")
    _check_finite(x)
    r, c = x.shape
    g = x.reshape(r, c // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2) if r else np.zeros((0, c // GROUP), np.float32)
    s = _scale_from_amax(amax)  # [R, C/128]
    y = (g / s[:, :, None]).astype(np.float32)  # fp32 division, one rounding
    q = e4m3_encode(y).reshape(r, c)
    return q, np.ascontiguousarray(s.T)


def quant_weight_128x128(w_bf16):
    """128x128 per-block quantisation of a weight.

    w_bf16: uint16 [N, K] (bf16 bits), N % 128 == K % 128 == 0.
    Returns (q uint8 [N, K], s float32 [N // 128, K // 128]).
    """
    w = bf16_bits_to_f32(w_bf16)
    if w.ndim != 2 or w.shape[0] % GROUP or w.shape[1] % GROUP:
        raise ValueError("expected [N, K] with N and K multiples of 128")
    _check_finite(w)
    n, k = w.shape
    b = w.reshape(n // GROUP, GROUP, k // GROUP, GROUP)
    amax = np.max(np.abs(b), axis=(1, 3))  # [N/128, K/128]
    s = _scale_from_amax(amax)
    y = (b / s[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(y).reshape(n, k)
    return q, s


def pairwise_sum_f32(v):
    """Pairwise-tree fp32 sum along the last axis of a 2-D float32 array.

    Level by level, element 2i is added to element 2i+1 (fp32 add); an odd last
    element is carried to the next level unchanged.
    """
    v = np.asarray(v, dtype=np.float32)
    if v.shape[1] == 0:
        return np.zeros(v.shape[0], np.float32)
    while v.shape[1] > 1:
        carry = None
        if v.shape[1] % 2:
            carry = v[:, -1:]
            v = v[:, :-1]
        v = (v[:, 0::2] + v[:, 1::2]).astype(np.float32)
        if carry is not None:
            v = np.concatenate([v, carry], axis=1)
    return v[:, 0]


def rmsnorm_f32(x_bf16, gamma_bf16, eps):
    """The fp32 RMSNorm output y [M, K] that rmsnorm_quant quantises.

    x_bf16: uint16 [M, K]; gamma_bf16: uint16 [K]; eps: python float (rounded
    to the nearest fp32).
    """
    x = bf16_bits_to_f32(x_bf16)
    gamma = bf16_bits_to_f32(gamma_bf16)
    if x.ndim != 2 or gamma.shape != (x.shape[1],) or x.shape[1] == 0:
        raise ValueError("expected x [M, K], gamma [K], K > 0")
    _check_finite(x)
    _check_finite(gamma)
    inv = _rstd_f32(x, eps)
    return ((x * inv[:, None]).astype(np.float32) * gamma[None, :]).astype(np.float32)


def _rstd_f32(x, eps):
    k = x.shape[1]
    # fp32 arithmetic throughout: a square or a sum past the fp32 range is +inf
    # (and the factor then 0), which numpy would otherwise report as a warning
    with np.errstate(over="ignore"):
        sq = (x * x).astype(np.float32)
        ss = pairwise_sum_f32(sq)
        ms = (ss / np.float32(k)).astype(np.float32)
        d = (ms + np.float32(eps)).astype(np.float32)
        return (_ONE / np.sqrt(d)).astype(np.float32)  # correctly rounded sqrt, then a division


def rmsnorm_rstd_f32(x_bf16, eps):
    """The per-row fp32 factor inv = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))))
    that rmsnorm_f32 multiplies by (the value a forward saves for the backward)."""
    x = bf16_bits_to_f32(x_bf16)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("expected x [M, K], K > 0")
    _check_finite(x)
    return _rstd_f32(x, eps)


def rmsnorm_quant(x_bf16, gamma_bf16, eps):
    """Fused RMSNorm followed by the 1x128 quantiser.

    x_bf16: uint16 [M, K] with K % 128 == 0; gamma_bf16: uint16 [K].
    Returns (q uint8 [M, K], s float32 [K // 128, M]).
    """
    if np.asarray(x_bf16).ndim != 2 or np.asarray(x_bf16).shape[1] % GROUP:
        raise ValueError("expected x [M, K] with K a multiple of 128")
    return quant_act_1x128_f32(rmsnorm_f32(x_bf16, gamma_bf16, eps))


def requant_transpose_128x1(q, s):
    """Requantise a saved 1x128 FP8 tensor into 128x1 groups along its rows.

    q: uint8 [M, K]; s: float32 [K // 128, M]; M % 128 == 0.
    v[m, k] = fl32(decode(q[m, k]) * s[k // 128, m]); then for every column k and
    128-row block mb: S' = amax / 448 (1 if that quotient is 0) and q' = e4m3(fl32(v / S')).
    Returns (qt uint8 [K, M], st float32 [M // 128, K]) -- q' stored transposed,
    so each 128x1 group is contiguous.
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    m, k = q.shape
    if m % GROUP or k % GROUP or s.shape != (k // GROUP, m):
        raise ValueError("expected q [M, K], s [K/128, M], M and K multiples of 128")
    _check_finite(s)
    dec = e4m3_decode(q).astype(np.float32)  # exact
    s_full = np.repeat(s.T, GROUP, axis=1)  # [M, K]: s[k // 128, m]
    v = (dec * s_full).astype(np.float32)
    vt = np.ascontiguousarray(v.T).reshape(k, m // GROUP, GROUP)  # [K, M/128, 128]
    amax = np.max(np.abs(vt), axis=2)  # [K, M/128]
    st = _scale_from_amax(amax)
    y = (vt / st[:, :, None]).astype(np.float32)
    qt = e4m3_encode(y).reshape(k, m)
    return qt, np.ascontiguousarray(st.T)
