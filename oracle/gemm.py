"""Block-scaled FP8 GEMMs of the Jet-RL linear layer (oracle; test infra only).

Definitions (page paper.rainbus.top/paper/2601.14243, sections
"GEMM 量化布局（Row-wise 与 Column-wise）", "核心方法", "方法步骤详情" steps 2
and 4): FProp Y = X W^T with (1x128) x (128x128) granularity, DGrad
dX = dY W reusing that configuration (the weight blocks transposed), WGrad
dW = dY^T X with (1x128) x (128x1) granularity.

The oracle is the plain definition: dequantise each operand exactly in fp64
(decode(q) * scale -- a 4-bit by 24-bit significand product, exact in fp64),
multiply in fp64, then round to bf16 (fp64 -> fp32 -> bf16, both round to
nearest even) for the elementwise check.

Acceptance: with Yref = bf16(Yref64) (the oracle's own bf16 result),
normwise ||Y - Yref||_F / ||Yref64||_F <= 1e-3, and elementwise
|Y - Yref| <= ulp_bf16(Yref) + 1e-3 * rms(Yref64); an all-zero reference
requires an all-zero result.  The normwise bound is taken against the
bf16-rounded reference because rounding to bf16 alone (8 significant bits)
leaves a relative RMS error of about 1.1e-3 against the unrounded product, so
a bound of 1e-3 against Yref64 could not be met by any bf16 output.
"""

import numpy as np

from .e4m3 import e4m3_decode

GROUP = 128


def dequant_groups(q, s):
    """Dequantise a 1x128-grouped tensor: q uint8 [R, C], s f32 [C/128, R] -> f64 [R, C]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    r, c = q.shape
    assert s.shape == (c // GROUP, r)
    return e4m3_decode(q) * np.repeat(s.T.astype(np.float64), GROUP, axis=1)


def dequant_blocks(q, s):
    """Dequantise a 128x128-blocked weight: q uint8 [N, K], s f32 [N/128, K/128] -> f64 [N, K]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    n, k = q.shape
    assert s.shape == (n // GROUP, k // GROUP)
    full = np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)
    return e4m3_decode(q) * full


def gemm_fprop_ref(qx, sx, qw, sw):
    """Y64[M, N] = X W^T on dequantised operands (qx [M,K], sx [K/128,M], qw [N,K], sw [N/128,K/128])."""
    return dequant_groups(qx, sx) @ dequant_blocks(qw, sw).T


def gemm_dgrad_ref(qdy, sdy, qw, sw):
    """dX64[M, K] = dY W (qdy [M,N], sdy [N/128,M], qw [N,K], sw [N/128,K/128])."""
    return dequant_groups(qdy, sdy) @ dequant_blocks(qw, sw)


def gemm_wgrad_ref(qdyt, sdyt, qxt, sxt):
    """dW64[N, K] = dY^T X (qdyt [N,M], sdyt [M/128,N], qxt [K,M], sxt [M/128,K])."""
    return dequant_groups(qdyt, sdyt) @ dequant_groups(qxt, sxt).T


def _rows_groups(q, s, rows):
    """Dequantise selected rows of a 1x128-grouped tensor -> f64 [len(rows), C]."""
    q = np.asarray(q, dtype=np.uint8)[rows]
    s = np.asarray(s, dtype=np.float32)[:, rows]
    return e4m3_decode(q) * np.repeat(s.T.astype(np.float64), GROUP, axis=1)


def _rows_blocks(q, s, rows):
    q = np.asarray(q, dtype=np.uint8)[rows]
    s = np.asarray(s, dtype=np.float32).astype(np.float64)[np.asarray(rows) // GROUP]
    return e4m3_decode(q) * np.repeat(s, GROUP, axis=1)


def _cols_blocks(q, s, cols):
    """Columns `cols` of a 128x128-blocked [N, K] weight -> f64 [N, len(cols)]."""
    q = np.asarray(q, dtype=np.uint8)[:, cols]
    s = np.asarray(s, dtype=np.float32).astype(np.float64)[:, np.asarray(cols) // GROUP]
    return e4m3_decode(q) * np.repeat(s, GROUP, axis=0)


def gemm_fprop_ref_at(qx, sx, qw, sw, rows, cols):
    """Y64[rows][:, cols] without forming the whole product."""
    return _rows_groups(qx, sx, rows) @ _rows_blocks(qw, sw, cols).T


def gemm_dgrad_ref_at(qdy, sdy, qw, sw, rows, cols):
    """dX64[rows][:, cols]."""
    return _rows_groups(qdy, sdy, rows) @ _cols_blocks(qw, sw, cols)


def gemm_wgrad_ref_at(qdyt, sdyt, qxt, sxt, rows, cols):
    """dW64[rows][:, cols]."""
    return _rows_groups(qdyt, sdyt, rows) @ _rows_groups(qxt, sxt, cols).T


def f64_to_bf16_bits(y):
    """fp64 -> fp32 (nearest even) -> bf16 (nearest even), as uint16 bits."""
    f = np.asarray(y, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(u):
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_ulp(y):
    """Spacing of bf16 numbers at |y|: 2**(max(floor(log2|y|), -126) - 7)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126.0), -126.0)
    return np.exp2(e - 7.0)


def check_gemm(y_bf16, yref64, rms=None, norm_tol=1e-3, elem_tol=1e-3):
    """Acceptance check of a bf16 GEMM result against the fp64 reference.

    ``rms`` defaults to rms(yref64); pass the full-tensor rms when checking a
    sample of entries.  Returns a dict with the two measured errors and 'ok'.
    """
    y = bf16_bits_to_f64(y_bf16)
    ref = np.asarray(yref64, dtype=np.float64)
    assert y.shape == ref.shape
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    ref_norm = float(np.linalg.norm(ref))
    if ref_norm == 0.0:
        ok = bool(np.all(y == 0.0))
        return {"ok": ok, "normwise": 0.0 if ok else float("inf"), "elem_excess": 0.0 if ok else float("inf")}
    ref_b = bf16_bits_to_f64(f64_to_bf16_bits(ref))
    normwise = float(np.linalg.norm(y - ref_b) / ref_norm)
    bound = bf16_ulp(ref_b) + elem_tol * rms
    excess = float(np.max(np.abs(y - ref_b) - bound)) if y.size else -1.0
    ok = normwise <= norm_tol and excess <= 0.0
    return {"ok": bool(ok), "normwise": normwise, "elem_excess": excess}


def check_gemm_f32(y_f32, yref64, contrib64=None, rms=None, norm_tol=1e-3, elem_tol=1e-3):
    """Acceptance check of an fp32 GEMM result (the weight gradient kept in fp32).

    The pages fix no output precision for it.  The fp32 result is the GEMM's
    accumulator before the bf16 rounding, so it is held to the bf16 result's
    bound, measured against the unrounded reference: normwise
    ||Y - Yref64|| / ||G64|| <= 1e-3 and elementwise
    |Y - Yref64| <= ulp_bf16(G64) + 1e-3 * rms(G64) + 2**-23 * |Yref64|.
    (The MFMA's own accumulation of a 128-deep block is not exact, so the
    accumulator is no more accurate than that; the last term covers the
    rounding of an addition to an existing value.)  G64 is the product itself:
    ``yref64``, or ``contrib64`` when the result was added to an existing value
    (``yref64`` then being that value plus G64).  An all-zero product requires
    Y == Yref64 exactly.
    """
    y = np.asarray(y_f32, dtype=np.float32).astype(np.float64)
    ref = np.asarray(yref64, dtype=np.float64)
    g = ref if contrib64 is None else np.asarray(contrib64, dtype=np.float64)
    assert y.shape == ref.shape == g.shape
    if rms is None:
        rms = float(np.sqrt(np.mean(g * g))) if g.size else 0.0
    g_norm = float(np.linalg.norm(g))
    if g_norm == 0.0:
        ok = bool(np.all(y == ref))
        return {"ok": ok, "normwise": 0.0 if ok else float("inf"), "elem_excess": 0.0 if ok else float("inf")}
    normwise = float(np.linalg.norm(y - ref) / g_norm)
    bound = bf16_ulp(g) + elem_tol * rms + 2.0 ** -23 * np.abs(ref)
    excess = float(np.max(np.abs(y - ref) - bound)) if y.size else -1.0
    ok = normwise <= norm_tol and excess <= 0.0
    return {"ok": bool(ok), "normwise": normwise, "elem_excess": excess}
