"""Rollout-packed order of the FP8 weight codes (oracle; TEST INFRASTRUCTURE ONLY).

The rollout runs the training forward's FP8 FProp (page
paper.rainbus.top/paper/2601.14243, sections "核心方法" and "方法步骤详情"
step 2); at rollout batch sizes that GEMM's cost is reading the weight
(section "独立分析的弱点").  The library can keep the quantised weight codes in
the order its rollout FProp reads them.  Codes, scales and arithmetic are
unchanged: the packed FProp's reference is gemm_fprop_ref on the unpacked
weight, and this module only states the byte order.

The order is the library's own definition (the pages fix no storage order for
the rollout engine), a byte permutation of qw [N][K]: for strip t (16 weight
rows), K-block kb (128 codes), half h, lane l (0..63) and byte b (0..15),

    packed[((t * K/128 + kb) * 2 + h) * 1024 + 16 l + b]
        = qw[16 t + (l mod 16)][128 kb + 32 (l div 16) + 16 h + b].

So each (strip, K-block) is one contiguous 2 KB chunk, and within it lane l
of a 64-lane wave finds, as two 16-byte pieces at 16 l and 1024 + 16 l, the 32
consecutive codes (row l mod 16, K-slice l div 16) that the 16x16x128 FP8
matrix instruction takes from that lane.

Pins (tests/test_oracle_layout.py): a product computed by reading the packed
bytes through that lane model equals the row-major product; the order is a
permutation, each chunk holds exactly its strip's K-block; a test-only copy with
the lane index transposed fails the product pin.
"""

import numpy as np


def pack_weight_rollout(qw):
    """uint8 [N, K] (N % 16 == 0, K % 128 == 0) -> uint8 [N, K] holding the packed order."""
    q = np.asarray(qw, dtype=np.uint8)
    n, k = q.shape
    if n % 16 or k % 128:
        raise ValueError(f"pack_weight_rollout: N % 16 and K % 128 must be 0, got {n} x {k}")
    # view row 16 t + r, column 128 kb + 32 j + 16 h + b as axes [t, r, kb, j, h, b] ...
    v = q.reshape(n // 16, 16, k // 128, 4, 2, 16)
    # ... and store them as [t, kb, h, lane = 16 j + r, b]
    return np.ascontiguousarray(v.transpose(0, 2, 4, 3, 1, 5)).reshape(n, k)
