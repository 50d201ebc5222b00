"""Pins of the oracle's rollout-packed weight order (no GPU).

The order must hand every lane of a 64-lane wave the operand bytes that the
16x16x128 FP8 matrix instruction takes from it: lane l holds 32 consecutive
K-elements of operand row l mod 16, starting at 32 (l div 16) within the
128-deep block (the instruction's operand layout, the same one the row-major
kernels load).  The first pin computes a product by reading the packed bytes
only through that lane model and compares it with the row-major product.
"""

import numpy as np
import pytest

import oracle


def lane_model_product(packed, n, k, x):
    """W x computed from the packed bytes: chunk (t, kb) at 2048 (t K/128 + kb);
    lane l's operand = bytes [16 l, 16 l + 16) and [1024 + 16 l, 1024 + 16 l + 16)
    of the chunk, the codes of row 16 t + l mod 16 at K = 128 kb + 32 (l div 16) + 0..31."""
    flat = np.asarray(packed, np.uint8).reshape(-1)
    nkb = k // 128
    y = np.zeros(n, np.int64)
    for t in range(n // 16):
        for kb in range(nkb):
            chunk = flat[2048 * (t * nkb + kb): 2048 * (t * nkb + kb + 1)]
            for lane in range(64):
                frag = np.concatenate([chunk[16 * lane: 16 * lane + 16], chunk[1024 + 16 * lane: 1024 + 16 * lane + 16]])
                k0 = 128 * kb + 32 * (lane // 16)
                y[16 * t + lane % 16] += int(frag.astype(np.int64) @ x[k0: k0 + 32])
    return y


@pytest.mark.parametrize("n,k", [(16, 128), (32, 256), (48, 384)])
def test_lane_model_reads_the_row_major_product(n, k):
    rng = np.random.default_rng(n + k)
    qw = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    x = rng.integers(-1000, 1000, size=k).astype(np.int64)
    packed = oracle.pack_weight_rollout(qw)
    assert packed.shape == (n, k) and packed.dtype == np.uint8
    assert np.array_equal(lane_model_product(packed, n, k, x), qw.astype(np.int64) @ x)


def _pack_index_bytes(n, k, pack):
    """The packed position's source index (row * K + col), through the byte permutation."""
    idx = np.arange(n * k, dtype=np.int64).reshape(n, k)
    out = np.zeros(n * k, np.int64)
    for sh in (0, 8, 16, 24):
        out |= pack(((idx >> sh) & 255).astype(np.uint8)).reshape(-1).astype(np.int64) << sh
    return out


def test_permutation_and_chunks():
    n, k = 64, 512
    src = _pack_index_bytes(n, k, oracle.pack_weight_rollout)
    assert np.array_equal(np.sort(src), np.arange(n * k))       # every code exactly once
    rows, cols = src // k, src % k
    for c in range(n * k // 2048):                               # chunk c = (strip t, K-block kb)
        t, kb = divmod(c, k // 128)
        sl = slice(2048 * c, 2048 * (c + 1))
        assert set(rows[sl]) == set(range(16 * t, 16 * t + 16))
        assert set(cols[sl]) == set(range(128 * kb, 128 * kb + 128))


def test_transposed_lane_slip_fails_the_product_pin():
    """A copy with lane = 4 r + j (row-major lanes) instead of 16 j + r: the lane-model
    product differs, so the first pin catches that slip; so does swapping the halves."""
    def slip_lanes(qw):
        n, k = qw.shape
        v = np.asarray(qw, np.uint8).reshape(n // 16, 16, k // 128, 4, 2, 16)
        return np.ascontiguousarray(v.transpose(0, 2, 4, 1, 3, 5)).reshape(n, k)

    def slip_halves(qw):
        n, k = qw.shape
        v = np.asarray(qw, np.uint8).reshape(n // 16, 16, k // 128, 2, 4, 16)  # h outer of j
        return np.ascontiguousarray(v.transpose(0, 2, 3, 4, 1, 5)).reshape(n, k)

    rng = np.random.default_rng(3)
    n, k = 32, 256
    qw = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    x = rng.integers(-1000, 1000, size=k).astype(np.int64)
    ref = qw.astype(np.int64) @ x
    for slip in (slip_lanes, slip_halves):
        assert not np.array_equal(lane_model_product(slip(qw), n, k, x), ref), slip.__name__


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.pack_weight_rollout(np.zeros((24, 128), np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_weight_rollout(np.zeros((16, 200), np.uint8))
