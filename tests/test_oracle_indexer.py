"""Pins of the indexer-score oracle (``oracle.indexer``) to hand-computed values and invariants.

The reading pinned: score[t, s] = c_s * sum_j w_{t,j} * max(0, q_{t,j} . k_s) over E4M3 keys and
queries, positions 0 .. seq_len - q_len + t, pages of 64 keys (128 bytes each) then 64 fp32 scales.
"""

import numpy as np
import pytest

from oracle import indexer as oi
from oracle import topk as ot

# E4M3 bytes of a few exact values (OCP OFP8: bias 7, 3 mantissa bits)
ONE = 0x38        # 1.0
ONE_HALF = 0x3C   # 1.5
HALF = 0x30       # 0.5
TWO = 0x40        # 2.0
NEG_ONE_HALF = 0xBC


def _cache(n_pages, keys, scales):
    """Pages holding keys uint8 [n_pages*64, 128] and scales [n_pages*64] (float32)."""
    c = np.zeros(n_pages * oi.PAGE_BYTES, dtype=np.uint8)
    for p in range(n_pages):
        base = p * oi.PAGE_BYTES
        c[base:base + 64 * 128] = keys[64 * p:64 * (p + 1)].reshape(-1)
        c[base + oi.SCALE_OFF:base + oi.PAGE_BYTES] = np.asarray(scales[64 * p:64 * (p + 1)], dtype="<f4").view(np.uint8)
    return c


def _hand_case():
    keys = np.zeros((64, 128), dtype=np.uint8)
    keys[5, 0] = ONE_HALF          # k_5 = 1.5 e_0
    keys[6, 0] = NEG_ONE_HALF      # k_6 = -1.5 e_0
    keys[7, 1] = TWO               # k_7 = 2 e_1
    scales = np.full(64, 0.25, dtype=np.float32)
    q = np.zeros((1, 1, 64, 128), dtype=np.uint8)
    q[0, 0, 3, 0] = ONE            # head 3 = e_0
    q[0, 0, 7, 0] = HALF           # head 7 = 0.5 e_0
    q[0, 0, 9, 1] = ONE_HALF       # head 9 = 1.5 e_1
    w = np.zeros((1, 1, 64))
    w[0, 0, 3], w[0, 0, 7], w[0, 0, 9] = 2.0, -1.0, 0.5
    return _cache(1, keys, scales), q, w


def test_hand_worked_scores():
    cache, q, w = _hand_case()
    s, vis = oi.indexer_scores(q, w, cache, oi.PAGE_BYTES, np.array([[0]]), [64], 64)
    assert vis.all()
    # position 5: 0.25 * (2 * max(0, 1.5) + (-1) * max(0, 0.75)) = 0.25 * 2.25
    assert s[0, 0, 5] == 0.5625
    # position 6: every head score is <= 0, so the ReLU leaves nothing
    assert s[0, 0, 6] == 0.0
    # position 7: 0.25 * 0.5 * max(0, 1.5 * 2)
    assert s[0, 0, 7] == 0.375
    # every other position has a zero key
    others = np.delete(s[0, 0], [5, 6, 7])
    assert np.all(others == 0.0)


def test_relu_is_per_head():
    """A negative head score is clipped before the weights combine the heads: with the head
    weights of opposite sign, the two heads do not cancel."""
    keys = np.zeros((64, 128), dtype=np.uint8)
    keys[0, 0] = ONE
    q = np.zeros((1, 1, 64, 128), dtype=np.uint8)
    q[0, 0, 0, 0] = ONE            # +1
    q[0, 0, 1, 0] = 0xB8           # -1
    w = np.zeros((1, 1, 64))
    w[0, 0, 0], w[0, 0, 1] = 1.0, 1.0
    s, _ = oi.indexer_scores(q, w, _cache(1, keys, np.ones(64, np.float32)), oi.PAGE_BYTES, np.array([[0]]), [64], 64)
    assert s[0, 0, 0] == 1.0       # max(0, 1) + max(0, -1), not 1 + (-1)


def test_visible_window_is_causal():
    cache, q, w = _hand_case()
    q3 = np.repeat(q, 3, axis=1)
    w3 = np.repeat(w, 3, axis=1)
    s, vis = oi.indexer_scores(q3, w3, cache, oi.PAGE_BYTES, np.array([[0]]), [10], 64)
    assert [int(vis[0, t].sum()) for t in range(3)] == [8, 9, 10]
    assert [ot.visible_count(10, 3, t) for t in range(3)] == [8, 9, 10]
    assert s[0, 0, 5] == 0.5625 and s[0, 0, 8] == 0.0 and not vis[0, 0, 8]


def test_paging_invariance_and_unmapped_pages():
    """The same logical keys placed in other physical pages score the same; the positions of an
    unmapped page score 0."""
    rng = np.random.default_rng(3)
    n = 4 * 64
    keys = rng.integers(0, 256, size=(n, 128), dtype=np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0                        # no NaN codes
    scales = rng.uniform(0.5, 1.5, n).astype(np.float32)
    q = rng.integers(0, 256, size=(1, 2, 64, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    w = rng.normal(size=(1, 2, 64))
    ident = _cache(4, keys, scales)
    a, _ = oi.indexer_scores(q, w, ident, oi.PAGE_BYTES, np.array([[0, 1, 2, 3]]), [n], n)
    perm = [2, 0, 3, 1]                                    # logical page i in physical perm[i]
    phys_keys = np.zeros_like(keys)
    phys_scales = np.zeros_like(scales)
    for i, p in enumerate(perm):
        phys_keys[64 * p:64 * (p + 1)] = keys[64 * i:64 * (i + 1)]
        phys_scales[64 * p:64 * (p + 1)] = scales[64 * i:64 * (i + 1)]
    wide = 9000                                            # a page stride above the page size
    c = np.zeros(4 * wide, dtype=np.uint8)
    packed = _cache(4, phys_keys, phys_scales)
    for p in range(4):
        c[p * wide:p * wide + oi.PAGE_BYTES] = packed[p * oi.PAGE_BYTES:(p + 1) * oi.PAGE_BYTES]
    b, _ = oi.indexer_scores(q, w, c, wide, np.array([perm]), [n], n)
    assert np.array_equal(a, b)
    assert np.any(a != 0)
    u, _ = oi.indexer_scores(q, w, c, wide, np.array([[perm[0], -1, perm[2], 7]]), [n], n)
    assert np.all(u[:, :, 64:128] == 0) and np.all(u[:, :, 192:] == 0)   # unmapped; page 7 outside
    assert np.array_equal(u[:, :, :64], a[:, :, :64])


def test_linear_in_weights_and_key_scale():
    rng = np.random.default_rng(4)
    keys = rng.integers(0, 0x70, size=(64, 128), dtype=np.uint8)   # finite positive and negative codes
    keys |= (rng.integers(0, 2, size=keys.shape) << 7).astype(np.uint8)
    q = rng.integers(0, 0x70, size=(1, 1, 64, 128), dtype=np.uint8)
    w1, w2 = rng.normal(size=(1, 1, 64)), rng.normal(size=(1, 1, 64))
    sc = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    bt = np.array([[0]])
    s1, _ = oi.indexer_scores(q, w1, _cache(1, keys, sc), oi.PAGE_BYTES, bt, [64], 64)
    s2, _ = oi.indexer_scores(q, w2, _cache(1, keys, sc), oi.PAGE_BYTES, bt, [64], 64)
    s12, _ = oi.indexer_scores(q, w1 + w2, _cache(1, keys, sc), oi.PAGE_BYTES, bt, [64], 64)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-12, atol=1e-9)
    s_twice, _ = oi.indexer_scores(q, w1, _cache(1, keys, 2 * sc), oi.PAGE_BYTES, bt, [64], 64)
    assert np.array_equal(s_twice, 2 * s1)                 # scaling by 2 is exact


@pytest.mark.parametrize("pos", [0, 5, 63])
def test_single_head_single_dim_is_a_product(pos):
    """With one head and one nonzero dim the score is c * w * max(0, q_d * k_d) for every code
    pair: checked over all finite E4M3 pairs of a few codes against the value table."""
    codes = [0x00, 0x01, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xB8, 0xFE]
    vals = {0x00: 0.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5, 0x7E: 448.0,
            0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for qc in codes:
        for kc in codes:
            keys = np.zeros((64, 128), dtype=np.uint8)
            keys[pos, 17] = kc
            q = np.zeros((1, 1, 64, 128), dtype=np.uint8)
            q[0, 0, 40, 17] = qc
            w = np.zeros((1, 1, 64))
            w[0, 0, 40] = -0.75
            s, _ = oi.indexer_scores(q, w, _cache(1, keys, np.full(64, 0.5, np.float32)), oi.PAGE_BYTES,
                                     np.array([[0]]), [64], 64)
            assert s[0, 0, pos] == 0.5 * -0.75 * max(0.0, vals[qc] * vals[kc])
