"""Pins of the oracle's fp64 sparse / dense decode against closed forms and invariants.

Every expected value here comes from a closed form on hand-chosen grid values, from an invariance
the definition implies, or from a brute-force sum on a tiny case; none re-runs the oracle's own
code path to produce the expectation.
"""

import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc
from oracle import nvfp4 as nv


def _rand_rows(rng, n):
    x = rng.standard_normal((n, 512)).astype(np.float32).astype(np.float64)
    r = rng.standard_normal((n, 64)).astype(np.float32).astype(np.float64)
    return nv.quantize_rows(x, r)


def _build_cache(rng, ctx, page_stride=64 * 352, shuffle=True):
    """Cache of one request with ctx rows placed through a random (or identity) block table."""
    pages = (ctx + 63) // 64
    perm = rng.permutation(pages) if shuffle else np.arange(pages)
    cache = np.zeros(pages * page_stride, dtype=np.uint8)
    rows = _rand_rows(rng, ctx)
    slots = [oc.logical_slot(perm, j) for j in range(ctx)]
    oc.write_rows(cache, page_stride, slots, rows)
    return cache, perm[None, :], rows


def _grid_row(latent_vals, rope_vals):
    """A row whose values are exactly representable (checked), so dequantize gives them back."""
    row = nv.quantize_rows(np.asarray(latent_vals)[None], np.asarray(rope_vals)[None])
    lat, rp = nv.dequantize_rows(row)
    assert np.array_equal(lat[0], latent_vals) and np.array_equal(rp[0], rope_vals)
    return row[0]


def test_uniform_scores_give_mean_and_log_count():
    rng = np.random.default_rng(1)
    cache, bt, rows = _build_cache(rng, 300)
    q = np.zeros((1, 1, 4, 576))
    sel = rng.choice(300, size=37, replace=False)
    idx = np.full((1, 1, 64), -1)
    idx[0, 0, :37] = sel
    out, lse = oa.sparse_decode(q, cache, 64 * 352, bt, idx, 0.125)
    lat, _ = nv.dequantize_rows(rows[sel])
    mean = np.sum(lat, axis=0) / 37
    assert np.allclose(out[0, 0], mean[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse[0, 0], math.log(37), rtol=0, atol=1e-12)


def test_single_token_returns_its_latent_and_score():
    # row with hand-set grid values: latent = 1.5 everywhere in group 0, rope = 2.0
    lat = np.zeros(512)
    lat[:16] = 1.5
    lat[16:32] = -6.0
    rope = np.full(64, 2.0)
    row = _grid_row(lat, rope)
    cache = np.zeros(64 * 352, dtype=np.uint8)
    oc.write_rows(cache, 64 * 352, [5], row[None])
    q = np.zeros((1, 1, 2, 576))
    q[0, 0, 0, :16] = 1.0            # head 0 score = 0.5 * (16 * 1.5)
    q[0, 0, 1, 512:] = -1.0          # head 1 score = 0.5 * (-64 * 2)
    idx = np.array([[[5, -1, -1]]])
    out, lse = oa.sparse_decode(q, cache, 64 * 352, np.array([[0]]), idx, 0.5)
    assert np.array_equal(out[0, 0, 0], lat) and np.array_equal(out[0, 0, 1], lat)
    assert lse[0, 0, 0] == 0.5 * 24.0 and lse[0, 0, 1] == -64.0


def test_two_rows_closed_form_uses_rope_and_latent():
    """Hand-built rows: softmax weights follow exp(scale * (latent dot + rope dot))."""
    # every group holds an element equal to 6*s for an E4M3 s, so all values are on the grid
    la = np.zeros(512); la[:16] = 1.0; la[0] = 1.5; la[100] = 0.75
    lb = np.zeros(512); lb[16:32] = -2.0; lb[16] = -3.0; lb[200] = 3.0
    ra = np.zeros(64); ra[0] = 1.0
    rb = np.zeros(64); rb[0] = -1.5
    cache = np.zeros(64 * 352, dtype=np.uint8)
    oc.write_rows(cache, 64 * 352, [0, 1], np.stack([_grid_row(la, ra), _grid_row(lb, rb)]))
    q = np.zeros((1, 1, 1, 576))
    q[0, 0, 0, 0] = 0.25          # latent: a -> 0.375, b -> 0
    q[0, 0, 0, 16] = 0.5          # latent: a -> 0, b -> -1.5
    q[0, 0, 0, 512] = 2.0         # rope:   a -> 2.0, b -> -3.0
    scale = 0.75
    sa = scale * (0.375 + 2.0)
    sb = scale * (-1.5 - 3.0)
    wa, wb = math.exp(sa), math.exp(sb)
    expect = (wa * la + wb * lb) / (wa + wb)
    out, lse = oa.sparse_decode(q, cache, 64 * 352, np.array([[0]]), np.array([[[1, 0]]]), scale)
    assert np.allclose(out[0, 0, 0], expect, rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(wa + wb)) < 1e-13


def test_topk_all_equals_dense():
    rng = np.random.default_rng(2)
    ctx = 200
    cache, bt, _ = _build_cache(rng, ctx)
    q = rng.standard_normal((1, 1, 3, 576))
    idx = rng.permutation(ctx)[None, None, :]
    o1, l1 = oa.sparse_decode(q, cache, 64 * 352, bt, idx, 0.06)
    o2, l2 = oa.dense_decode(q, cache, 64 * 352, bt, [ctx], 0.06)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_padding_permutation_and_paging_invariance():
    rng = np.random.default_rng(3)
    ctx = 330
    cache, bt, rows = _build_cache(rng, ctx)
    # the same logical rows placed through the identity page table
    cache_id = np.zeros_like(cache)
    bt_id = np.arange(bt.shape[1])[None, :]
    oc.write_rows(cache_id, 64 * 352, [oc.logical_slot(bt_id[0], j) for j in range(ctx)], rows)
    q = rng.standard_normal((1, 1, 2, 576))
    sel = rng.choice(ctx, size=50, replace=False)
    idx = np.full((1, 1, 80), -1)
    idx[0, 0, rng.choice(80, size=50, replace=False)] = sel
    base_o, base_l = oa.sparse_decode(q, cache, 64 * 352, bt, sel[None, None, :], 0.05)
    for variant in (idx, rng.permutation(sel)[None, None, :]):
        o, l = oa.sparse_decode(q, cache, 64 * 352, bt, variant, 0.05)
        assert np.allclose(o, base_o, rtol=0, atol=1e-12)
        assert np.allclose(l, base_l, rtol=0, atol=1e-12)
    o, l = oa.sparse_decode(q, cache_id, 64 * 352, bt_id, sel[None, None, :], 0.05)
    assert np.allclose(o, base_o, rtol=0, atol=1e-12)


def test_empty_list_gives_zero_and_minus_inf():
    cache = np.zeros(64 * 352, dtype=np.uint8)
    q = np.ones((1, 1, 2, 576))
    out, lse = oa.sparse_decode(q, cache, 64 * 352, np.array([[0]]), np.full((1, 1, 8), -1), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(4)
    ctx = 500
    cache, bt, rows = _build_cache(rng, ctx)
    q = rng.standard_normal((1, 1, 4, 576)) * 3
    idx = rng.permutation(ctx)[:257]
    full_o, full_l = oa.sparse_decode(q, cache, 64 * 352, bt, idx[None, None], 0.1)
    for n_split in (2, 3, 8):
        parts = []
        for chunk in np.array_split(idx, n_split):
            k, v = oa.rows_to_kv(oc.read_rows(cache, 64 * 352, bt[0], chunk))
            parts.append(oa.attend(q[0, 0], k, v, 0.1))
        parts.append(oa.attend(q[0, 0], np.zeros((0, 576)), np.zeros((0, 512)), 0.1))  # empty split
        o, l = oa.lse_merge(parts)
        assert np.allclose(o, full_o[0, 0], rtol=0, atol=1e-12)
        assert np.allclose(l, full_l[0, 0], rtol=0, atol=1e-12)


def test_brute_force_tiny_sum():
    """Attention of one head over three rows by explicit scalar sums (math.fsum)."""
    rng = np.random.default_rng(5)
    cache, bt, rows = _build_cache(rng, 64, shuffle=False)
    q = rng.standard_normal((1, 1, 1, 576))
    sel = [7, 40, 3]
    lat, rp = nv.dequantize_rows(rows[sel])
    scale = 0.04
    scores = [scale * math.fsum(q[0, 0, 0, i] * (lat[n, i] if i < 512 else rp[n, i - 512])
                                for i in range(576)) for n in range(3)]
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = math.fsum(w)
    expect = np.array([math.fsum(w[n] * lat[n, d] for n in range(3)) / tot for d in range(512)])
    out, lse = oa.sparse_decode(q, cache, 64 * 352, bt, np.array([[sel]]), scale)
    assert np.allclose(out[0, 0, 0], expect, rtol=1e-13, atol=1e-14)
    assert abs(lse[0, 0, 0] - (mx + math.log(tot))) < 1e-12


def test_dense_causal_window():
    rng = np.random.default_rng(6)
    ctx = 150
    cache, bt, _ = _build_cache(rng, ctx)
    q = rng.standard_normal((1, 3, 2, 576))
    o, l = oa.dense_decode(q, cache, 64 * 352, bt, [ctx], 0.05)
    for t in range(3):
        n_vis = ctx - 3 + t + 1
        os_, ls_ = oa.sparse_decode(q[:, t:t + 1], cache, 64 * 352, bt,
                                    np.arange(n_vis)[None, None], 0.05)
        assert np.allclose(o[0, t], os_[0, 0], rtol=0, atol=1e-12)
        assert np.allclose(l[0, t], ls_[0, 0], rtol=0, atol=1e-12)
    assert oa.dense_positions(10, 3, 0) == list(range(8))


def test_duplicates_count_twice():
    rng = np.random.default_rng(8)
    cache, bt, rows = _build_cache(rng, 64, shuffle=False)
    q = np.zeros((1, 1, 1, 576))
    out, lse = oa.sparse_decode(q, cache, 64 * 352, bt, np.array([[[3, 3, 9]]]), 1.0)
    lat, _ = nv.dequantize_rows(rows[[3, 9]])
    assert np.allclose(out[0, 0, 0], (2 * lat[0] + lat[1]) / 3, rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - math.log(3)) < 1e-14


def test_row_relative_error_hand_worked_rows():
    """The parity comparator on rows worked out by hand: max |out - ref| over the row divided by
    max |ref| over the row (the absolute error where the reference row is all zero); the result
    has one value per row of the leading axes, and a NaN anywhere in a row makes that row NaN."""
    out = np.array([[1.0, 2.0, 3.0],        # worst difference 1 at the last dim, max |ref| 4
                    [0.5, -1.0, 0.0],       # reference row all zero: absolute error 1
                    [1000.0, 3.0, 1.0],     # one large entry sets the denominator: 2 / 1000
                    [-1.0, 0.0, 0.0],       # sign flip: |-1 - 1| / 1
                    [np.nan, 1.0, 1.0],     # NaN propagates
                    [np.inf, 1.0, 1.0]])    # an infinite output gives an infinite error
    ref = np.array([[1.0, 2.0, 4.0],
                    [0.0, 0.0, 0.0],
                    [1000.0, 1.0, 1.0],
                    [1.0, 0.0, 0.0],
                    [1.0, 1.0, 1.0],
                    [1.0, 1.0, 1.0]])
    err = oa.row_relative_error(out, ref)
    assert err.shape == (6,)
    assert err[0] == 0.25 and err[1] == 1.0 and err[2] == 0.002 and err[3] == 2.0
    assert np.isnan(err[4]) and np.isposinf(err[5])
    # leading axes are kept: [2, 3, dims] -> [2, 3]
    e3 = oa.row_relative_error(np.zeros((2, 3, 5)), np.ones((2, 3, 5)))
    assert e3.shape == (2, 3) and np.all(e3 == 1.0)
