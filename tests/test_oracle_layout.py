"""Pins of the oracle's multi-layer page layouts against NumPy's own array indexing and closed
forms of the transfer descriptor counts.

Pins: a block-major pool is a C-ordered array [pool_blocks][n_layers][page], a layer-major pool
an array [n_layers][pool_blocks][page]; NumPy's reshape views give the page of (block, layer)
independently of the oracle's offset formulas. Descriptor counts: n_blocks regions for a
block-major transfer of non-adjacent blocks, n_layers * n_blocks for layer-major, and a single
region for a run of consecutive block-major blocks.
"""

import numpy as np
import pytest

from oracle import layout as lo

P = 352 * 4          # small page for the tests (4 rows)


def _pool(blocks, layers, seed):
    return np.random.default_rng(seed).integers(0, 256, blocks * layers * P, dtype=np.uint8)


@pytest.mark.parametrize("layout", [lo.BLOCK_MAJOR, lo.LAYER_MAJOR])
def test_page_offsets_match_array_views(layout):
    nb, nl = 7, 5
    pool = _pool(nb, nl, 1)
    view = pool.reshape(nb, nl, P) if layout == lo.BLOCK_MAJOR else pool.reshape(nl, nb, P)
    for b in range(nb):
        for l in range(nl):
            o = lo.page_offset(layout, b, l, nl, P, nb)
            want = view[b, l] if layout == lo.BLOCK_MAJOR else view[l, b]
            assert np.array_equal(pool[o:o + P], want)


@pytest.mark.parametrize("layout", [lo.BLOCK_MAJOR, lo.LAYER_MAJOR])
def test_layer_view_is_a_paged_cache(layout):
    nb, nl = 6, 4
    pool = _pool(nb, nl, 2)
    view = pool.reshape(nb, nl, P) if layout == lo.BLOCK_MAJOR else pool.reshape(nl, nb, P)
    for l in range(nl):
        base, stride = lo.layer_view(layout, l, nl, P, nb)
        for b in range(nb):
            want = view[b, l] if layout == lo.BLOCK_MAJOR else view[l, b]
            assert np.array_equal(pool[base + b * stride:base + b * stride + P], want)


def test_descriptor_counts_closed_forms():
    nl, pool_blocks = 8, 100
    blocks = [3, 17, 40, 41, 90]          # 40 and 41 are neighbours
    bm = lo.transfer_regions(lo.BLOCK_MAJOR, blocks, nl, P, pool_blocks)
    lm = lo.transfer_regions(lo.LAYER_MAJOR, blocks, nl, P, pool_blocks)
    assert len(bm) == len(blocks) - 1                 # one region per block, 40+41 merged
    assert len(lm) == nl * (len(blocks) - 1)          # per layer, 40+41 adjacent in each layer
    assert sum(n for _, n in bm) == sum(n for _, n in lm) == len(blocks) * nl * P
    assert len(lo.transfer_regions(lo.BLOCK_MAJOR, range(10, 20), nl, P, pool_blocks)) == 1
    assert len(lo.transfer_regions(lo.LAYER_MAJOR, range(10, 20), nl, P, pool_blocks)) == nl


@pytest.mark.parametrize("layout", [lo.BLOCK_MAJOR, lo.LAYER_MAJOR])
def test_copy_blocks_moves_exactly_the_pages(layout):
    nl = 3
    src = _pool(9, nl, 3)
    dst = np.zeros(12 * nl * P, dtype=np.uint8)
    sb, db = [4, 0, 7], [11, 2, 5]
    lo.copy_blocks(src, dst, layout, nl, P, sb, db)
    sv = src.reshape(9, nl, P) if layout == lo.BLOCK_MAJOR else src.reshape(nl, 9, P)
    dv = dst.reshape(12, nl, P) if layout == lo.BLOCK_MAJOR else dst.reshape(nl, 12, P)
    touched = np.zeros(dst.size, dtype=bool)
    for s, d in zip(sb, db):
        for l in range(nl):
            a = sv[s, l] if layout == lo.BLOCK_MAJOR else sv[l, s]
            b = dv[d, l] if layout == lo.BLOCK_MAJOR else dv[l, d]
            assert np.array_equal(a, b)
            o = lo.page_offset(layout, d, l, nl, P, 12)
            touched[o:o + P] = True
    assert not dst[~touched].any()
