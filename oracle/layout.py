"""Multi-layer KV page layouts and block transfer (plain byte arithmetic, NumPy slicing).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Changing the layout to reduce fragmentation": in the layer-major layout (LBHNC)
each layer's cache is stored on its own, so moving one logical block between engines needs one
descriptor per layer; the block-major layout (BLHNC) keeps the data of all layers of a block
next to each other, so a block moves as one contiguous region. Blocks are 64 tokens.

Readings (the page gives no byte formula):

* a pool holds ``pool_blocks`` blocks of ``n_layers`` layer pages of ``page_bytes`` each
  (one 64-row page of one layer: 64 * 352 bytes for NVFP4 rows);
* block-major: page (block b, layer l) starts at ``(b * n_layers + l) * page_bytes``;
* layer-major: page (block b, layer l) starts at ``(l * pool_blocks + b) * page_bytes``;
* a transfer descriptor is one contiguous byte range; the ranges a set of blocks needs are the
  pages of those blocks, with touching ranges merged.
"""

from __future__ import annotations

import numpy as np

BLOCK_MAJOR = 0          # BLHNC
LAYER_MAJOR = 1          # LBHNC


def page_offset(layout: int, block: int, layer: int, n_layers: int, page_bytes: int,
                pool_blocks: int) -> int:
    """Byte offset of the page of (block, layer) in a pool."""
    if layout == BLOCK_MAJOR:
        return (int(block) * n_layers + int(layer)) * page_bytes
    if layout == LAYER_MAJOR:
        return (int(layer) * pool_blocks + int(block)) * page_bytes
    raise ValueError("unknown layout")


def layer_view(layout: int, layer: int, n_layers: int, page_bytes: int, pool_blocks: int):
    """(base offset, page stride) under which one layer of a pool is an ordinary paged cache."""
    if layout == BLOCK_MAJOR:
        return layer * page_bytes, n_layers * page_bytes
    return layer * pool_blocks * page_bytes, page_bytes


def transfer_regions(layout: int, blocks, n_layers: int, page_bytes: int, pool_blocks: int):
    """Contiguous byte ranges (start, length) covering every page of the given blocks, in order of
    start, touching ranges merged."""
    spans = sorted(page_offset(layout, b, l, n_layers, page_bytes, pool_blocks)
                   for b in np.asarray(blocks).tolist() for l in range(n_layers))
    regions = []
    for s in spans:
        if regions and regions[-1][0] + regions[-1][1] == s:
            regions[-1][1] += page_bytes
        else:
            regions.append([s, page_bytes])
    return [tuple(r) for r in regions]


def copy_blocks(src, dst, layout: int, n_layers: int, page_bytes: int, src_blocks, dst_blocks):
    """dst gets, for every i and layer, the page of (src_blocks[i], layer) of src at the page of
    (dst_blocks[i], layer). Pool block counts follow from the array sizes."""
    src_pool = src.size // (n_layers * page_bytes)
    dst_pool = dst.size // (n_layers * page_bytes)
    for sb, db in zip(np.asarray(src_blocks).tolist(), np.asarray(dst_blocks).tolist()):
        for l in range(n_layers):
            so = page_offset(layout, sb, l, n_layers, page_bytes, src_pool)
            do = page_offset(layout, db, l, n_layers, page_bytes, dst_pool)
            dst[do:do + page_bytes] = src[so:so + page_bytes]
