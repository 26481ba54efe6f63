"""Paged cache addressing for 352-byte NVFP4 rows (and 576-byte FP8 rows), plain byte arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Changing the layout to reduce fragmentation": the cache is paged in blocks of 64
tokens; with the block-major layout a block holds the rows of several layers side by side. A page
is therefore addressed through a byte stride (``page_stride``) that is at least 64 rows and, in
the block-major case, covers all layers of the block.

Readings: a physical slot is ``page * 64 + offset``; its row starts at byte
``page * page_stride + offset * 352`` (``offset * 576`` for FP8 rows). A logical position ``j`` of request ``b`` lives in page
``block_table[b][j // 64]`` at offset ``j % 64``. Slot ``-1`` means "do not write".
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import ROW_BYTES

PAGE_ROWS = 64


def row_offset(slot: int, page_stride: int, row_bytes: int = ROW_BYTES) -> int:
    """Byte offset of physical slot ``slot`` in a cache whose pages are ``page_stride`` bytes."""
    page, off = divmod(int(slot), PAGE_ROWS)
    return page * int(page_stride) + off * int(row_bytes)


def write_rows(cache: np.ndarray, page_stride: int, slots, rows) -> None:
    """Store each row (352-byte NVFP4 or 576-byte FP8) at its slot (in place). Slots equal to
    -1 are skipped."""
    rows = np.asarray(rows, dtype=np.uint8)
    row_bytes = rows.shape[1]
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        o = row_offset(slot, page_stride, row_bytes)
        cache[o:o + row_bytes] = rows[i]


def logical_slot(block_table_row, position: int) -> int:
    """Physical slot of logical position ``position`` through one request's block table."""
    page = int(block_table_row[position // PAGE_ROWS])
    if page < 0:
        raise ValueError(f"logical_slot: position {position} falls in an unmapped page")
    return page * PAGE_ROWS + position % PAGE_ROWS


def read_rows(cache: np.ndarray, page_stride: int, block_table_row, positions,
              row_bytes: int = ROW_BYTES) -> np.ndarray:
    """Gather the rows (``row_bytes`` each) of the given logical positions of one request."""
    positions = np.asarray(positions).tolist()
    out = np.empty((len(positions), row_bytes), dtype=np.uint8)
    for i, j in enumerate(positions):
        o = row_offset(logical_slot(block_table_row, j), page_stride, row_bytes)
        out[i] = cache[o:o + row_bytes]
    return out
