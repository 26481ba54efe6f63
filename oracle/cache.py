"""Paged cache addressing for 352-byte rows (plain byte arithmetic, no blocking).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Changing the layout to reduce fragmentation": the cache is paged in blocks of 64
tokens; with the block-major layout a block holds the rows of several layers side by side. A page
is therefore addressed through a byte stride (``page_stride``) that is at least 64 rows and, in
the block-major case, covers all layers of the block.

Readings: a physical slot is ``page * 64 + offset``; its row starts at byte
``page * page_stride + offset * 352``. A logical position ``j`` of request ``b`` lives in page
``block_table[b][j // 64]`` at offset ``j % 64``. Slot ``-1`` means "do not write".
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import ROW_BYTES

PAGE_ROWS = 64


def row_offset(slot: int, page_stride: int) -> int:
    """Byte offset of physical slot ``slot`` in a cache whose pages are ``page_stride`` bytes."""
    page, off = divmod(int(slot), PAGE_ROWS)
    return page * int(page_stride) + off * ROW_BYTES


def write_rows(cache: np.ndarray, page_stride: int, slots, rows) -> None:
    """Store each 352-byte row at its slot (in place). Slots equal to -1 are skipped."""
    rows = np.asarray(rows, dtype=np.uint8)
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        o = row_offset(slot, page_stride)
        cache[o:o + ROW_BYTES] = rows[i]


def logical_slot(block_table_row, position: int) -> int:
    """Physical slot of logical position ``position`` through one request's block table."""
    return int(block_table_row[position // PAGE_ROWS]) * PAGE_ROWS + position % PAGE_ROWS


def read_rows(cache: np.ndarray, page_stride: int, block_table_row, positions) -> np.ndarray:
    """Gather the 352-byte rows of the given logical positions of one request."""
    positions = np.asarray(positions).tolist()
    out = np.empty((len(positions), ROW_BYTES), dtype=np.uint8)
    for i, j in enumerate(positions):
        o = row_offset(logical_slot(block_table_row, j), page_stride)
        out[i] = cache[o:o + ROW_BYTES]
    return out
