"""The opt-in content checks (MLA_DEBUG_CHECKS): the host check functions on hand-made index
arrays (no GPU needed), and the switch. Each bad case names the entry the message must point at."""

import numpy as np
import pytest

import nvfp4_compressed_mla_amd as m
from nvfp4_compressed_mla_amd import _lib

PAGE = 64 * 352


def _bt():
    # two requests, 3 pages each, pages 0..5 of a 6-page cache; request 1's last column unmapped
    return np.array([[4, 0, 2], [1, 5, -1]], dtype=np.int32)


def test_good_sparse_lists_pass():
    idx = np.full((2, 2, 8), -1, dtype=np.int32)
    idx[0, 0, :3] = [0, 63, 191]
    idx[1, 1, :2] = [64, 127]
    m.mla_check_sparse_indices(idx, _bt(), PAGE, 6 * PAGE)


@pytest.mark.parametrize("b,t,s,val,msg", [
    (0, 1, 4, -2, "negative and not -1"),
    (1, 0, 0, 130, "unmapped"),                      # column 2 of request 1 is -1
    (0, 0, 7, 3 * 64, "beyond the block table"),
    (1, 1, 3, 1 << 30, "beyond the block table"),
])
def test_bad_sparse_entries_are_named(b, t, s, val, msg):
    idx = np.full((2, 2, 8), -1, dtype=np.int32)
    idx[b, t, s] = val
    with pytest.raises(m.MlaError, match=msg) as e:
        m.mla_check_sparse_indices(idx, _bt(), PAGE, 6 * PAGE)
    assert e.value.status == _lib.MLA_ERR_INVALID_ARG
    assert f"[{b}][{t}][{s}]" in str(e.value)


def test_sparse_row_outside_the_cache():
    idx = np.full((2, 1, 4), -1, dtype=np.int32)
    idx[0, 0, 0] = 40                                  # row 40 of page 4; the cache holds 4.5 pages
    with pytest.raises(m.MlaError, match="outside"):
        m.mla_check_sparse_indices(idx, _bt(), PAGE, 4 * PAGE + PAGE // 2)
    idx[0, 0, 0] = 64 + 5                              # page 0: inside
    m.mla_check_sparse_indices(idx, _bt(), PAGE, 4 * PAGE + PAGE // 2)
    # a page id whose offset is past 2^36 (and so past any cache the library accepts)
    bt = _bt()
    bt[0, 1] = (1 << 20) + 6
    idx[0, 0, 0] = 64
    with pytest.raises(m.MlaError, match="outside"):
        m.mla_check_sparse_indices(idx, bt, 65536, 9 * 65536)


def test_fp8_row_bytes_are_used():
    idx = np.full((1, 1, 2), -1, dtype=np.int32)
    idx[0, 0, 0] = 63                                  # last row of page 0
    bt = np.array([[0]], dtype=np.int32)
    m.mla_check_sparse_indices(idx, bt, 64 * 576, 64 * 576, row_bytes=576)
    with pytest.raises(m.MlaError, match="outside"):
        m.mla_check_sparse_indices(idx, bt, 64 * 576, 64 * 576 - 1, row_bytes=576)


def test_dense_tables():
    bt = _bt()
    m.mla_check_dense_tables([192, 128], 1, bt, PAGE, 6 * PAGE)
    m.mla_check_dense_tables([0, 1], 3, bt, PAGE, 6 * PAGE)            # empty windows are fine
    with pytest.raises(m.MlaError, match=r"seq_lens\[1\] = 129"):
        m.mla_check_dense_tables([192, 129], 1, bt, PAGE, 6 * PAGE)   # reaches the -1 page
    with pytest.raises(m.MlaError, match="negative"):
        m.mla_check_dense_tables([-1, 5], 1, bt, PAGE, 6 * PAGE)
    with pytest.raises(m.MlaError, match="exceeds the block table"):
        m.mla_check_dense_tables([193, 5], 1, bt, PAGE, 6 * PAGE)
    with pytest.raises(m.MlaError, match="outside"):
        m.mla_check_dense_tables([10, 5], 1, bt, PAGE, 4 * PAGE + 9 * 352)   # page 4, 10 rows


def test_slots():
    m.mla_check_slots([-1, 0, 6 * 64 - 1], PAGE, 6 * PAGE)
    with pytest.raises(m.MlaError, match=r"slot_mapping\[1\] = -5"):
        m.mla_check_slots([0, -5], PAGE, 6 * PAGE)
    with pytest.raises(m.MlaError, match=r"slot_mapping\[2\] = 384"):
        m.mla_check_slots([0, 1, 6 * 64], PAGE, 6 * PAGE)
    with pytest.raises(m.MlaError, match="outside"):
        m.mla_check_slots([1 << 62], PAGE, 6 * PAGE)


def test_switch():
    before = m.mla_debug_checks_enabled()
    try:
        m.mla_set_debug_checks(True)
        assert m.mla_debug_checks_enabled()
        m.mla_set_debug_checks(False)
        assert not m.mla_debug_checks_enabled()
    finally:
        m.mla_set_debug_checks(before)
