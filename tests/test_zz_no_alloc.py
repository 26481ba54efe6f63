"""The allocation-free sparse decode (``mla_sparse_decode_noalloc``), called through the C ABI
with raw pointers: on two calls in a row (the second with a smaller input) it must give the same
bits as ``mla_sparse_decode`` with a caller workspace, match the oracle, and allocate nothing
(torch's allocator is unchanged across the call). Sizes beyond its scratch array are rejected on
the host."""

import ctypes

import pytest
import torch

from nvfp4_compressed_mla_amd import _lib
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _raw_noalloc(case, splits, out, lse):
    lib = _lib.load_library()
    B, q_len, H, _ = case.q.shape
    st = lib.mla_sparse_decode_noalloc(
        ctypes.c_void_p(case.q.data_ptr()), _lib.MLA_BF16, ctypes.c_void_p(case.cache.data_ptr()),
        case.page_stride, case.cache.numel(), ctypes.c_void_p(case.block_table.data_ptr()),
        case.block_table.shape[1], ctypes.c_void_p(case.topk_idx.data_ptr()), case.topk_idx.shape[2],
        B, q_len, H, th.softmax_scale(), splits, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    import nvfp4_compressed_mla_amd as m
    cases = [
        ("first", th.build_case(4, 2, 64, [3000, 2500, 1800, 4100], 1024, seed=501), 4),
        ("second, smaller", th.build_case(2, 1, 32, [900, 1200], 256, seed=502), 2),
    ]
    scratch = _lib.load_library().mla_noalloc_scratch_bytes()
    assert scratch == 32 << 20
    for what, case, splits in cases:
        print(f"case: noalloc {what} B={case.B} q_len={case.q_len} H={case.H} splits={splits}", flush=True)
        B, q_len, H, _ = case.q.shape
        assert 0 < m.mla_decode_workspace_size(B * q_len, H, splits) <= scratch
        out = torch.full((B, q_len, H, 512), float("nan"), device="cuda")
        lse = torch.full((B, q_len, H), float("nan"), device="cuda")
        torch.cuda.synchronize()
        before = (torch.cuda.memory_allocated(), torch.cuda.memory_reserved())
        st = _raw_noalloc(case, splits, out, lse)
        torch.cuda.synchronize()
        assert st == _lib.MLA_OK, _lib.load_library().mla_last_error()
        assert (torch.cuda.memory_allocated(), torch.cuda.memory_reserved()) == before
        ref_out, ref_lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride,
                                               case.block_table, case.topk_idx, th.softmax_scale(),
                                               num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), what
        ro, rl = th.oracle_sparse(case)
        th.assert_parity(out, lse, ro, rl, what=f"noalloc {what}")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = _lib.load_library()
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: the size check comes first
    st = lib.mla_sparse_decode_noalloc(fake, 0, fake, 22528, 22528 * 64, fake, 64, fake, 2048,
                                       32, 15, 128, 0.04, 16, fake, fake, None)
    assert st == _lib.MLA_ERR_WORKSPACE
    assert b"scratch" in lib.mla_last_error()
