"""Shared-row sparse decode (each distinct row of a group of up to 4 query tokens gathered and
decoded once) against the fp64 oracle, which computes the plain per-token softmax over each
token's own list: the shared path must give the same result.

Lists come from the overlap model ``workloads.gen_topk_overlap`` (the tokens of a request keep a
share of one base set), from independent draws, and with -1 entries; groups of 1 to 4 tokens
(q_len 1, 5, 7, 15); 16 and 32 heads; the full-size MTP shape at 16 heads per token.
"""

import numpy as np
import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _run(case, tokens=None, what="shared"):
    m = _m()
    out, lse = m.mla_sparse_decode_shared(case.q, case.cache, case.page_stride, case.block_table,
                                          case.topk_idx, th.softmax_scale())
    torch.cuda.synchronize()
    idx = case.topk_idx.cpu().numpy()
    if tokens is None:
        tokens = [(b, t) for b in range(case.B) for t in range(case.q_len)]
    need = {}
    for b, t in tokens:
        need.setdefault(b, set()).update(int(j) for j in idx[b, t] if j >= 0)
    ref_o, ref_l = th.oracle_sparse(case, tokens=tokens, cache=th.oracle_cache(case, need))
    w = th.assert_parity(out, lse, ref_o, ref_l, tokens=tokens, what=what)
    splits = m.mla_shared_decode_num_splits(case.B, case.q_len, case.H, case.topk)
    print(f"{what}: splits={splits} worst row err {w[0]:.2e} lse {w[1]:.2e}", flush=True)
    return out, lse


@pytest.mark.parametrize("q_len,H,overlap", [(7, 16, 0.5), (5, 32, 0.9), (1, 16, 0.0), (15, 16, 0.9)])
def test_shared_matches_oracle_overlap_lists(q_len, H, overlap):
    ctx = [3000, 5000]
    print(f"case: shared B=2 q_len={q_len} H={H} overlap={overlap} ctx={ctx} k=256", flush=True)
    case = th.build_case(2, q_len, H, ctx, 256, seed=2201 + q_len,
                         topk_fn=lambda B, q, k, c, s, d: wl.gen_topk_overlap(B, q, k, c, overlap, s, d))
    _run(case, what=f"shared q_len={q_len} H={H} overlap={overlap}")


def test_shared_independent_lists_with_empty_entries():
    """Independent lists (little sharing), -1 entries scattered, one token with an empty list and
    contexts shorter than k (lists padded with -1)."""
    ctx = [700, 4000, 1500]
    case = th.build_case(3, 6, 16, ctx, 1024, seed=2210)
    idx = case.topk_idx.clone()
    g = torch.Generator(device="cpu").manual_seed(9)
    drop = torch.rand(idx.shape, generator=g) < 0.2
    idx[drop.to(idx.device)] = -1
    idx[1, 3] = -1                                          # an empty list
    case.topk_idx = idx.contiguous()
    out, lse = _run(case, what="shared independent lists")
    assert torch.all(out[1, 3] == 0) and torch.all(torch.isneginf(lse[1, 3]))


def test_shared_equals_plain_path_closely():
    """The shared and the per-token paths compute the same softmax; they differ only by FP16
    rounding of probabilities under different running maxima (each within the parity bar)."""
    m = _m()
    case = th.build_case(2, 4, 16, [6000, 6000], 2048, seed=2211,
                         topk_fn=lambda B, q, k, c, s, d: wl.gen_topk_overlap(B, q, k, c, 0.8, s, d))
    a_o, a_l = m.mla_sparse_decode_shared(case.q, case.cache, case.page_stride, case.block_table,
                                          case.topk_idx, th.softmax_scale())
    b_o, b_l = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                   case.topk_idx, th.softmax_scale())
    torch.cuda.synchronize()
    ref = b_o.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    assert float(((a_o - b_o).abs() / ref).max()) < 2e-3
    assert float((a_l - b_l).abs().max()) < 2e-3
    a2_o, _ = m.mla_sparse_decode_shared(case.q, case.cache, case.page_stride, case.block_table,
                                         case.topk_idx, th.softmax_scale())
    torch.cuda.synchronize()
    assert torch.equal(a_o, a2_o), "the shared path is not deterministic"


def test_shared_rejects_long_block_tables_and_small_workspace():
    m = _m()
    case = th.build_case(1, 2, 16, [1000], 64, seed=2212)
    wide = torch.zeros(1, 16385, dtype=torch.int32, device="cuda")   # 1,048,640 positions
    wide[0, :case.block_table.shape[1]] = case.block_table[0]
    with pytest.raises(m.MlaError, match="UNSUPPORTED"):
        m.mla_sparse_decode_shared(case.q, case.cache, case.page_stride, wide, case.topk_idx,
                                   th.softmax_scale())
    with pytest.raises(m.MlaError, match="WORKSPACE"):
        m.mla_sparse_decode_shared(case.q, case.cache, case.page_stride, case.block_table,
                                   case.topk_idx, th.softmax_scale(),
                                   workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))


def test_shared_mtp_shape_16_heads_overlap_0_9():
    """The MTP shape at 16 heads per token (B=16, q_len=15, 149,504-token contexts, top-k 2048),
    lists under the overlap model at 0.9; every token of two requests against the oracle."""
    print("case: shared MTP B=16 q_len=15 H=16 overlap=0.9", flush=True)
    case = th.build_case(16, 15, 16, [149504] * 16, 2048, seed=2213, spare_pages=0,
                         topk_fn=lambda B, q, k, c, s, d: wl.gen_topk_overlap(B, q, k, c, 0.9, s, d))
    _run(case, tokens=[(b, t) for b in (0, 11) for t in range(15)], what="shared MTP H=16")
