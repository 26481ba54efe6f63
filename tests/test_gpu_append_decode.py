"""Quantize-append fused into the sparse decode (``mla_sparse_decode_append``).

The call must write the same cache bytes as ``mla_nvfp4_quantize_append`` and give the same
result as that append followed by ``mla_sparse_decode``: the two are compared bit for bit (the
decode arithmetic is the same; a list entry on a new row reads the workgroup's copy, encoded by
the same encoder). The outputs are also checked against the fp64 oracle, whose cache is its own
quantization of the bf16 rows, new rows included.

Before each call the new rows' slots hold stale rows (another row's encoding), so an entry that
read the cache instead of the new row would change the result. Lists hold history positions drawn
uniformly, plus the new positions a token may see (new row k for token t >= k), placed at the
start or at the end of the list so that both the first and the last split meet them.
"""

import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _lists_with_new_rows(B, q_len, topk, ctx, seed):
    """History positions of every token, with the new positions k <= t placed at list entries
    k (odd t) or topk - 1 - k (even t)."""
    hist = [c - q_len for c in ctx]
    idx = wl.gen_topk(B, q_len, topk, hist, seed, "cpu")
    for b in range(B):
        for t in range(q_len):
            for k in range(t + 1):
                idx[b, t, k if t % 2 else topk - 1 - k] = hist[b] + k
    return idx.cuda().contiguous()


def _setup(B, q_len, H, ctx, topk, seed):
    case = th.build_case(B, q_len, H, ctx, topk, seed)
    case.topk_idx = _lists_with_new_rows(B, q_len, topk, ctx, seed + 7)
    slots = torch.cat([wl.slot_mapping_for(case.block_table, b, c - q_len, q_len)
                       for b, c in enumerate(ctx)])
    rows = torch.cat([torch.arange(case.row_base[b] + c - q_len, case.row_base[b] + c, device="cuda")
                      for b, c in enumerate(ctx)])
    new_lat, new_rope = case.latent[rows].contiguous(), case.rope[rows].contiguous()
    good = case.cache.clone()                       # the cache with the new rows appended
    stale = case.cache.clone()                      # the new slots hold other rows
    other = torch.arange(rows.numel(), device="cuda")
    _m().mla_nvfp4_quantize_append(case.latent[other], case.rope[other], slots, stale, case.page_stride)
    return case, slots, new_lat, new_rope, good, stale


def _fused(case, cache, lat, rope, slots, num_splits=0, workspace=None):
    return _m().mla_sparse_decode_append(case.q, cache, case.page_stride, case.block_table,
                                         case.topk_idx, th.softmax_scale(), lat, rope, slots,
                                         num_splits=num_splits, workspace=workspace)


def _separate(case, cache, lat, rope, slots, num_splits=0):
    m = _m()
    m.mla_nvfp4_quantize_append(lat, rope, slots, cache, case.page_stride)
    return m.mla_sparse_decode(case.q, cache, case.page_stride, case.block_table, case.topk_idx,
                               th.softmax_scale(), num_splits=num_splits)


@pytest.mark.parametrize("q_len,H,ctx,topk,splits", [
    (1, 64, [3000, 5000, 700], 512, 0),
    (3, 16, [2000, 4100], 256, 1),
    (4, 32, [1500, 6000], 1024, 4),
    (15, 16, [1000, 2200], 256, 2),      # MTP-like: 15 new rows per request, 4 passes
    (16, 32, [1100, 2300], 256, 3),      # the largest q_len the fused call takes
    (2, 80, [900, 2500], 256, 2),        # two decode launches (64 + 16 heads)
])
def test_fused_append_equals_append_then_decode(q_len, H, ctx, topk, splits):
    print(f"case: fused append q_len={q_len} H={H} ctx={ctx} k={topk} splits={splits}", flush=True)
    case, slots, lat, rope, good, stale = _setup(len(ctx), q_len, H, ctx, topk, 2301 + q_len)
    assert not torch.equal(stale, good)
    c1 = stale.clone()
    o1, l1 = _fused(case, c1, lat, rope, slots, splits)
    c2 = stale.clone()
    o2, l2 = _separate(case, c2, lat, rope, slots, splits)
    torch.cuda.synchronize()
    assert torch.equal(c1, good), "the fused call wrote other cache bytes than the append"
    assert torch.equal(c2, good)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "fused and separate results differ"
    ref_o, ref_l = th.oracle_sparse(case)
    w = th.assert_parity(o1, l1, ref_o, ref_l, what="fused append")
    print(f"fused append: worst row err {w[0]:.2e} lse {w[1]:.2e}", flush=True)


def test_fused_append_skipped_slot_and_empty_list():
    """A new row with slot -1 is not written, and entries on its position read the cache as it
    was (as after a skipped append); a token with an all -1 list gets zeros and lse -inf; the
    request's rows are still written by its writer workgroup."""
    print("case: fused append skipped slot + empty list", flush=True)
    case, slots, lat, rope, good, stale = _setup(2, 2, 16, [1200, 3000], 256, 2310)
    slots = slots.clone()
    slots[1] = -1                                   # request 0, new row 1: not appended
    case.topk_idx[1, 0] = -1                        # request 1, token 0: empty list
    c1 = stale.clone()
    o1, l1 = _fused(case, c1, lat, rope, slots, 1)
    c2 = stale.clone()
    o2, l2 = _separate(case, c2, lat, rope, slots, 1)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(o1[1, 0] == 0) and torch.all(torch.isneginf(l1[1, 0]))
    # the other rows of the call are the appended ones
    ref_o, ref_l = th.oracle_sparse(case, tokens=[(0, 0), (1, 1)])
    th.assert_parity(o1, l1, ref_o, ref_l, tokens=[(0, 0), (1, 1)], what="fused append, skipped slot")


def test_fused_append_batched_shape():
    """B = 32 requests of 143,360 positions, one query token each, 64 heads, top-k 2048 (the
    batched decode step): fused vs separate bit for bit over the whole output and the new rows'
    bytes; two tokens against the oracle."""
    print("case: fused append B=32 q_len=1 H=64 ctx=143360 k=2048", flush=True)
    B, ctx = 32, [143360] * 32
    case, slots, lat, rope, good, stale = _setup(B, 1, 64, ctx, 2048, 2320)
    c1 = stale.clone()
    o1, l1 = _fused(case, c1, lat, rope, slots)
    c2 = stale.clone()
    o2, l2 = _separate(case, c2, lat, rope, slots)
    torch.cuda.synchronize()
    assert torch.equal(c1, good)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    tokens = [(0, 0), (21, 0)]
    idx = case.topk_idx.cpu().numpy()
    need = {b: set(int(j) for j in idx[b, 0] if j >= 0) for b, _ in tokens}
    ref_o, ref_l = th.oracle_sparse(case, tokens=tokens, cache=th.oracle_cache(case, need))
    w = th.assert_parity(o1, l1, ref_o, ref_l, tokens=tokens, what="fused append batched")
    print(f"fused append batched: worst row err {w[0]:.2e} lse {w[1]:.2e}", flush=True)


def test_fused_append_graph_replays():
    """The fused call captured in a HIP graph: every replay (with eager work and a
    synchronization between replays) gives the eager result and the appended cache."""
    print("case: fused append graph replay", flush=True)
    m = _m()
    case, slots, lat, rope, good, stale = _setup(2, 1, 64, [4000, 2600], 512, 2330)
    splits = m.mla_sparse_decode_num_splits(2, 64, 512, 0)
    ws = torch.empty(max(256, m.mla_decode_workspace_size(2, 64, splits)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(2, 1, 64, 512, device="cuda")
    lse = torch.empty(2, 1, 64, device="cuda")
    cache = stale.clone()
    e_o, e_l = _fused(case, cache, lat, rope, slots)
    torch.cuda.synchronize()
    assert torch.equal(cache, good)
    cache.copy_(stale)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        m.mla_sparse_decode_append(case.q, cache, case.page_stride, case.block_table, case.topk_idx,
                                   th.softmax_scale(), lat, rope, slots, out=out, lse=lse,
                                   num_splits=splits, workspace=ws, stream=s)   # warm-up
        torch.cuda.synchronize()
        cache.copy_(stale)
        with torch.cuda.graph(g, stream=s):
            m.mla_sparse_decode_append(case.q, cache, case.page_stride, case.block_table,
                                       case.topk_idx, th.softmax_scale(), lat, rope, slots, out=out,
                                       lse=lse, num_splits=splits, workspace=ws, stream=s)
    for r in range(3):
        cache.copy_(stale)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache, good), f"replay {r}: cache"
        assert torch.equal(out, e_o) and torch.equal(lse, e_l), f"replay {r}: output"
