"""GPU sparse / dense decode parity against the fp64 oracle (row relative error <= 2e-3)."""

import math

import numpy as np
import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _sparse(case, num_splits=0):
    m = _m()
    out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                   case.topk_idx, th.softmax_scale(), num_splits=num_splits)
    torch.cuda.synchronize()
    return out, lse


def _dense(case, split_tokens=4096):
    m = _m()
    out, lse = m.mla_dense_decode(case.q, case.cache, case.page_stride, case.block_table,
                                  case.seq_lens, th.softmax_scale(), split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out, lse


def test_tiny_config_fp32_queries():
    """B=1, q_len=1, H=16, 4096-token cache, top-k 256 uniform, fp32 queries."""
    print("case: tiny H=16 k=256 fp32 q", flush=True)
    case = th.build_case(1, 1, 16, [4096], 256, seed=1001, q_dtype="fp32")
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (0, 1, 2, 4):
        out, lse = _sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"tiny splits={s}")


@pytest.mark.parametrize("H", [16, 32, 48, 64, 80, 128])
def test_head_counts_ragged_tail(H):
    """Several tiles plus a ragged last tile (k=1000), 2 requests x 2 query tokens."""
    print(f"case: H={H} k=1000 ctx=[3000,2100] q_len=2", flush=True)
    case = th.build_case(2, 2, H, [3000, 2100], 1000, seed=200 + H)
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (1, 3):
        out, lse = _sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"H={H} splits={s}")


def test_short_contexts_minus_one_padding():
    """Contexts shorter than k leave -1 entries anywhere in the list (they are skipped)."""
    print("case: ctx in {1, 31, 300, 1000, 2047} with k=2048", flush=True)
    ctx = [1, 31, 300, 1000, 2047]
    case = th.build_case(len(ctx), 1, 64, ctx, 2048, seed=77)
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (0, 1, 8):
        out, lse = _sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"short ctx splits={s}")


def test_empty_and_single_entry_lists():
    print("case: all -1 list and single-entry list", flush=True)
    case = th.build_case(2, 1, 16, [500, 500], 64, seed=31)
    idx = torch.full_like(case.topk_idx, -1)
    idx[1, 0, 17] = 123
    case.topk_idx = idx
    out, lse = _sparse(case, 1)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(out, lse, ref_o, ref_l, what="single entry")
    # a single selected row returns that row's decoded latent
    m = _m()
    slot = int(case.block_table[1, 123 // 64]) * 64 + 123 % 64
    row = m.mla_nvfp4_dequantize_rows(case.cache, case.page_stride,
                                      torch.tensor([slot], dtype=torch.int64, device="cuda"))
    assert torch.allclose(out[1, 0], row[0, :512].expand(16, 512), rtol=0, atol=1e-6)


def test_split_invariance_and_determinism():
    print("case: split invariance, determinism", flush=True)
    case = th.build_case(2, 1, 64, [5000, 4000], 2048, seed=55)
    outs = []
    for s in (1, 2, 3, 4, 8, 16, 32):
        o, l = _sparse(case, s)
        outs.append((s, o.clone(), l.clone()))
    base_o, base_l = outs[0][1], outs[0][2]
    # Each split rounds its probabilities to FP16 against its own running maximum, so different
    # split counts agree to the FP16 rounding of P (unit roundoff 2^-11), not bitwise.
    for s, o, l in outs[1:]:
        rel = (o - base_o).abs().amax() / base_o.abs().amax()
        assert rel < 1e-3, f"splits={s} differs from 1 split by {rel}"
        assert (l - base_l).abs().amax() < 1e-4
    o2, l2 = _sparse(case, 8)
    assert torch.equal(o2, outs[4][1]) and torch.equal(l2, outs[4][2]), "not bitwise reproducible"
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(outs[4][1], outs[4][2], ref_o, ref_l, what="split 8")


@pytest.mark.parametrize("H,splits", [(16, 9), (16, 12), (64, 13), (16, 17), (80, 37)])
def test_split_merge_with_shared_split_ranges(H, splits):
    """Past 8 splits the merge's four waves each take a contiguous share of the splits (uneven
    shares at 9, 13, 17; the 8-at-a-time loop past 16) and meet in LDS; the result matches one
    split to the FP16 rounding of P, repeats bit for bit, and matches the oracle. H = 80 runs two
    decode launches (64 + 16 heads) into one merge."""
    print(f"case: split merge H={H} splits={splits}", flush=True)
    case = th.build_case(2, 2, H, [6000, 3500], 2048, seed=70 + splits)
    o1, l1 = _sparse(case, 1)
    o, l = _sparse(case, splits)
    rel = (o - o1).abs().amax() / o1.abs().amax()
    assert rel < 1e-3, f"splits={splits} differs from 1 split by {rel}"
    assert (l - l1).abs().amax() < 1e-4
    o2, l2 = _sparse(case, splits)
    assert torch.equal(o, o2) and torch.equal(l, l2), "not bitwise reproducible"
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(o, l, ref_o, ref_l, what=f"H={H} splits={splits}")


def test_permutation_and_duplicates():
    print("case: permuted list, duplicates", flush=True)
    case = th.build_case(1, 2, 16, [1500], 300, seed=91)
    o1, l1 = _sparse(case, 1)
    perm = torch.randperm(300, device="cuda")
    case.topk_idx = case.topk_idx[:, :, perm].contiguous()
    o2, l2 = _sparse(case, 1)
    assert (o1 - o2).abs().amax() / o1.abs().amax() < 1e-3
    dup = case.topk_idx.clone()
    dup[0, 0, :10] = dup[0, 0, 10:20]
    case.topk_idx = dup
    ref_o, ref_l = th.oracle_sparse(case)
    o3, l3 = _sparse(case, 2)
    th.assert_parity(o3, l3, ref_o, ref_l, what="duplicates")


def test_topk_all_equals_dense():
    print("case: top-k = every position vs dense", flush=True)
    ctx = 1500
    case = th.build_case(1, 1, 64, [ctx], 2048, seed=8)
    o_s, l_s = _sparse(case, 2)
    o_d, l_d = _dense(case, split_tokens=512)
    assert (o_s - o_d).abs().amax() / o_d.abs().amax() < 1e-3
    assert (l_s - l_d).abs().amax() < 1e-4


def test_dense_causal_and_splits():
    print("case: dense q_len=3 causal, split 64/512/4096/one-wave", flush=True)
    case = th.build_case(2, 3, 32, [2000, 700], 0, seed=12)
    ref_o, ref_l = th.oracle_dense(case)
    auto = _m().mla_dense_decode_split_tokens(6, 32, case.block_table.shape[1])
    for st in (64, 512, 4096, auto):
        out, lse = _dense(case, st)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"dense split_tokens={st}")


def test_uniform_scores_give_mean():
    print("case: q = 0 gives mean of V and lse = ln k", flush=True)
    case = th.build_case(1, 1, 16, [800], 96, seed=14)
    case.q = torch.zeros_like(case.q)
    m = _m()
    pos = case.topk_idx[0, 0].long()
    slots = case.block_table[0].long()[pos // 64] * 64 + pos % 64
    rows = m.mla_nvfp4_dequantize_rows(case.cache, case.page_stride, slots)
    mean = rows[:, :512].double().mean(0)
    # One split: the kernel's own FP32 accumulation. Two splits: each split's normalised partial
    # is kept in FP16, so the merge can be off by half an FP16 ulp of a partial (a mean of rows,
    # hence at most max |V|): 2^-11 * max |V|.
    for splits, atol in ((1, 2e-6), (2, 2.0 ** -11 * float(rows[:, :512].abs().max()) + 2e-6)):
        out, lse = _sparse(case, splits)
        assert torch.allclose(out[0, 0].double(), mean.expand(16, 512), rtol=0, atol=atol), splits
        assert torch.allclose(lse[0, 0], torch.full_like(lse[0, 0], math.log(96)), atol=1e-5), splits


def test_overlapping_lists_across_query_tokens():
    """Multi-token decode lists under an overlap model: the query tokens of a request share 80% of
    their positions (ascending lists), so rows repeat across the workgroups of one request."""
    print("case: overlap 0.8, B=2, q_len=4, H=64, ctx [5000, 4200], k=1024", flush=True)
    fn = lambda B, q, k, ctx, seed, dev: wl.gen_topk_overlap(B, q, k, ctx, 0.8, seed, dev)
    case = th.build_case(2, 4, 64, [5000, 4200], 1024, seed=321, topk_fn=fn)
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (0, 1, 3):
        out, lse = _sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"overlap 0.8 splits={s}")


def test_cache_beyond_4_gib():
    """A 4.5 GiB cache whose pages all lie past the 4 GiB mark: 64-bit row offsets in the append
    and in the decode's gathers (sparse and dense). The oracle works on a compact copy of the same
    rows, which it quantizes itself; the bytes past 4 GiB must equal its rows."""
    from oracle import attention as oa
    from oracle import cache as oc
    from oracle import nvfp4 as nv
    print("case: 4.5 GiB cache, every page past 4 GiB", flush=True)
    m = _m()
    dev = "cuda"
    page = th.PAGE_BYTES
    B, q_len, H, topk = 2, 2, 64, 512
    ctx = [2000, 1500]
    ppr = [(c + 63) // 64 for c in ctx]
    n_big = (9 << 29) // page + 1                       # 4.5 GiB of pages
    base = (1 << 32) // page + 7                        # first page used: past 4 GiB
    assert (base + sum(ppr)) <= n_big and base * page > (1 << 32)
    bt_small = torch.full((B, max(ppr)), -1, dtype=torch.int32)
    first = 0
    for b in range(B):
        bt_small[b, :ppr[b]] = torch.arange(first, first + ppr[b], dtype=torch.int32)
        first += ppr[b]
    bt_big = torch.where(bt_small >= 0, bt_small + base, bt_small).to(dev)
    lat, rope = wl.gen_latent_rope(sum(ctx), 61, dev)
    cache = torch.zeros(n_big * page, dtype=torch.uint8, device=dev)
    slots = torch.cat([wl.slot_mapping_for(bt_big, b, 0, c) for b, c in enumerate(ctx)])
    m.mla_nvfp4_quantize_append(lat, rope, slots, cache, page)
    q = wl.gen_queries(B, q_len, H, "bf16", 62, dev)
    idx = wl.gen_topk(B, q_len, topk, ctx, 63, dev)
    seq = torch.tensor(ctx, dtype=torch.int32, device=dev)
    scale = th.softmax_scale()
    out, lse = m.mla_sparse_decode(q, cache, page, bt_big, idx, scale)
    out_d, lse_d = m.mla_dense_decode(q, cache, page, bt_big, seq, scale, split_tokens=1024)
    torch.cuda.synchronize()
    got = cache[base * page:(base + sum(ppr)) * page].cpu().numpy()
    del cache
    torch.cuda.empty_cache()

    host = np.zeros(sum(ppr) * page, dtype=np.uint8)
    slots_small = torch.cat([wl.slot_mapping_for(bt_small, b, 0, c) for b, c in enumerate(ctx)]).numpy()
    oc.write_rows(host, page, slots_small,
                  nv.quantize_rows(lat.double().cpu().numpy(), rope.double().cpu().numpy()))
    assert np.array_equal(got, host), "bytes written past 4 GiB differ from the oracle's rows"
    q64 = q.float().cpu().numpy().astype(np.float64)
    ref_o, ref_l = oa.sparse_decode(q64, host, page, bt_small.numpy(), idx.cpu().numpy(), scale)
    th.assert_parity(out, lse, ref_o, ref_l, what="sparse, pages past 4 GiB")
    ref_od, ref_ld = oa.dense_decode(q64, host, page, bt_small.numpy(), seq.cpu().numpy(), scale)
    th.assert_parity(out_d, lse_d, ref_od, ref_ld, what="dense, pages past 4 GiB")


@pytest.mark.parametrize("H", [48, 64])
def test_fp32_queries_every_head_block(H):
    """fp32 queries with three and four 16-head blocks per workgroup, sparse and dense."""
    print(f"case: fp32 queries H={H} k=700 ctx=[1900, 800] q_len=2", flush=True)
    case = th.build_case(2, 2, H, [1900, 800], 700, seed=300 + H, q_dtype="fp32")
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (1, 3):
        out, lse = _sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"fp32 q H={H} splits={s}")
    ref_od, ref_ld = th.oracle_dense(case)
    out, lse = _dense(case, 512)
    th.assert_parity(out, lse, ref_od, ref_ld, what=f"fp32 q dense H={H}")


def test_dense_empty_and_tiny_windows():
    """q_len = 3 over requests of 1, 2, 65 and 130 positions: query token t sees positions
    0..seq_len-3+t, so the first tokens of the short requests see nothing (output 0, lse -inf),
    and the others see 1, 2, 63..66 or 128..130 positions."""
    print("case: dense empty / one-position windows, q_len=3", flush=True)
    case = th.build_case(4, 3, 64, [1, 2, 65, 130], 0, seed=17)
    ref_o, ref_l = th.oracle_dense(case)
    assert np.isneginf(ref_l[0, 0]).all() and np.isneginf(ref_l[0, 1]).all()
    for st in (64, 4096):
        out, lse = _dense(case, st)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"dense tiny windows split_tokens={st}")
        o = out.cpu().numpy()
        assert np.all(o[0, 0] == 0) and np.all(o[0, 1] == 0) and np.all(o[1, 0] == 0)


def test_dense_split_tokens_zero_is_the_one_wave_size():
    """split_tokens=0 in the binding takes the library's one-wave split size: the same bits as
    passing that size, and parity with the oracle."""
    print("case: dense split_tokens=0", flush=True)
    m = _m()
    case = th.build_case(3, 2, 64, [5000, 3100, 800], 0, seed=23)
    auto = m.mla_dense_decode_split_tokens(6, 64, case.block_table.shape[1])
    o0, l0 = _dense(case, 0)
    o1, l1 = _dense(case, auto)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    ref_o, ref_l = th.oracle_dense(case)
    th.assert_parity(o0, l0, ref_o, ref_l, what="dense split_tokens=0")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("H", [64, 80, 128])
def test_empty_tokens_and_empty_splits_write_every_output(fmt, H):
    """Workgroups with no valid row leave before the tile loop: requests padded with all -1 lists
    (a mixed step's shorter requests) and tokens whose valid entries all sit in the first split's
    part of the list, so that the later splits are empty. The output and the split workspace start
    as NaN bytes: every element must be written, empty tokens give +0 and lse -inf, and the others
    match the oracle."""
    print(f"case: empty tokens / empty splits fmt={fmt} H={H}", flush=True)
    m = _m()
    B, q_len, k = 4, 5, 1024
    case = th.build_case(B, q_len, H, [3000, 2500, 1800, 4100], k, seed=900 + H, fmt=fmt)
    idx = case.topk_idx.clone()
    q_lens = [5, 1, 2, 5]
    for b, n in enumerate(q_lens):
        idx[b, n:] = -1                                    # padding tokens of shorter requests
    idx[0, 1, 100:] = -1                                   # valid entries only in the first 100
    idx[3, 2, :] = -1
    idx[3, 2, 7] = 11                                      # one entry, in the first split
    case.topk_idx = idx.contiguous()
    ref_o, ref_l = th.oracle_sparse(case)
    fn = m.mla_sparse_decode if fmt == "nvfp4" else m.mla_fp8_sparse_decode
    for s in (1, 4, 16):
        out = torch.full((B, q_len, H, 512), float("nan"), device="cuda")
        lse = torch.full((B, q_len, H), float("nan"), device="cuda")
        ws = torch.full((max(m.mla_decode_workspace_size(B * q_len, H, s), 256),), 0xFF,
                        dtype=torch.uint8, device="cuda")
        fn(case.q, case.cache, case.page_stride, case.block_table, case.topk_idx,
           th.softmax_scale(), out=out, lse=lse, num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any() and not torch.isnan(lse).any(), f"splits={s}"
        th.assert_parity(out, lse, ref_o, ref_l, what=f"{fmt} H={H} empty tokens splits={s}")
        for b, n in enumerate(q_lens):
            if n < q_len:
                pad = out[b, n:]
                assert torch.all(pad == 0) and not torch.signbit(pad).any(), f"splits={s} b={b}"
                assert torch.all(torch.isneginf(lse[b, n:])), f"splits={s} b={b}"


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_block_table_width_staged_and_memory_lookups(fmt):
    """The block table's width is only a stride: padding it with -1 columns (to 9,216 and 9,217
    entries per row) gives the same bits as the unpadded table. List entries that point into the
    padding, or beyond the narrow table, are empty entries."""
    print(f"case: block-table widths 9216 / 9217 fmt={fmt}", flush=True)
    m = _m()
    case = th.build_case(3, 2, 64, [3000, 2200, 700], 512, seed=61, fmt=fmt)
    fn = m.mla_sparse_decode if fmt == "nvfp4" else m.mla_fp8_sparse_decode
    idx = case.topk_idx.clone()
    idx[0, 0, 5] = 9000 * 64 + 3                        # page column 9000: padding (-1), skipped
    idx[1, 1, 9] = 9216 * 64                            # column 9216: only in the wider table
    idx[2, 0, 0] = 200000                               # beyond the narrow table
    # the library treats an unmapped page or a position beyond the table as an empty entry
    case.topk_idx = idx.clone()
    case.topk_idx[0, 0, 5] = case.topk_idx[1, 1, 9] = case.topk_idx[2, 0, 0] = -1
    ref_o, ref_l = th.oracle_sparse(case)
    results = []
    for width in (case.block_table.shape[1], 9216, 9217):
        bt = torch.full((3, width), -1, dtype=torch.int32, device="cuda")
        bt[:, :case.block_table.shape[1]] = case.block_table
        for s in (1, 4):
            out, lse = fn(case.q, case.cache, case.page_stride, bt.contiguous(), idx.contiguous(),
                          th.softmax_scale(), num_splits=s)
            torch.cuda.synchronize()
            results.append((width, s, out.clone(), lse.clone()))
    for width, s, out, lse in results:
        th.assert_parity(out, lse, ref_o, ref_l, what=f"{fmt} width={width} splits={s}")
        base = next(r for r in results if r[1] == s)
        assert torch.equal(out, base[2]) and torch.equal(lse, base[3]), f"width={width} splits={s}"


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_page_offset_past_2_36_is_an_empty_page(fmt):
    """A block-table entry whose byte offset (page id x page stride) exceeds 2^36 must be treated
    as an unmapped page, never as the page its offset would wrap onto in 32-bit 16-byte units.
    With a 65,536-byte page stride, page id 2^20 + 6 lies at 2^36 + 6 * 65,536: a 32-bit wrap of
    that offset lands exactly on page 6, which holds real rows of the other request. Dense and
    sparse decode must both leave the 64 positions of that page out, as they leave out the
    positions of an unmapped (-1) page inside the context."""
    from oracle import attention as oa
    from oracle import cache as oc
    from oracle import fp8 as f8
    from oracle import nvfp4 as nv
    print(f"case: page offset past 2^36 fmt={fmt}", flush=True)
    m = _m()
    dev = "cuda"
    stride = 65536
    row_bytes = 576 if fmt == "fp8" else 352
    ctx = [300, 200]
    B, q_len, H = 2, 1, 64
    bt_real = torch.tensor([[0, 1, 2, 3, 4], [5, 6, 7, 8, -1]], dtype=torch.int32)
    cache = torch.zeros(9 * stride, dtype=torch.uint8, device=dev)
    lat, rope = wl.gen_latent_rope(sum(ctx), 71, dev)
    slots = torch.cat([wl.slot_mapping_for(bt_real, b, 0, c) for b, c in enumerate(ctx)]).to(dev)
    (m.mla_fp8_append if fmt == "fp8" else m.mla_nvfp4_quantize_append)(lat, rope, slots, cache, stride)
    bad = (1 << 20) + 6
    assert bad * stride >= (1 << 36) and (bad * stride) % (1 << 36) == 6 * stride
    bt = bt_real.clone()
    bt[0, 2] = bad                                   # positions 128..191 of request 0
    bt[1, 1] = -1                                    # and an unmapped page: 64..127 of request 1
    bt_d = bt.to(dev)
    q = wl.gen_queries(B, q_len, H, "bf16", 72, dev)
    seq = torch.tensor(ctx, dtype=torch.int32, device=dev)
    scale = th.softmax_scale()
    dense = m.mla_fp8_dense_decode if fmt == "fp8" else m.mla_dense_decode
    sparse = m.mla_fp8_sparse_decode if fmt == "fp8" else m.mla_sparse_decode
    results = [("dense", st, dense(q, cache, stride, bt_d, seq, scale, split_tokens=st)) for st in (64, 4096)]
    idx = torch.full((B, q_len, 256), -1, dtype=torch.int32)
    idx[0, 0, :200] = torch.arange(50, 250, dtype=torch.int32)      # crosses the bad page
    idx[1, 0, :150] = torch.arange(0, 150, dtype=torch.int32)
    results += [("sparse", s, sparse(q, cache, stride, bt_d, idx.to(dev), scale, num_splits=s)) for s in (1, 2)]
    torch.cuda.synchronize()
    # oracle: its own rows at the real slots; the bad page's positions are left out
    host = np.zeros(9 * stride, dtype=np.uint8)
    enc = (f8.quantize_rows_fp8 if fmt == "fp8" else nv.quantize_rows)(
        lat.double().cpu().numpy(), rope.double().cpu().numpy())
    oc.write_rows(host, stride, slots.cpu().numpy(), enc)
    keep0 = [j for j in range(300) if not 128 <= j < 192]
    keep1 = [j for j in range(200) if not 64 <= j < 128]
    dense_idx = np.full((B, q_len, 300), -1)
    dense_idx[0, 0, :len(keep0)] = keep0
    dense_idx[1, 0, :len(keep1)] = keep1
    q64 = q.float().cpu().numpy().astype(np.float64)
    ref_d = oa.sparse_decode(q64, host, stride, bt_real.numpy(), dense_idx, scale, row_bytes=row_bytes)
    sp_idx = idx.numpy().copy()
    sp_idx[(sp_idx >= 128) & (sp_idx < 192) & (np.arange(B)[:, None, None] == 0)] = -1
    sp_idx[(sp_idx >= 64) & (sp_idx < 128) & (np.arange(B)[:, None, None] == 1)] = -1
    ref_s = oa.sparse_decode(q64, host, stride, bt_real.numpy(), sp_idx, scale, row_bytes=row_bytes)
    for kind, arg, (out, lse) in results:
        ref_o, ref_l = ref_d if kind == "dense" else ref_s
        th.assert_parity(out, lse, ref_o, ref_l, what=f"{fmt} {kind} {arg} page past 2^36")


def test_debug_checks_reject_bad_entries_on_device_calls():
    """With the opt-in checks on, a device call whose list holds an entry the kernel would skip
    (an unmapped page) fails with MLA_ERR_INVALID_ARG before launching; with them off the same call
    runs and treats the entry as empty (parity with the list that has -1 there)."""
    print("case: debug checks on device calls", flush=True)
    m = _m()
    case = th.build_case(2, 1, 16, [900, 500], 256, seed=77)
    bt = case.block_table.clone()
    bt[1, 7] = -1                                   # positions 448..499 of request 1 unmapped
    idx = case.topk_idx.clone()
    idx[1, 0, 3] = 460
    before = m.mla_debug_checks_enabled()
    try:
        m.mla_set_debug_checks(True)
        with pytest.raises(m.MlaError, match="unmapped"):
            m.mla_sparse_decode(case.q, case.cache, case.page_stride, bt, idx, th.softmax_scale())
        with pytest.raises(m.MlaError, match="unmapped"):
            m.mla_dense_decode(case.q, case.cache, case.page_stride, bt, case.seq_lens, th.softmax_scale())
        bad_slots = torch.tensor([0, -3], dtype=torch.int64, device="cuda")
        with pytest.raises(m.MlaError, match="negative"):
            m.mla_nvfp4_quantize_append(case.latent[:2], case.rope[:2], bad_slots, case.cache,
                                        case.page_stride)
        out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                       case.topk_idx, th.softmax_scale())   # a good call passes
        m.mla_set_debug_checks(False)
        out_b, lse_b = m.mla_sparse_decode(case.q, case.cache, case.page_stride, bt, idx,
                                           th.softmax_scale())
        torch.cuda.synchronize()
    finally:
        m.mla_set_debug_checks(before)
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(out, lse, ref_o, ref_l, what="debug checks on, good call")
    ref_idx = idx.clone()
    in_page7 = (ref_idx[1] >= 448) & (ref_idx[1] < 512)      # every entry of request 1 in page 7
    ref_idx[1][in_page7] = -1
    case.topk_idx = ref_idx
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(out_b, lse_b, ref_o, ref_l, what="debug checks off, unmapped page skipped")
