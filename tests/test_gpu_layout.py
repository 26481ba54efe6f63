"""GPU block transfer between multi-layer page pools (bit-exact against the oracle's copy) and
decode over one layer of a block-major pool after a transfer (parity against the oracle)."""

import math

import numpy as np
import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import layout as lo
from oracle import nvfp4 as nv
from tests import helpers as th

pytestmark = pytest.mark.gpu
P = 64 * 352


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


@pytest.mark.parametrize("layout", [lo.BLOCK_MAJOR, lo.LAYER_MAJOR])
def test_copy_blocks_bit_exact(layout):
    print(f"case: copy_kv_blocks layout={layout}", flush=True)
    m = _m()
    L, nsrc, ndst = 5, 23, 31
    rng = np.random.default_rng(10 + layout)
    src = rng.integers(0, 256, nsrc * L * P, dtype=np.uint8)
    dst0 = rng.integers(0, 256, ndst * L * P, dtype=np.uint8)
    sb = rng.choice(nsrc, 12, replace=False).astype(np.int32)
    db = rng.choice(ndst, 12, replace=False).astype(np.int32)
    sb[3] = nsrc + 4                      # outside the source pool: this pair is skipped
    db[7] = -1                            # outside the destination pool: skipped
    d_src = torch.from_numpy(src).cuda()
    d_dst = torch.from_numpy(dst0.copy()).cuda()
    m.mla_copy_kv_blocks(d_src, d_dst, layout, L, P, torch.from_numpy(sb).cuda(), torch.from_numpy(db).cuda())
    torch.cuda.synchronize()
    want = dst0.copy()
    keep = [i for i in range(12) if i not in (3, 7)]
    lo.copy_blocks(src, want, layout, L, P, sb[keep], db[keep])
    got = d_dst.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ"


def test_decode_one_layer_of_block_major_pool_after_transfer():
    print("case: decode layer 1 of a block-major pool after copy_kv_blocks", flush=True)
    m = _m()
    L, layer, ctx, H = 3, 1, 1000, 64
    nsrc, ndst = 40, 50
    n_blk = wl.pages_for(ctx)
    g = torch.Generator().manual_seed(77)
    bt_src = torch.randperm(nsrc, generator=g)[:n_blk].to(torch.int32)
    bt_dst = torch.randperm(ndst, generator=g)[:n_blk].to(torch.int32)
    lat, rope = wl.gen_latent_rope(ctx, 78, "cuda")
    src = torch.zeros(nsrc * L * P, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(ndst * L * P, dtype=torch.uint8, device="cuda")
    slots = wl.slot_mapping_for(bt_src[None].cuda(), 0, 0, ctx)
    base, stride = lo.layer_view(lo.BLOCK_MAJOR, layer, L, P, nsrc)
    m.mla_nvfp4_quantize_append(lat, rope, slots, src[base:], stride)
    m.mla_copy_kv_blocks(src, dst, lo.BLOCK_MAJOR, L, P, bt_src.cuda(), bt_dst.cuda())
    q = wl.gen_queries(1, 2, H, "bf16", 79, "cuda")
    idx = wl.gen_topk(1, 2, 300, [ctx], 80, "cuda")
    dbase, dstride = lo.layer_view(lo.BLOCK_MAJOR, layer, L, P, ndst)
    out, lse = m.mla_sparse_decode(q, dst[dbase:], dstride, bt_dst[None].cuda(), idx, th.softmax_scale())
    torch.cuda.synchronize()
    # oracle: its own quantization placed through its own layer view of the destination pool
    pool = np.zeros(ndst * L * P, dtype=np.uint8)
    view = pool[dbase:]
    enc = nv.quantize_rows(th.bf16_to_f64(lat), th.bf16_to_f64(rope))
    bt = bt_dst.numpy()
    oc.write_rows(view, dstride, [oc.logical_slot(bt, j) for j in range(ctx)], enc)
    ref_o, ref_l = oa.sparse_decode(q.float().cpu().numpy().astype(np.float64), view, dstride,
                                    bt[None], idx.cpu().numpy(), th.softmax_scale())
    th.assert_parity(out, lse, ref_o, ref_l, what="block-major layer decode")
    # the other layers of the destination pool stay untouched
    other = dst.cpu().numpy().reshape(ndst, L, P)
    assert not other[:, [0, 2]].any()


@pytest.mark.parametrize("layout", [lo.BLOCK_MAJOR, lo.LAYER_MAJOR])
def test_copy_blocks_past_4_gib(layout):
    """64-layer pools of about 4.2 GiB: blocks whose pages lie past the 4 GiB mark are copied
    (64-bit page offsets); every page of every copied pair is compared at the offsets the oracle's
    layout gives, and the pages of a block that is not copied stay untouched."""
    print(f"case: copy_kv_blocks past 4 GiB, layout={layout}", flush=True)
    m = _m()
    L, nb = 64, 3100
    pool = nb * L * P
    assert pool > (1 << 32)
    g = torch.Generator(device="cuda").manual_seed(70 + layout)
    src = torch.randint(0, 256, (pool,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(pool, dtype=torch.uint8, device="cuda")
    sb = np.array([3099, 3050, 2990, 17, 3001], dtype=np.int32)
    db = np.array([3098, 5, 3097, 3090, 2999], dtype=np.int32)
    m.mla_copy_kv_blocks(src, dst, layout, L, P, torch.from_numpy(sb).cuda(), torch.from_numpy(db).cuda())
    torch.cuda.synchronize()
    high = 0
    for s_blk, d_blk in zip(sb, db):
        for layer in range(L):
            so = lo.page_offset(layout, int(s_blk), layer, L, P, nb)
            do = lo.page_offset(layout, int(d_blk), layer, L, P, nb)
            high += do + P > (1 << 32)
            assert torch.equal(dst[do:do + P], src[so:so + P]), f"block {s_blk}->{d_blk} layer {layer}"
    assert high > 0
    for layer in (0, 31, 63):
        o = lo.page_offset(layout, 3096, layer, L, P, nb)      # never a destination
        assert int(dst[o:o + P].count_nonzero()) == 0
    del src, dst
    torch.cuda.empty_cache()
