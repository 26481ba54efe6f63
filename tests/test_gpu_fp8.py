"""GPU parity of the FP8 baseline (576-byte rows) and of the staged NVFP4 -> FP8 path.

Codec work (FP8 append, staging conversion) is compared byte for byte with the oracle; attention
is held to the same bar as the NVFP4 path (row relative error and |lse error| <= 2e-3).
"""

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import fp8 as f8
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def test_fp8_append_bit_exact():
    """Random magnitudes from E4M3 subnormals to beyond 448, hand ties, signed zeros, skips."""
    print("case: fp8 append 3000 rows", flush=True)
    m = _m()
    g = torch.Generator().manual_seed(5)
    N = 3000
    lat = torch.randn(N, 512, generator=g) * torch.exp2(torch.randint(-14, 10, (N, 1), generator=g).float())
    rope = torch.randn(N, 64, generator=g) * torch.exp2(torch.randint(-12, 9, (N, 1), generator=g).float())
    lat[0, :10] = torch.tensor([2.8125, 3.375, -464.0, 448.0, -0.0, 2.0 ** -10, 1.5 * 2 ** -9,
                                1.0625, 1.1875, 1e30])
    rope[0, :4] = torch.tensor([-0.0, 248.0, -3.25, 2.0 ** -9])
    lat, rope = lat.bfloat16(), rope.bfloat16()
    n_pages = N // 64 + 4
    perm = torch.randperm(n_pages * 64, generator=g)[:N]
    slots = perm.to(torch.int64)
    slots[::97] = -1                                          # skipped rows
    page = th.FP8_PAGE_BYTES
    cache = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    m.mla_fp8_append(lat.cuda(), rope.cuda(), slots.cuda(), cache, page)
    torch.cuda.synchronize()
    want = np.zeros(n_pages * page, dtype=np.uint8)
    enc = f8.quantize_rows_fp8(lat.double().numpy(), rope.double().numpy())
    oc.write_rows(want, page, slots.numpy(), enc)
    got = cache.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_fp8_append_every_finite_bf16_value():
    """Every finite bf16 value as a latent element and as a rope element (exhaustive)."""
    print("case: fp8 append, exhaustive bf16 values", flush=True)
    m = _m()
    bits = torch.arange(0, 65536, dtype=torch.int32)
    vals = bits.to(torch.int16).view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals)]
    n_lat = (vals.numel() + 511) // 512
    n_rope = (vals.numel() + 63) // 64
    N = max(n_lat, n_rope)
    lat = torch.zeros(N * 512)
    lat[:vals.numel()] = vals
    rope = torch.zeros(N * 64)
    rope[:vals.numel()] = vals
    lat, rope = lat.reshape(N, 512).bfloat16(), rope.reshape(N, 64).bfloat16()
    page = th.FP8_PAGE_BYTES
    n_pages = (N + 63) // 64
    slots = torch.arange(N, dtype=torch.int64)
    cache = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    m.mla_fp8_append(lat.cuda(), rope.cuda(), slots.cuda(), cache, page)
    torch.cuda.synchronize()
    want = np.zeros(n_pages * page, dtype=np.uint8)
    oc.write_rows(want, page, slots.numpy(), f8.quantize_rows_fp8(lat.double().numpy(), rope.double().numpy()))
    got = cache.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def _random_nvfp4_cache(n_pages, seed):
    """Uniform random bytes with the E4M3 NaN codes (0x7F, 0xFF) replaced in the scale and rope
    parts: every scale value and sign, every code."""
    rng = np.random.default_rng(seed)
    cache = rng.integers(0, 256, n_pages * th.PAGE_BYTES, dtype=np.uint8)
    rows = cache.reshape(n_pages * 64, 352)
    tail = rows[:, 256:]
    tail[(tail & 0x7F) == 0x7F] ^= 0x01
    return cache


def test_stage_fp8_bit_exact_on_random_bytes():
    print("case: staging conversion over random NVFP4 bytes", flush=True)
    m = _m()
    n_pages = 8
    host = _random_nvfp4_cache(n_pages, 8)
    B, q_len, topk = 2, 3, 100
    bt = np.array([[5, 1, 7, -1], [0, 2, 6, 3]], dtype=np.int32)      # request 0: page 3 unmapped
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 256, (B, q_len, topk)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.15] = -1
    idx[0, 0, :5] = [255, 192, 300, -1, 0]           # unmapped page, beyond the table, -1
    cache = torch.from_numpy(host).cuda()
    rows, sidx, sbt = m.mla_nvfp4_stage_fp8(cache, th.PAGE_BYTES, torch.from_numpy(bt).cuda(),
                                            torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    P = 128
    rows = rows.cpu().numpy().reshape(B * q_len, P, 576)
    sidx = sidx.cpu().numpy().reshape(B * q_len, topk)
    sbt = sbt.cpu().numpy()
    assert np.array_equal(sbt, np.arange(B * q_len * 2, dtype=np.int32).reshape(B * q_len, 2))
    for b in range(B):
        for t in range(q_len):
            tok = b * q_len + t
            for e in range(topk):
                j = int(idx[b, t, e])
                valid = 0 <= j < 4 * 64 and bt[b, j // 64] >= 0
                assert sidx[tok, e] == (e if valid else -1), (b, t, e, j)
                if valid:
                    src = oc.read_rows(host, th.PAGE_BYTES, bt[b], [j])
                    want = f8.nvfp4_rows_to_fp8(src)[0]
                    assert np.array_equal(rows[tok, e], want), (b, t, e, j)


def _fp8_sparse(case, splits):
    m = _m()
    out, lse = m.mla_fp8_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                       case.topk_idx, th.softmax_scale(), num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("H", [16, 64, 80])
def test_fp8_sparse_parity_ragged_tail(H):
    print(f"case: fp8 sparse H={H} k=1000 ctx=[3000,2100] q_len=2", flush=True)
    case = th.build_case(2, 2, H, [3000, 2100], 1000, seed=400 + H, fmt="fp8")
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (1, 3):
        out, lse = _fp8_sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"fp8 H={H} splits={s}")


def test_fp8_sparse_short_contexts_and_empty_list():
    print("case: fp8 sparse ctx in {1, 31, 300, 2047} with k=2048, plus an empty list", flush=True)
    ctx = [1, 31, 300, 2047]
    case = th.build_case(len(ctx), 1, 64, ctx, 2048, seed=78, fmt="fp8")
    case.topk_idx[2, 0] = -1
    ref_o, ref_l = th.oracle_sparse(case)
    for s in (0, 1, 8):
        out, lse = _fp8_sparse(case, s)
        th.assert_parity(out, lse, ref_o, ref_l, what=f"fp8 short ctx splits={s}")
        assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_fp8_dense_parity():
    print("case: fp8 dense ctx=[5000,700] q_len=3 H=64", flush=True)
    m = _m()
    case = th.build_case(2, 3, 64, [5000, 700], 0, seed=91, fmt="fp8")
    ref_o, ref_l = th.oracle_dense(case)
    for split in (1024, 4096):
        out, lse = m.mla_fp8_dense_decode(case.q, case.cache, case.page_stride, case.block_table,
                                          case.seq_lens, th.softmax_scale(), split_tokens=split)
        torch.cuda.synchronize()
        th.assert_parity(out, lse, ref_o, ref_l, what=f"fp8 dense split={split}")


def _staged_reference(case):
    staged = th.oracle_staged_cache(case)
    q = case.q.detach().float().cpu().numpy().astype(np.float64)
    return oa.sparse_decode(q, staged, th.FP8_PAGE_BYTES, case.block_table.cpu().numpy(),
                            case.topk_idx.cpu().numpy(), th.softmax_scale(), row_bytes=576)


@pytest.mark.parametrize("ctx,topk,H", [([3000, 2100], 1000, 64), ([1, 300, 2047], 2048, 16)])
def test_staged_parity(ctx, topk, H):
    print(f"case: staged ctx={ctx} k={topk} H={H}", flush=True)
    m = _m()
    case = th.build_case(len(ctx), 2, H, ctx, topk, seed=500 + topk)
    ref_o, ref_l = _staged_reference(case)
    for s in (0, 1, 4):
        out, lse = m.mla_staged_sparse_decode(case.q, case.cache, case.page_stride,
                                              case.block_table, case.topk_idx, th.softmax_scale(),
                                              num_splits=s)
        torch.cuda.synchronize()
        th.assert_parity(out, lse, ref_o, ref_l, what=f"staged splits={s}")
