"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Each case builds the whole cache on the GPU at its real size (140K-200K-token requests, 64-row
pages, random block tables), runs the decode with the library's own split choice (the one
bench.py uses), and compares query tokens -- all heads and all 512 output dims of each -- with
the fp64 oracle: every output row of the batched, MTP and dense configurations, and sampled
tokens of the mixed one. The oracle quantizes, by itself, only the bf16 rows those tokens read.
The MTP and dense comparisons are split over several tests (a module-level fixture runs the GPU
side once) so that each keeps the oracle's CPU time to about a minute.
"""

import numpy as np
import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import nvfp4 as nv
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _sampled_sparse(case, tokens, what):
    m = _m()
    splits = m.mla_sparse_decode_num_splits(case.B * case.q_len, case.H, case.topk, 0)
    out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                   case.topk_idx, th.softmax_scale())
    torch.cuda.synchronize()
    idx = case.topk_idx.cpu().numpy()
    need = {}
    for b, t in tokens:
        need.setdefault(b, set()).update(int(j) for j in idx[b, t] if j >= 0)
    cache = th.oracle_cache(case, need)
    ref_o, ref_l = th.oracle_sparse(case, tokens=tokens, cache=cache)
    worst, worst_lse = th.assert_parity(out, lse, ref_o, ref_l, tokens=tokens, what=what)
    print(f"{what}: splits={splits} worst row err {worst:.2e} lse {worst_lse:.2e}", flush=True)
    return out, lse


def test_batched_140k_topk2048():
    """B=32, q_len=1, H=64, 143,360-token caches, top-k 2048 (8 row splits per token)."""
    print("case: batched B=32 H=64 ctx=143360 k=2048", flush=True)
    case = th.build_case(32, 1, 64, [143360] * 32, 2048, seed=1001, spare_pages=0,
                         topk_fn=lambda B, q, k, ctx, s, d: wl.gen_topk_batched(B, q, k, ctx[0], s, d))
    assert _m().mla_sparse_decode_num_splits(32, 64, 2048, 0) == 8
    _sampled_sparse(case, [(b, 0) for b in range(32)], "batched (every output row)")


@pytest.fixture(scope="module")
def mtp_run():
    """B=16, q_len=15, H=64, 149,504-token caches (6144 rows of each appended by one call),
    independent top-k 2048 per query token; decoded once with the library's split choice."""
    print("case: mtp B=16 q_len=15 H=64 ctx=149504 k=2048", flush=True)
    case = th.build_case(16, 15, 64, [149504] * 16, 2048, seed=1002, spare_pages=0,
                         topk_fn=lambda B, q, k, ctx, s, d: wl.gen_topk_batched(B, q, k, ctx[0], s, d),
                         append_rows=6144)
    m = _m()
    out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table,
                                   case.topk_idx, th.softmax_scale())
    torch.cuda.synchronize()
    return case, out, lse


@pytest.mark.parametrize("part", [0, 1])
def test_mtp_146k_q15_every_row(mtp_run, part):
    """Every output row of the MTP configuration: requests 8*part .. 8*part+7, all 15 tokens."""
    case, out, lse = mtp_run
    idx = case.topk_idx.cpu().numpy()
    worst = (0.0, 0.0)
    for b in range(8 * part, 8 * part + 8):
        tokens = [(b, t) for t in range(15)]
        cache = th.oracle_cache(case, {b: set(int(j) for j in idx[b].ravel() if j >= 0)})
        ref_o, ref_l = th.oracle_sparse(case, tokens=tokens, cache=cache)
        w = th.assert_parity(out, lse, ref_o, ref_l, tokens=tokens, what=f"mtp request {b}")
        worst = (max(worst[0], w[0]), max(worst[1], w[1]))
        print(f"mtp request {b}: worst row err {w[0]:.2e} lse {w[1]:.2e}", flush=True)
    print(f"mtp part {part}: worst row err {worst[0]:.2e} lse {worst[1]:.2e}", flush=True)


@pytest.fixture(scope="module")
def dense_run():
    """B=8, q_len=1, H=64, 149,504-token caches, dense over every row: decoded with the
    configured 4096-position splits and with the library's one-wave split size."""
    print("case: dense B=8 H=64 ctx=149504", flush=True)
    case = th.build_case(8, 1, 64, [149504] * 8, 0, seed=1003, spare_pages=0)
    m = _m()
    assert m.mla_dense_decode_num_splits(case.block_table.shape[1], 4096) == 37
    runs = {}
    for st in (4096, 0):
        runs[st] = m.mla_dense_decode(case.q, case.cache, case.page_stride, case.block_table,
                                      case.seq_lens, th.softmax_scale(), split_tokens=st)
    torch.cuda.synchronize()
    return case, runs


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_dense_146k_every_row(dense_run, part):
    """Every output row of the dense configuration: tokens of requests 2*part and 2*part+1, for
    both split sizes."""
    case, runs = dense_run
    for b in (2 * part, 2 * part + 1):
        tokens = [(b, 0)]
        cache = th.oracle_cache(case, {b: range(case.ctx[b])})
        ref_o, ref_l = th.oracle_dense(case, tokens=tokens, cache=cache)
        for st, (out, lse) in runs.items():
            w = th.assert_parity(out, lse, ref_o, ref_l, tokens=tokens, what=f"dense request {b} split {st}")
            print(f"dense request {b} split_tokens={st}: worst row err {w[0]:.2e} lse {w[1]:.2e}", flush=True)


def test_mixed_serving_step():
    """B=64, contexts log-uniform in [4K, 200K] (6144 of them appended by one call covering all
    requests, 393,216 rows), q_len in {1, 15}, H=64, top-k 2048. The appended rows are checked
    bit-exact on a sample; the decode on tokens of short and long requests, including padding
    tokens of q_len=1 requests (empty lists: zero output, lse -inf)."""
    mx = wl.named_workload("mixed")
    print(f"case: mixed B={mx.B} ctx {min(mx.ctx)}..{max(mx.ctx)} + 6144 appended", flush=True)
    ctx = [c + 6144 for c in mx.ctx]
    case = th.build_case(mx.B, 15, 64, ctx, 2048, seed=1004, spare_pages=0, append_rows=6144,
                         topk_fn=lambda B, q, k, c, s, d: wl.gen_topk(B, q, k, c, s, d, q_lens=mx.q_lens))
    # appended rows: bit-exact on 32,768 sampled rows of the 393,216
    g = np.random.default_rng(7)
    bt = case.block_table.cpu().numpy()
    pick_b = g.integers(0, mx.B, 32768)
    pick_p = np.array([ctx[b] - 6144 for b in pick_b]) + g.integers(0, 6144, 32768)
    rows = torch.as_tensor(np.array([case.row_base[b] for b in pick_b]) + pick_p, device=case.latent.device)
    enc = nv.quantize_rows(th.bf16_to_f64(case.latent[rows]), th.bf16_to_f64(case.rope[rows]))
    slots = np.array([oc.logical_slot(bt[b], int(p)) for b, p in zip(pick_b, pick_p)])
    offs = torch.as_tensor((slots // 64) * case.page_stride + (slots % 64) * 352, device=case.cache.device)
    got = case.cache[offs[:, None] + torch.arange(352, device=offs.device)[None, :]].cpu().numpy()
    assert np.array_equal(got, enc), "appended rows differ from the oracle's encoding"
    # decode on sampled tokens
    order = np.argsort(mx.ctx)
    short, long_ = int(order[0]), int(order[-1])
    q15 = [b for b in range(mx.B) if mx.q_lens[b] == 15]
    q1 = [b for b in range(mx.B) if mx.q_lens[b] == 1]
    tokens = [(short, 0), (long_, 0), (q15[0], 14), (q15[-1], 6), (q1[0], 0), (q1[0], 9)]
    out, lse = _sampled_sparse(case, tokens, "mixed")
    pad = out[q1[0], 1:].cpu()
    assert torch.all(pad == 0) and torch.all(torch.isneginf(lse[q1[0], 1:].cpu()))
