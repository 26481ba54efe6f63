"""The FP8 indexer scoring pass on the GPU against the fp64 oracle, and the chain it starts:
indexer scores -> top-k selection -> sparse decode.

Tolerance: each head's dot product is a sum of 128 E4M3 x E4M3 products, exact in fp32, summed in
fp32; the ReLU cannot grow an error; the 64 weighted head terms are summed in fp32 and scaled
once. With M = c_s * sum_j |w_j| * sum_d |q_jd k_sd| the error is below (128 + 64 + 2) * 2^-24 * M
~ 1.2e-5 M; the test allows 2e-5 M. Where the scores decide a list (top-k), both sides take the
decision on the same fp32 scores (the GPU's).
"""

import numpy as np
import pytest
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from oracle import indexer as oi
from oracle import topk as ot
from tests import helpers as th

pytestmark = pytest.mark.gpu

TOL = 2e-5


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _inputs(ctx, q_len, seed, spare_pages=3, page_stride=wl.INDEXER_PAGE_BYTES):
    B = len(ctx)
    bt, n_pages = wl.gen_block_table(ctx, seed, "cuda", spare_pages=spare_pages)
    packed, q, w = wl.gen_indexer(n_pages, B, q_len, seed + 1, "cuda")
    if page_stride != wl.INDEXER_PAGE_BYTES:
        cache = torch.zeros(n_pages, page_stride, dtype=torch.uint8, device="cuda")
        cache[:, :wl.INDEXER_PAGE_BYTES] = packed.view(n_pages, -1)
        packed = cache.reshape(-1)
    seq = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    return bt, packed, q, w, seq


def _check(got, ref, mag, what):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > TOL * mag + 1e-30
    assert np.all(np.isfinite(got)), f"{what}: non-finite scores"
    assert not np.any(bad), (f"{what}: {int(bad.sum())} scores off, worst "
                             f"{float(np.max(err / np.maximum(mag, 1e-30))):.3e} of the magnitude")
    return float(np.max(err / np.maximum(mag, 1e-30)))


@pytest.mark.parametrize("page_stride", [wl.INDEXER_PAGE_BYTES, 8448 + 4096])
def test_indexer_scores_every_visible_position(page_stride):
    """Two requests with ragged contexts (partial last pages), q_len 3, every visible position of
    every token; positions a token may not select keep the sentinel the output held."""
    ctx, q_len = [700, 1300], 3
    print(f"case: indexer ctx={ctx} q_len={q_len} page_stride={page_stride}", flush=True)
    bt, cache, q, w, seq = _inputs(ctx, q_len, 2101, page_stride=page_stride)
    n_max = bt.shape[1] * 64
    out = torch.full((2, q_len, n_max), float("nan"), device="cuda")
    _m().mla_indexer_scores(q, w, cache, page_stride, bt, seq, n_max=n_max, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, vis = oi.indexer_scores(q.cpu().numpy(), w.cpu().numpy().astype(np.float64), cache.cpu().numpy(),
                                 page_stride, bt.cpu().numpy(), ctx, n_max)
    assert np.all(np.isnan(got[~vis])), "positions outside the window were written"
    qc, wc, bc, cc = q.cpu().numpy(), w.cpu().numpy().astype(np.float64), bt.cpu().numpy(), cache.cpu().numpy()
    worst = 0.0
    for b in range(2):
        for t in range(q_len):
            n = ot.visible_count(ctx[b], q_len, t)
            codes, scales = oi.read_keys(cc, page_stride, bc[b], np.arange(n))
            mag = oi.score_magnitude_at(qc[b, t], wc[b, t], codes, scales)
            worst = max(worst, _check(got[b, t, :n], ref[b, t, :n], mag, f"token ({b}, {t})"))
    print(f"worst error {worst:.3e} of the score magnitude", flush=True)


def test_indexer_unmapped_and_outside_pages_score_zero():
    ctx, q_len = [640], 1
    bt, cache, q, w, seq = _inputs(ctx, q_len, 2102, spare_pages=0)
    bt[0, 2] = -1                                    # unmapped
    bt[0, 5] = cache.numel() // wl.INDEXER_PAGE_BYTES + 4   # past the end of the cache
    out = _m().mla_indexer_scores(q, w, cache, wl.INDEXER_PAGE_BYTES, bt, seq, n_max=640)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0, 0]
    assert np.all(got[128:192] == 0) and np.all(got[320:384] == 0)
    ref, _ = oi.indexer_scores(q.cpu().numpy(), w.cpu().numpy().astype(np.float64), cache.cpu().numpy(),
                               wl.INDEXER_PAGE_BYTES, bt.cpu().numpy(), ctx, 640)
    codes, scales = oi.read_keys(cache.cpu().numpy(), wl.INDEXER_PAGE_BYTES, bt.cpu().numpy()[0], np.arange(640))
    mag = oi.score_magnitude_at(q.cpu().numpy()[0, 0], w.cpu().numpy()[0, 0].astype(np.float64), codes, scales)
    _check(got, ref[0, 0], mag, "unmapped pages")


def test_indexer_topk_decode_chain_pages_shape():
    """The pages' launch shape: one request, 15 query tokens, 149,504 positions, 16 heads.
    Indexer scores on sampled positions against the oracle; the top-2048 lists of the GPU scores
    exactly as the oracle selects them from the same scores; the decode over those lists against
    the oracle on two tokens."""
    m = _m()
    ctx, q_len, H = [149504], 15, 16
    print("case: indexer chain B=1 q_len=15 ctx=149504 H=16", flush=True)
    case = th.build_case(1, q_len, H, ctx, 2048, seed=2103, spare_pages=0,
                         topk_fn=lambda B, q, k, c, s, d: wl.gen_topk_batched(B, q, k, c[0], s, d))
    packed, iq, iw = wl.gen_indexer(case.n_pages, 1, q_len, 2104, "cuda")
    n_max = ctx[0]
    scores = m.mla_indexer_scores(iq, iw, packed, wl.INDEXER_PAGE_BYTES, case.block_table, case.seq_lens,
                                  n_max=n_max)
    idx = m.mla_topk_indices(scores, case.seq_lens, 2048)
    case.topk_idx = idx
    out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table, idx,
                                   th.softmax_scale())
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    qc, wc = iq.cpu().numpy(), iw.cpu().numpy().astype(np.float64)
    cc, bc = packed.cpu().numpy(), case.block_table.cpu().numpy()
    rng = np.random.default_rng(5)
    worst = 0.0
    for t in range(q_len):
        n = ot.visible_count(ctx[0], q_len, t)
        pos = np.unique(np.concatenate([rng.integers(0, n, 1024), np.arange(n - 20, n)]))
        codes, scales = oi.read_keys(cc, wl.INDEXER_PAGE_BYTES, bc[0], pos)
        ref = oi.scores_at(qc[0, t], wc[0, t], codes, scales)
        mag = oi.score_magnitude_at(qc[0, t], wc[0, t], codes, scales)
        worst = max(worst, _check(got[0, t, pos], ref, mag, f"token {t}"))
    print(f"indexer: worst sampled error {worst:.3e} of the score magnitude", flush=True)
    ref_idx = ot.topk_indices(got, case.seq_lens.cpu().numpy(), q_len, 2048)
    assert np.array_equal(idx.cpu().numpy(), ref_idx), "top-k of the indexer scores differs"
    tokens = [(0, 0), (0, 14)]
    need = {0: set(int(j) for t in (0, 14) for j in ref_idx[0, t] if j >= 0)}
    ref_o, ref_l = th.oracle_sparse(case, tokens=tokens, cache=th.oracle_cache(case, need))
    w_o, w_l = th.assert_parity(out, lse, ref_o, ref_l, tokens=tokens, what="indexer-selected decode")
    print(f"decode over the indexer's lists: worst row err {w_o:.2e} lse {w_l:.2e}", flush=True)
