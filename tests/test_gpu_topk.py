"""GPU top-k position selection: bit-exact against the oracle (positions are integers), with
ties, signed zeros, causal windows, short contexts (-1 padding), every path of the kernels (rows
selected whole in LDS, the sampled cut, and the exact fallback after a cut that missed or
overflowed), the pages', batched and MTP launch shapes at full size, and the selected lists
feeding the sparse decode."""

import numpy as np
import pytest
import torch

from oracle import topk as tk
from tests import helpers as th

pytestmark = pytest.mark.gpu


def _m():
    import nvfp4_compressed_mla_amd as m
    return m


def _run(scores, seq_lens, q_len, k):
    m = _m()
    s = torch.from_numpy(np.ascontiguousarray(scores)).cuda()
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out = m.mla_topk_indices(s, sl, k)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("n_max,k,q_len,seq_lens,ties", [
    (5000, 256, 1, [5000, 3000, 100], False),
    (40000, 2048, 3, [40000, 17000], True),        # causal window per token
    (16384, 2048, 2, [16385, 2049], True),         # a window of 2048 - 1 + t
    (33000, 512, 1, [33000], True),
    (700, 2048, 1, [700], False),                  # fewer positions than k: -1 padding
    (1 << 20, 2048, 1, [1 << 20, 700001], False),  # the longest row the entry point accepts
    (1 << 20, 1, 2, [1 << 20, 1 << 20], True),     # k = 1 among many equal maxima: position order
])
def test_topk_matches_oracle(n_max, k, q_len, seq_lens, ties):
    print(f"case: topk n_max={n_max} k={k} q_len={q_len} seq_lens={seq_lens} ties={ties}", flush=True)
    rng = np.random.default_rng(n_max + k)
    B = len(seq_lens)
    s = rng.standard_normal((B, q_len, n_max)).astype(np.float32)
    if ties:
        s = np.round(s * 4) / 4                       # few distinct values: ties at the threshold
        s[..., ::7] = -0.0
        s[..., 3::11] = 0.0
    got = _run(s, seq_lens, q_len, k)
    want = tk.topk_indices(s, seq_lens, q_len, k)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    assert np.array_equal(_run(s, seq_lens, q_len, k), got)     # deterministic


def test_topk_all_equal_and_signed_zeros():
    print("case: topk all-equal scores and signed zeros", flush=True)
    s = np.zeros((1, 2, 40000), dtype=np.float32)
    s[0, 0] = 1.5
    s[0, 1, ::2] = -0.0
    got = _run(s, [40000], 2, 1000)
    assert list(got[0, 0]) == list(range(1000))                 # ties by position
    assert list(got[0, 1]) == list(range(1, 2000, 2))           # +0 above -0
    assert np.array_equal(got, tk.topk_indices(s, [40000], 2, 1000))



def test_topk_negative_threshold():
    """Every score negative, so the k-th largest key is below the key of +0: the stream takes its
    general comparison (the one-compare form needs a threshold at or above +0). Row 1's 12,000
    largest scores are -0.0, more than k: ties by position, through the fallback."""
    print("case: topk negative threshold", flush=True)
    rng = np.random.default_rng(77)
    s = (-np.abs(rng.standard_normal((2, 1, 60000))) - 0.5).astype(np.float32)
    s[1, 0, ::5] = -0.0
    got = _run(s, [60000, 60000], 1, 2048)
    assert np.array_equal(got, tk.topk_indices(s, [60000, 60000], 1, 2048))
    assert list(got[1, 0]) == list(range(0, 5 * 2048, 5))

def _sample_positions(n):
    # the 2048 positions the cut is drawn from: 256 evenly spaced runs of 8
    return np.array([(i >> 3) * n // 256 + (i & 7) for i in range(2048)])


def test_topk_fallback_when_the_sample_misses():
    """Scores that are high exactly at the sampled positions put the cut so high that fewer than k
    positions pass it; the merge must then select from the whole row (still exact)."""
    print("case: topk sample-miss fallback", flush=True)
    rng = np.random.default_rng(77)
    n = 50000
    s = rng.standard_normal((1, 2, n)).astype(np.float32)
    s[0, 0, _sample_positions(n)] += 100.0              # token 0 sees all n positions
    s[0, 1, _sample_positions(n - 1)] += 100.0          # token 1 sees n - 1
    got = _run(s, [n], 2, 2048)
    assert np.array_equal(got, tk.topk_indices(s, [n], 2, 2048))


def test_topk_fallback_when_candidates_overflow():
    """Heavy ties at the cut: far more than 8192 positions pass it."""
    print("case: topk candidate-overflow fallback", flush=True)
    rng = np.random.default_rng(78)
    s = (rng.integers(0, 3, size=(2, 1, 60000)) * 0.5).astype(np.float32)   # three values
    got = _run(s, [60000, 31000], 1, 2048)
    assert np.array_equal(got, tk.topk_indices(s, [60000, 31000], 1, 2048))


@pytest.mark.parametrize("k", [1, 2048])
def test_topk_mixed_lengths_one_launch(k):
    """Rows selected whole (<= 8192 visible), at the 8192 / 8193 boundary, and long rows."""
    print(f"case: topk mixed lengths k={k}", flush=True)
    rng = np.random.default_rng(79 + k)
    lens = [0, 1, 2047, 2048, 8192, 8193, 8194, 20000, 90001]
    s = rng.standard_normal((len(lens), 1, 90001)).astype(np.float32)
    got = _run(s, lens, 1, k)
    assert np.array_equal(got, tk.topk_indices(s, lens, 1, k))


def test_topk_pages_shape_full_size():
    """15 query tokens of one 149,504-token request, k = 2048 (the pages' launch shape)."""
    print("case: topk pages shape 15 x 149504, k=2048", flush=True)
    rng = np.random.default_rng(5)
    s = rng.standard_normal((1, 15, 149504)).astype(np.float32)
    got = _run(s, [149504], 15, 2048)
    want = tk.topk_indices(s, [149504], 15, 2048)
    assert np.array_equal(got, want)


def test_topk_feeds_sparse_decode():
    print("case: topk -> sparse decode", flush=True)
    m = _m()
    case = th.build_case(2, 2, 64, [3000, 2100], 0, seed=55)
    rng = np.random.default_rng(56)
    n_max = 3000
    s = rng.standard_normal((2, 2, n_max)).astype(np.float32)
    idx = m.mla_topk_indices(torch.from_numpy(s).cuda(), case.seq_lens, 700)
    case.topk_idx = idx
    case.topk = 700
    out, lse = m.mla_sparse_decode(case.q, case.cache, case.page_stride, case.block_table, idx,
                                   th.softmax_scale())
    torch.cuda.synchronize()
    want_idx = tk.topk_indices(s, [3000, 2100], 2, 700)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    ref_o, ref_l = th.oracle_sparse(case)
    th.assert_parity(out, lse, ref_o, ref_l, what="topk -> decode")


def test_topk_batched_shape_full_size():
    """32 requests of 143,360 positions, one query token each, k = 2048."""
    print("case: topk batched shape 32 x 143360, k=2048", flush=True)
    rng = np.random.default_rng(6)
    s = rng.standard_normal((32, 1, 143360)).astype(np.float32)
    got = _run(s, [143360] * 32, 1, 2048)
    assert np.array_equal(got, tk.topk_indices(s, [143360] * 32, 1, 2048))


def test_topk_mtp_shape_every_row():
    """16 requests x 15 query tokens of 149,504 positions (240 rows in one launch), each request
    with its own length; every row is compared with the oracle (the tie rule makes the selected
    list unique)."""
    print("case: topk MTP shape 16 x 15 x 149504, k=2048", flush=True)
    rng = np.random.default_rng(7)
    n = 149504
    s = rng.standard_normal((16, 15, n)).astype(np.float32)
    lens = [n - 97 * b for b in range(16)]
    got = _run(s, lens, 15, 2048)
    for b in range(16):
        for t in range(15):
            nv = min(tk.visible_count(lens[b], 15, t), n)
            assert np.array_equal(got[b, t], tk.select_topk(s[b, t], nv, 2048)), (b, t)
