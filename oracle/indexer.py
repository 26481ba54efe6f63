"""Indexer scores over an FP8 indexer cache: the scoring pass top-k selection reads (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Native NVFP4 sparse MLA decode kernel": attention reads the positions that a sparse
indexer selected for each query token; section "Decode: NVFP4 KV compression": at most 2048 per
query; section "Making room for low-latency decode": the indexer keeps its own cache state beside
the compressed MLA rows. The page gives no formula for the indexer's scores.

Reading taken (the plainest scoring that fits those statements; the inputs are synthetic, there
are no trained weights):

* every position s of a request holds a 128-dim indexer key k_s in E4M3 (OCP OFP8, decoded by
  ``nvfp4.e4m3_decode``) and a positive fp32 scale c_s;
* query token t has 64 indexer heads q_{t,j} (128 dims, E4M3) and real head weights w_{t,j};
* score[t, s] = c_s * sum_j w_{t,j} * max(0, q_{t,j} . k_s), computed here exactly in fp64 on
  the decoded values;
* token t of a request with seq_len positions and q_len query tokens scores positions
  0 .. seq_len - q_len + t (the window ``topk.topk_indices`` selects from);
* indexer page layout: 64 keys of 128 bytes, then the 64 scales as little-endian fp32 (8448
  bytes); position s of request b lives in page block_table[b][s // 64] at offset s % 64, the
  same table as the MLA rows. A page that is unmapped (negative) or not wholly inside the cache
  contributes keys and scales of zero.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import e4m3_decode

HEADS = 64
DIM = 128
PAGE_ROWS = 64
PAGE_BYTES = PAGE_ROWS * DIM + PAGE_ROWS * 4     # 8448
SCALE_OFF = PAGE_ROWS * DIM                      # 8192


def visible_count(seq_len: int, q_len: int, t: int) -> int:
    return max(0, int(seq_len) - int(q_len) + 1 + int(t))


def read_keys(cache: np.ndarray, page_stride: int, block_table_row, positions):
    """(E4M3 key bytes uint8 [n, 128], fp64 scales [n]) of the given logical positions."""
    pos = np.asarray(positions, dtype=np.int64)
    codes = np.zeros((pos.size, DIM), dtype=np.uint8)
    scales = np.zeros(pos.size, dtype=np.float64)
    bt = np.asarray(block_table_row, dtype=np.int64)
    for i, p in enumerate(pos.tolist()):
        page = int(bt[p // PAGE_ROWS])
        off = page * int(page_stride)
        if page < 0 or off + PAGE_BYTES > cache.size:
            continue
        r = p % PAGE_ROWS
        codes[i] = cache[off + r * DIM: off + (r + 1) * DIM]
        scales[i] = float(cache[off + SCALE_OFF + 4 * r: off + SCALE_OFF + 4 * r + 4].view("<f4")[0])
    return codes, scales


def scores_at(q_codes, weights, key_codes, key_scales):
    """Scores of one query token at n positions: q_codes uint8 [64, 128], weights [64],
    key_codes uint8 [n, 128], key_scales [n]. Returns fp64 [n]."""
    q = e4m3_decode(np.asarray(q_codes))                    # [64, 128]
    k = e4m3_decode(np.asarray(key_codes))                  # [n, 128]
    dots = q @ k.T                                          # [64, n] head scores
    w = np.asarray(weights, dtype=np.float64)
    return np.asarray(key_scales, dtype=np.float64) * (w @ np.maximum(dots, 0.0))


def score_magnitude_at(q_codes, weights, key_codes, key_scales):
    """c_s * sum_j |w_j| * sum_d |q_jd k_sd|: the scale of the rounding error an fp32
    evaluation of ``scores_at`` may make (used for tolerances)."""
    q = np.abs(e4m3_decode(np.asarray(q_codes)))
    k = np.abs(e4m3_decode(np.asarray(key_codes)))
    return np.abs(np.asarray(key_scales, dtype=np.float64)) * (np.abs(np.asarray(weights, dtype=np.float64)) @ (q @ k.T))


def indexer_scores(q_codes, weights, cache, page_stride, block_table, seq_lens, n_max, tokens=None):
    """Scores of the visible positions of each token.

    q_codes uint8 [B, q_len, 64, 128], weights [B, q_len, 64]. Returns (scores fp64
    [B, q_len, n_max], visible bool [B, q_len, n_max]); invisible entries are 0.
    ``tokens``: optional list of (b, t) to compute (the rest stay invisible).
    """
    q_codes = np.asarray(q_codes)
    B, q_len = q_codes.shape[:2]
    bt = np.asarray(block_table)
    cache = np.asarray(cache, dtype=np.uint8)
    out = np.zeros((B, q_len, n_max), dtype=np.float64)
    vis = np.zeros((B, q_len, n_max), dtype=bool)
    if tokens is None:
        tokens = [(b, t) for b in range(B) for t in range(q_len)]
    for b, t in tokens:
        n = min(visible_count(seq_lens[b], q_len, t), int(n_max), bt.shape[1] * PAGE_ROWS)
        if n <= 0:
            continue
        codes, scales = read_keys(cache, page_stride, bt[b], np.arange(n))
        out[b, t, :n] = scores_at(q_codes[b, t], weights[b, t], codes, scales)
        vis[b, t, :n] = True
    return out, vis
