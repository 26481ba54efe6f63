"""Top-k selection of context positions from per-position scores (the step before the path).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Native NVFP4 sparse MLA decode kernel": the sparse indexer selects, for every query
token, the positions attention will read (2048 per token); unused slots of the list hold -1. The
page does not define the indexer's scoring function, so the scores are an input here.

Readings taken:

* token t of request b (q_len tokens per step) may select positions 0 .. seq_len - q_len + t
  (the causal window of the dense path);
* the k positions with the largest scores are selected; scores are ordered by IEEE-754
  totalOrder of the float32 value (so -0 ranks below +0), and equal scores by position, smaller
  first; scores are finite;
* the list holds the selected positions in ascending order, then -1 up to k entries.
"""

from __future__ import annotations

import numpy as np


def visible_count(seq_len: int, q_len: int, t: int) -> int:
    return max(0, int(seq_len) - int(q_len) + 1 + int(t))


def select_topk(scores, n: int, k: int) -> np.ndarray:
    """Selected positions (ascending) among scores[0:n], padded with -1 to k entries."""
    v = np.asarray(scores, dtype=np.float32)[:n]
    pos = np.arange(n)
    # lexsort: last key is primary -> value descending, then +0 before -0, then position
    order = np.lexsort((pos, np.signbit(v).astype(np.int8), -v.astype(np.float64)))
    chosen = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.size] = chosen
    return out


def topk_indices(scores, seq_lens, q_len: int, k: int) -> np.ndarray:
    """scores float32 [B, q_len, n_max]; returns int64 [B, q_len, k]."""
    scores = np.asarray(scores, dtype=np.float32)
    B = scores.shape[0]
    out = np.empty((B, q_len, k), dtype=np.int64)
    for b in range(B):
        for t in range(q_len):
            n = min(visible_count(seq_lens[b], q_len, t), scores.shape[2])
            out[b, t] = select_topk(scores[b, t], n, k)
    return out
