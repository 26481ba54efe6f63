"""fp64 absorbed-MLA decode over NVFP4 rows: the plain softmax definition, no blocking.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

What is computed ([PI] section "Native NVFP4 sparse MLA decode kernel"): for each query token the
kernel reads the rows chosen by the sparse indexer, unpacks them, and computes attention over
them. The page gives no equations; the plainest reading of absorbed MLA decode with one shared
latent KV head is used:

* key of row j: ``K_j = [c_j ; r_j]`` (512 latent + 64 rope = 576 values),
* value of row j: ``V_j = c_j`` (the same latent; output stays in latent space),
* for head h: ``s_j = scale * (q_h . K_j)``, ``o_h = sum_j softmax(s)_j V_j``,
  ``lse_h = log sum_j exp(s_j)`` (natural log).

Readings (the page is silent or terse):

* One index list per query token, shared by all heads (the page selects rows per query token
  and splits that token's rows across blocks).
* Entry ``-1`` is an empty slot (subsection "Skip loads for empty slots"): it is not loaded and
  contributes no term; an all-empty list yields ``o = 0`` and ``lse = -inf``.
* Duplicated positions each contribute a term.
* Dense decode attends to positions ``0..seq_len-1``; with ``q_len > 1`` query token ``t`` sees
  positions ``j <= seq_len - q_len + t``.
* Splitting a token's rows across blocks and merging the blocks' partial results leaves the
  result equal to the unsplit softmax; ``lse_merge`` is that merge written out.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import LATENT_DIM, ROPE_DIM, ROW_BYTES, dequantize_rows
from .fp8 import FP8_ROW_BYTES, dequantize_rows_fp8
from .cache import read_rows

QK_DIM = LATENT_DIM + ROPE_DIM    # 576


def attend(q_heads, keys, values, softmax_scale):
    """Softmax attention of H query rows over n key/value rows, fp64.

    q_heads [H, 576], keys [n, 576], values [n, 512]. Returns (o [H, 512], lse [H]).
    With n == 0 returns o = 0 and lse = -inf.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    h = q_heads.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((h, values.shape[1])), np.full(h, -np.inf)
    s = softmax_scale * (q_heads @ keys.T)               # [H, n]
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=1, keepdims=True)
    o = (p @ values) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def rows_to_kv(rows):
    """Dequantize 352-byte NVFP4 rows (or 576-byte FP8 rows) into (K [n,576], V [n,512]) fp64."""
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.shape[1] == FP8_ROW_BYTES:
        lat, rope = dequantize_rows_fp8(rows)
    else:
        lat, rope = dequantize_rows(rows)
    return np.concatenate([lat, rope], axis=1), lat


def sparse_decode(q, cache, page_stride, block_table, topk_idx, softmax_scale, tokens=None,
                  row_bytes=ROW_BYTES):
    """Sparse decode: each query token attends to the rows its index list selects.

    q [B, q_len, H, 576] (real values), cache uint8 flat bytes, block_table int [B, max_pages],
    topk_idx int [B, q_len, k] (logical positions, -1 = empty).
    ``tokens``: optional list of (b, t) pairs to compute; the other outputs are left as NaN.
    ``row_bytes``: 352 for the NVFP4 cache, 576 for the FP8 baseline cache.
    Returns out fp64 [B, q_len, H, 512], lse fp64 [B, q_len, H].
    """
    q = np.asarray(q, dtype=np.float64)
    b_n, q_len, h, d = q.shape
    if d != QK_DIM:
        raise ValueError("sparse_decode: q last dim must be 576")
    out = np.full((b_n, q_len, h, LATENT_DIM), np.nan)
    lse = np.full((b_n, q_len, h), np.nan)
    todo = tokens if tokens is not None else [(b, t) for b in range(b_n) for t in range(q_len)]
    for b, t in todo:
        sel = [int(j) for j in np.asarray(topk_idx[b, t]).tolist() if j >= 0]
        rows = read_rows(cache, page_stride, block_table[b], sel, row_bytes)
        keys, values = rows_to_kv(rows)
        out[b, t], lse[b, t] = attend(q[b, t], keys, values, softmax_scale)
    return out, lse


def dense_positions(seq_len: int, q_len: int, t: int):
    """Positions visible to query token t of a q_len-token step over a seq_len-token context."""
    last = seq_len - q_len + t
    return list(range(0, max(0, last + 1)))


def dense_decode(q, cache, page_stride, block_table, seq_lens, softmax_scale, tokens=None,
                 row_bytes=ROW_BYTES):
    """Dense decode: query token t of request b attends to positions 0..seq_len-q_len+t.
    ``row_bytes``: 352 for the NVFP4 cache, 576 for the FP8 baseline cache."""
    q = np.asarray(q, dtype=np.float64)
    b_n, q_len, h, _ = q.shape
    out = np.full((b_n, q_len, h, LATENT_DIM), np.nan)
    lse = np.full((b_n, q_len, h), np.nan)
    todo = tokens if tokens is not None else [(b, t) for b in range(b_n) for t in range(q_len)]
    for b, t in todo:
        pos = dense_positions(int(seq_lens[b]), q_len, t)
        rows = read_rows(cache, page_stride, block_table[b], pos, row_bytes)
        keys, values = rows_to_kv(rows)
        out[b, t], lse[b, t] = attend(q[b, t], keys, values, softmax_scale)
    return out, lse


def lse_merge(parts):
    """Merge partial softmax results of disjoint row subsets.

    parts: list of (o [H, 512], lse [H]) for the same heads. With M = max_s lse_s,
    w_s = exp(lse_s - M): o = sum_s w_s o_s / sum_s w_s and lse = M + log sum_s w_s.
    Subsets with lse = -inf (no rows) get weight 0; if all are empty, o = 0 and lse = -inf.
    """
    lses = np.stack([p[1] for p in parts])               # [S, H]
    os_ = np.stack([p[0] for p in parts])                # [S, H, 512]
    m = np.max(lses, axis=0)                              # [H]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)   # [S, H]
    wsum = np.sum(w, axis=0)
    o = np.einsum("sh,shd->hd", w, os_) / np.where(wsum > 0, wsum, 1.0)[:, None]
    o = np.where(finite[:, None], o, 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    return o, lse


def row_relative_error(out, ref):
    """Per output row (last axis) ``max_i |out_i - ref_i| / max_i |ref_i|``."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.where(den > 0, den, 1.0)
