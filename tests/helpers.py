"""Shared test plumbing: build a paged cache case on the GPU and its oracle reference on the CPU.

The oracle side never sees anything the HIP path produced: it re-quantizes the same bf16 inputs
(drawn by the seeded generators) with ``oracle.nvfp4`` and places them with ``oracle.cache``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from nvfp4_compressed_mla_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import fp8 as f8
from oracle import nvfp4 as nv

PAGE_BYTES = 64 * 352
FP8_PAGE_BYTES = 64 * 576
ROW_TOL = 2e-3          # max over a row of |out - ref| / max |ref|, the stated parity bar
LSE_TOL = 2e-3          # absolute, natural log


@dataclass
class Case:
    B: int
    q_len: int
    H: int
    ctx: list
    topk: int
    page_stride: int
    latent: torch.Tensor        # bf16 [sum ctx, 512] on device, request-major
    rope: torch.Tensor          # bf16 [sum ctx, 64]
    row_base: list              # first latent row of each request
    block_table: torch.Tensor   # int32 [B, max_pages]
    n_pages: int
    cache: torch.Tensor         # uint8 [n_pages * page_stride] (GPU-quantized)
    q: torch.Tensor             # [B, q_len, H, 576]
    topk_idx: torch.Tensor      # int32 [B, q_len, topk] (None for dense)
    seq_lens: torch.Tensor      # int32 [B]
    fmt: str = "nvfp4"          # "nvfp4" (352-byte rows) or "fp8" (576-byte rows)

    @property
    def row_bytes(self) -> int:
        return 576 if self.fmt == "fp8" else 352


def softmax_scale() -> float:
    return 1.0 / math.sqrt(576.0)


def build_case(B, q_len, H, ctx, topk, seed, q_dtype="bf16", page_stride=None,
               device="cuda", spare_pages=3, topk_fn=None, append_rows=0, fmt="nvfp4"):
    """Generate inputs on the device and quantize them into a paged cache with the HIP path.

    ``append_rows`` > 0 writes the last ``append_rows`` positions of every request with a second
    quantize-append call covering all requests at once (a serving step's append), after the
    history rows. ``fmt`` "fp8" writes 576-byte FP8 rows instead of NVFP4 rows.
    """
    import nvfp4_compressed_mla_amd as m
    if page_stride is None:
        page_stride = FP8_PAGE_BYTES if fmt == "fp8" else PAGE_BYTES
    mla_nvfp4_quantize_append = m.mla_fp8_append if fmt == "fp8" else m.mla_nvfp4_quantize_append
    ctx = list(ctx)
    total = sum(ctx)
    latent, rope = wl.gen_latent_rope(total, seed, device)
    bt, n_pages = wl.gen_block_table(ctx, seed + 1, device, spare_pages=spare_pages)
    cache = torch.zeros(n_pages * page_stride, dtype=torch.uint8, device=device)
    row_base = [0]
    for c in ctx[:-1]:
        row_base.append(row_base[-1] + c)
    hist = [c - append_rows for c in ctx]
    if min(hist) < 0:
        raise ValueError("append_rows exceeds a context length")
    slots = torch.cat([wl.slot_mapping_for(bt, b, 0, c) for b, c in enumerate(hist)])
    if append_rows:
        rows = torch.cat([torch.arange(row_base[b], row_base[b] + c, device=device)
                          for b, c in enumerate(hist)])
        mla_nvfp4_quantize_append(latent[rows], rope[rows], slots, cache, page_stride)
    else:
        mla_nvfp4_quantize_append(latent, rope, slots, cache, page_stride)
    if append_rows:
        slots = torch.cat([wl.slot_mapping_for(bt, b, hist[b], append_rows) for b in range(B)])
        rows = torch.cat([torch.arange(row_base[b] + hist[b], row_base[b] + ctx[b], device=device)
                          for b in range(B)])
        mla_nvfp4_quantize_append(latent[rows], rope[rows], slots, cache, page_stride)
    q = wl.gen_queries(B, q_len, H, q_dtype, seed + 2, device)
    idx = None
    if topk:
        idx = (topk_fn or wl.gen_topk)(B, q_len, topk, ctx, seed + 3, device)
    seq = torch.tensor(ctx, dtype=torch.int32, device=device)
    return Case(B, q_len, H, ctx, topk, page_stride, latent, rope, row_base, bt, n_pages, cache,
                q, idx, seq, fmt)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_cache(case: Case, positions_per_request=None) -> np.ndarray:
    """The oracle's own cache: its quantization of the same bf16 rows, placed by its addressing.

    ``positions_per_request``: optional {b: iterable of logical positions}; only those rows are
    quantized (the rest of the cache stays zero), which keeps full-size sampled checks cheap.
    """
    cache = np.zeros(case.n_pages * case.page_stride, dtype=np.uint8)
    bt = case.block_table.cpu().numpy()
    for b, c in enumerate(case.ctx):
        if positions_per_request is None:
            pos = np.arange(c)
        else:
            pos = np.array(sorted(set(int(p) for p in positions_per_request.get(b, []))), dtype=np.int64)
            if pos.size == 0:
                continue
        rows_lat = bf16_to_f64(case.latent[case.row_base[b] + torch.as_tensor(pos, device=case.latent.device)])
        rows_rope = bf16_to_f64(case.rope[case.row_base[b] + torch.as_tensor(pos, device=case.rope.device)])
        enc = (f8.quantize_rows_fp8 if case.fmt == "fp8" else nv.quantize_rows)(rows_lat, rows_rope)
        slots = [oc.logical_slot(bt[b], int(j)) for j in pos]
        oc.write_rows(cache, case.page_stride, slots, enc)
    return cache


def oracle_sparse(case: Case, tokens=None, cache=None):
    if cache is None:
        cache = oracle_cache(case)
    q = case.q.detach().float().cpu().numpy().astype(np.float64)
    return oa.sparse_decode(q, cache, case.page_stride, case.block_table.cpu().numpy(),
                            case.topk_idx.cpu().numpy(), softmax_scale(), tokens=tokens,
                            row_bytes=case.row_bytes)


def oracle_dense(case: Case, tokens=None, cache=None):
    if cache is None:
        cache = oracle_cache(case)
    q = case.q.detach().float().cpu().numpy().astype(np.float64)
    return oa.dense_decode(q, cache, case.page_stride, case.block_table.cpu().numpy(),
                           case.seq_lens.cpu().numpy(), softmax_scale(), tokens=tokens,
                           row_bytes=case.row_bytes)


def oracle_staged_cache(case: Case, cache=None) -> np.ndarray:
    """The staged path's FP8 rows, by the oracle: each row of the oracle's NVFP4 cache converted
    to a 576-byte FP8 row at the same slot of a cache with 64*576-byte pages."""
    if cache is None:
        cache = oracle_cache(case)
    n_slots = case.n_pages * 64
    out = np.zeros(case.n_pages * FP8_PAGE_BYTES, dtype=np.uint8)
    rows = np.stack([cache[oc.row_offset(s, case.page_stride):oc.row_offset(s, case.page_stride) + 352]
                     for s in range(n_slots)])
    oc.write_rows(out, FP8_PAGE_BYTES, np.arange(n_slots), f8.nvfp4_rows_to_fp8(rows))
    return out


def assert_parity(out, lse, ref_out, ref_lse, tokens=None, what=""):
    """Row-wise relative error <= ROW_TOL and |lse - ref| <= LSE_TOL on the given tokens.

    Every compared value must be finite where the reference is: a NaN or infinite output row, or
    a NaN / wrongly infinite lse, fails (the errors are checked with ``np.isfinite`` before they
    are folded, so a NaN can never be dropped by the fold). A token whose reference lse is -inf
    (an empty list) must have exactly zero outputs and lse -inf.
    """
    out = out.detach().cpu().numpy().astype(np.float64)
    lse = lse.detach().cpu().numpy().astype(np.float64)
    if tokens is None:
        tokens = [(b, t) for b in range(out.shape[0]) for t in range(out.shape[1])]
    worst = 0.0
    worst_lse = 0.0
    for b, t in tokens:
        err = oa.row_relative_error(out[b, t], ref_out[b, t])
        if not np.all(np.isfinite(err)):
            bad = np.flatnonzero(~np.isfinite(err))
            raise AssertionError(f"{what}: token ({b}, {t}) heads {bad[:8].tolist()} have "
                                 f"non-finite outputs or errors")
        worst = max(worst, float(np.max(err)))
        rl, gl = ref_lse[b, t], lse[b, t]
        both_inf = np.isneginf(rl) & np.isneginf(gl)
        with np.errstate(invalid="ignore"):
            d = np.where(both_inf, 0.0, np.abs(gl - rl))
        if not np.all(np.isfinite(d)):
            bad = np.flatnonzero(~np.isfinite(d))
            raise AssertionError(f"{what}: token ({b}, {t}) heads {bad[:8].tolist()} have lse "
                                 f"{gl[bad[:4]].tolist()} against {rl[bad[:4]].tolist()}")
        worst_lse = max(worst_lse, float(np.max(d)))
        if np.any(np.isneginf(rl)):
            assert np.all(out[b, t][np.isneginf(rl)] == 0), f"{what}: empty rows must be zero"
    assert worst <= ROW_TOL, f"{what}: row relative error {worst:.3e} > {ROW_TOL}"
    assert worst_lse <= LSE_TOL, f"{what}: lse error {worst_lse:.3e} > {LSE_TOL}"
    return worst, worst_lse
