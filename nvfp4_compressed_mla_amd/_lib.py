"""ctypes binding of ``libmla_nvfp4.so`` (declared in ``include/mla_nvfp4.h``).

Argument marshalling only: tensors are checked for dtype / device / layout and handed over as
device pointers with torch's current HIP stream. Every step of the computation runs in the HIP
library; if the library is missing this module raises instead of falling back to anything.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_nvfp4.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_BF16, MLA_FP32 = 0, 1
MLA_LAYOUT_BLOCK_MAJOR, MLA_LAYOUT_LAYER_MAJOR = 0, 1
ROW_BYTES = 352
FP8_ROW_BYTES = 576
PAGE_ROWS = 64
LATENT_DIM = 512
QK_DIM = 576

EXPORTED = [
    "mla_nvfp4_quantize_append",
    "mla_decode_workspace_size",
    "mla_sparse_decode_num_splits",
    "mla_dense_decode_num_splits",
    "mla_dense_decode_split_tokens",
    "mla_sparse_decode",
    "mla_sparse_decode_append",
    "mla_shared_decode_workspace_size",
    "mla_shared_decode_num_splits",
    "mla_sparse_decode_shared",
    "mla_dense_decode",
    "mla_nvfp4_dequantize_rows",
    "mla_fp8_append",
    "mla_fp8_sparse_decode",
    "mla_fp8_dense_decode",
    "mla_nvfp4_stage_fp8",
    "mla_staged_workspace_size",
    "mla_staged_sparse_decode",
    "mla_copy_kv_blocks",
    "mla_kv_transfer_regions",
    "mla_topk_workspace_size",
    "mla_topk_indices",
    "mla_indexer_scores",
    "mla_set_timing_events",
    "mla_status_string",
    "mla_last_error",
    "mla_set_debug_checks",
    "mla_debug_checks_enabled",
    "mla_check_sparse_indices",
    "mla_check_dense_tables",
    "mla_check_slots",
    "mla_noalloc_scratch_bytes",
    "mla_sparse_decode_noalloc",
]


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load and type the library (once). Raises FileNotFoundError if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m nvfp4_compressed_mla_amd.build`")
    try:
        # torch first: its HIP runtime then also serves this library (one runtime per process,
        # so torch streams and events are valid handles here)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.mla_nvfp4_quantize_append.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, vp]
    lib.mla_nvfp4_quantize_append.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [i32, i32, i32]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_sparse_decode_num_splits.argtypes = [i32, i32, i32, i32]
    lib.mla_sparse_decode_num_splits.restype = i32
    lib.mla_dense_decode_num_splits.argtypes = [i32, i32]
    lib.mla_dense_decode_num_splits.restype = i32
    lib.mla_dense_decode_split_tokens.argtypes = [i32, i32, i32]
    lib.mla_dense_decode_split_tokens.restype = i32
    lib.mla_sparse_decode.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i32, vp, i32, i32, i32,
                                      i32, f32, i32, vp, vp, vp, sz, vp]
    lib.mla_sparse_decode.restype = ctypes.c_int
    lib.mla_sparse_decode_append.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i32, vp, i32, i32,
                                             i32, i32, f32, i32, vp, i64, vp, i64, vp, vp, vp, vp,
                                             sz, vp]
    lib.mla_sparse_decode_append.restype = ctypes.c_int
    lib.mla_shared_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.mla_shared_decode_workspace_size.restype = sz
    lib.mla_shared_decode_num_splits.argtypes = [i32, i32, i32, i32]
    lib.mla_shared_decode_num_splits.restype = i32
    lib.mla_sparse_decode_shared.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i32, vp, i32, i32,
                                             i32, i32, f32, vp, vp, vp, sz, vp]
    lib.mla_sparse_decode_shared.restype = ctypes.c_int
    lib.mla_dense_decode.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i32, vp, i32, i32, i32,
                                     f32, i32, i32, vp, vp, vp, sz, vp]
    lib.mla_dense_decode.restype = ctypes.c_int
    lib.mla_nvfp4_dequantize_rows.argtypes = [vp, i64, i64, vp, i64, vp, vp]
    lib.mla_nvfp4_dequantize_rows.restype = ctypes.c_int
    lib.mla_fp8_append.argtypes = lib.mla_nvfp4_quantize_append.argtypes
    lib.mla_fp8_append.restype = ctypes.c_int
    lib.mla_fp8_sparse_decode.argtypes = lib.mla_sparse_decode.argtypes
    lib.mla_fp8_sparse_decode.restype = ctypes.c_int
    lib.mla_fp8_dense_decode.argtypes = lib.mla_dense_decode.argtypes
    lib.mla_fp8_dense_decode.restype = ctypes.c_int
    lib.mla_nvfp4_stage_fp8.argtypes = [vp, i64, i64, vp, i32, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.mla_nvfp4_stage_fp8.restype = ctypes.c_int
    lib.mla_staged_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.mla_staged_workspace_size.restype = sz
    lib.mla_staged_sparse_decode.argtypes = lib.mla_sparse_decode.argtypes
    lib.mla_staged_sparse_decode.restype = ctypes.c_int
    lib.mla_copy_kv_blocks.argtypes = [vp, i64, vp, i64, ctypes.c_int, i32, i64, vp, vp, i32, vp]
    lib.mla_copy_kv_blocks.restype = ctypes.c_int
    lib.mla_kv_transfer_regions.argtypes = [ctypes.c_int, i32, i64, i64, vp, i32]
    lib.mla_kv_transfer_regions.restype = i64
    lib.mla_topk_workspace_size.argtypes = [i32, i64, i32]
    lib.mla_topk_workspace_size.restype = sz
    lib.mla_topk_indices.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.mla_topk_indices.restype = ctypes.c_int
    lib.mla_indexer_scores.argtypes = [vp, vp, vp, i64, i64, vp, i32, vp, i32, i32, i64, vp, vp]
    lib.mla_indexer_scores.restype = ctypes.c_int
    lib.mla_set_timing_events.argtypes = [vp, vp]
    lib.mla_set_timing_events.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_set_debug_checks.argtypes = [i32]
    lib.mla_set_debug_checks.restype = ctypes.c_int
    lib.mla_debug_checks_enabled.argtypes = []
    lib.mla_debug_checks_enabled.restype = i32
    lib.mla_check_sparse_indices.argtypes = [vp, i32, i32, i32, vp, i32, i64, i64, i64]
    lib.mla_check_sparse_indices.restype = ctypes.c_int
    lib.mla_check_dense_tables.argtypes = [vp, i32, i32, vp, i32, i64, i64, i64]
    lib.mla_check_dense_tables.restype = ctypes.c_int
    lib.mla_check_slots.argtypes = [vp, i64, i64, i64, i64]
    lib.mla_check_slots.restype = ctypes.c_int
    lib.mla_noalloc_scratch_bytes.argtypes = []
    lib.mla_noalloc_scratch_bytes.restype = sz
    lib.mla_sparse_decode_noalloc.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, i32, vp, i32, i32,
                                              i32, i32, f32, i32, vp, vp, vp]
    lib.mla_sparse_decode_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return load_library().mla_status_string(s).decode()
    except Exception:
        return f"status {s}"


def _check(status: int) -> None:
    if status != MLA_OK:
        raise MlaError(status, load_library().mla_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype=None, device=True):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# ---- entry points (same names as the C ABI) --------------------------------------------------

def mla_nvfp4_quantize_append(latent, rope, slot_mapping, kv_cache, page_stride_bytes, stream=None):
    """Quantize bf16 latent [N,512] / rope [N,64] rows into the cache at ``slot_mapping`` (int64)."""
    _append("mla_nvfp4_quantize_append", latent, rope, slot_mapping, kv_cache, page_stride_bytes,
            stream)


def mla_fp8_append(latent, rope, slot_mapping, kv_cache, page_stride_bytes, stream=None):
    """Write bf16 latent [N,512] / rope [N,64] rows as 576-byte FP8 rows at ``slot_mapping``."""
    _append("mla_fp8_append", latent, rope, slot_mapping, kv_cache, page_stride_bytes, stream)


def _append(name, latent, rope, slot_mapping, kv_cache, page_stride_bytes, stream):
    torch = _torch()
    _require(latent, "latent", torch.bfloat16)
    _require(rope, "rope", torch.bfloat16)
    _require(slot_mapping, "slot_mapping", torch.int64)
    _require(kv_cache, "kv_cache", torch.uint8)
    if latent.dim() != 2 or latent.shape[1] != 512 or latent.stride(1) != 1:
        raise ValueError("latent must be [N, 512] with unit inner stride")
    if rope.dim() != 2 or rope.shape[1] != 64 or rope.stride(1) != 1 or rope.shape[0] != latent.shape[0]:
        raise ValueError("rope must be [N, 64] with unit inner stride")
    if not slot_mapping.is_contiguous() or slot_mapping.numel() != latent.shape[0]:
        raise ValueError("slot_mapping must be contiguous [N]")
    lib = load_library()
    _check(getattr(lib, name)(
        _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(slot_mapping),
        latent.shape[0], _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(), _stream(stream)))


def mla_decode_workspace_size(num_tokens: int, H: int, num_splits: int) -> int:
    return int(load_library().mla_decode_workspace_size(num_tokens, H, num_splits))


def mla_sparse_decode_num_splits(num_tokens: int, H: int, topk: int, max_splits: int = 0) -> int:
    return int(load_library().mla_sparse_decode_num_splits(num_tokens, H, topk, max_splits))


def mla_dense_decode_num_splits(max_pages: int, split_tokens: int) -> int:
    return int(load_library().mla_dense_decode_num_splits(max_pages, split_tokens))


def mla_dense_decode_split_tokens(num_tokens: int, H: int, max_pages: int) -> int:
    return int(load_library().mla_dense_decode_split_tokens(num_tokens, H, max_pages))


def _q_dtype(q):
    torch = _torch()
    if q.dtype == torch.bfloat16:
        return MLA_BF16
    if q.dtype == torch.float32:
        return MLA_FP32
    raise ValueError("q must be bf16 or fp32")


def _outputs(q, out, lse, want_lse):
    torch = _torch()
    B, q_len, H, _ = q.shape
    if out is None:
        out = torch.empty(B, q_len, H, LATENT_DIM, device=q.device, dtype=torch.float32)
    if lse is None and want_lse:
        lse = torch.empty(B, q_len, H, device=q.device, dtype=torch.float32)
    _require(out, "out", torch.float32)
    if not out.is_contiguous() or tuple(out.shape) != (B, q_len, H, LATENT_DIM):
        raise ValueError("out must be contiguous fp32 [B, q_len, H, 512]")
    if lse is not None and (not lse.is_contiguous() or tuple(lse.shape) != (B, q_len, H)):
        raise ValueError("lse must be contiguous fp32 [B, q_len, H]")
    return out, lse


def _workspace(workspace, n_tokens, H, splits, device):
    torch = _torch()
    need = mla_decode_workspace_size(n_tokens, H, splits)
    if need == 0:
        return workspace, 0 if workspace is None else workspace.numel()
    if workspace is None:
        workspace = torch.empty(need, device=device, dtype=torch.uint8)
    return workspace, workspace.numel()


def mla_sparse_decode(q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale,
                      out=None, lse=None, num_splits: int = 0, workspace=None, want_lse=True,
                      stream=None):
    """Sparse decode; returns (out fp32 [B,q_len,H,512], lse fp32 [B,q_len,H] or None).

    ``num_splits`` 0 picks the library's launch-shaping choice. ``workspace`` (uint8 device
    tensor) may be passed to keep the call free of allocations (graph capture).
    """
    return _sparse("mla_sparse_decode", q, kv_cache, page_stride_bytes, block_table, topk_idx,
                   softmax_scale, out, lse, num_splits, workspace, want_lse, stream)


def mla_sparse_decode_append(q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale,
                             latent, rope, slot_mapping, out=None, lse=None, num_splits: int = 0,
                             workspace=None, want_lse=True, stream=None):
    """Quantize-append of one new row per query token (``latent`` bf16 [B*q_len, 512], ``rope``
    bf16 [B*q_len, 64], ``slot_mapping`` int64 [B*q_len]) fused into the sparse decode: the same
    cache bytes and result as :func:`mla_nvfp4_quantize_append` then :func:`mla_sparse_decode`.
    Returns (out, lse)."""
    torch = _torch()
    _require(q, "q")
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(topk_idx, "topk_idx", torch.int32)
    _require(latent, "latent", torch.bfloat16)
    _require(rope, "rope", torch.bfloat16)
    _require(slot_mapping, "slot_mapping", torch.int64)
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, q_len, H, 576]")
    B, q_len, H, _ = q.shape
    if topk_idx.dim() != 3 or tuple(topk_idx.shape[:2]) != (B, q_len) or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous int32 [B, q_len, topk]")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    if latent.dim() != 2 or tuple(latent.shape) != (B * q_len, 512) or latent.stride(1) != 1:
        raise ValueError("latent must be [B*q_len, 512] with unit inner stride")
    if rope.dim() != 2 or tuple(rope.shape) != (B * q_len, 64) or rope.stride(1) != 1:
        raise ValueError("rope must be [B*q_len, 64] with unit inner stride")
    if not slot_mapping.is_contiguous() or slot_mapping.numel() != B * q_len:
        raise ValueError("slot_mapping must be contiguous int64 [B*q_len]")
    topk = topk_idx.shape[2]
    splits = num_splits or mla_sparse_decode_num_splits(B * q_len, H, topk, 0)
    out, lse = _outputs(q, out, lse, want_lse)
    workspace, ws_bytes = _workspace(workspace, B * q_len, H, splits, q.device)
    _check(load_library().mla_sparse_decode_append(
        _ptr(q), _q_dtype(q), _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(),
        _ptr(block_table), block_table.shape[1], _ptr(topk_idx), topk, B, q_len, H,
        float(softmax_scale), splits, _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0),
        _ptr(slot_mapping), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def mla_shared_decode_workspace_size(B: int, q_len: int, H: int, topk: int) -> int:
    return int(load_library().mla_shared_decode_workspace_size(B, q_len, H, topk))


def mla_shared_decode_num_splits(B: int, q_len: int, H: int, topk: int) -> int:
    return int(load_library().mla_shared_decode_num_splits(B, q_len, H, topk))


def mla_sparse_decode_shared(q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale,
                             out=None, lse=None, workspace=None, want_lse=True, stream=None):
    """Sparse decode with each distinct row of a group of up to 4 consecutive query tokens
    gathered and decoded once (same result as ``mla_sparse_decode``); returns (out, lse)."""
    torch = _torch()
    _require(q, "q")
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(topk_idx, "topk_idx", torch.int32)
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, q_len, H, 576]")
    B, q_len, H, _ = q.shape
    if topk_idx.dim() != 3 or tuple(topk_idx.shape[:2]) != (B, q_len) or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous int32 [B, q_len, topk]")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    topk = topk_idx.shape[2]
    out, lse = _outputs(q, out, lse, want_lse)
    need = mla_shared_decode_workspace_size(B, q_len, H, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    _check(load_library().mla_sparse_decode_shared(
        _ptr(q), _q_dtype(q), _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(),
        _ptr(block_table), block_table.shape[1], _ptr(topk_idx), topk, B, q_len, H,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out, lse


def mla_fp8_sparse_decode(q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale,
                          out=None, lse=None, num_splits: int = 0, workspace=None, want_lse=True,
                          stream=None):
    """Sparse decode over a cache of 576-byte FP8 rows; as :func:`mla_sparse_decode`."""
    return _sparse("mla_fp8_sparse_decode", q, kv_cache, page_stride_bytes, block_table, topk_idx,
                   softmax_scale, out, lse, num_splits, workspace, want_lse, stream)


def mla_staged_sparse_decode(q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale,
                             out=None, lse=None, num_splits: int = 0, workspace=None,
                             want_lse=True, stream=None):
    """The staged path over an NVFP4 cache: selected rows converted to FP8 in the workspace,
    then the FP8 kernel; arguments as :func:`mla_sparse_decode`."""
    return _sparse("mla_staged_sparse_decode", q, kv_cache, page_stride_bytes, block_table,
                   topk_idx, softmax_scale, out, lse, num_splits, workspace, want_lse, stream)


def mla_staged_workspace_size(num_tokens: int, H: int, topk: int, num_splits: int) -> int:
    return int(load_library().mla_staged_workspace_size(num_tokens, H, topk, num_splits))


def _sparse(name, q, kv_cache, page_stride_bytes, block_table, topk_idx, softmax_scale, out, lse,
            num_splits, workspace, want_lse, stream):
    torch = _torch()
    _require(q, "q")
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(topk_idx, "topk_idx", torch.int32)
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, q_len, H, 576]")
    B, q_len, H, _ = q.shape
    if topk_idx.dim() != 3 or tuple(topk_idx.shape[:2]) != (B, q_len) or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous int32 [B, q_len, topk]")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    topk = topk_idx.shape[2]
    splits = num_splits or mla_sparse_decode_num_splits(B * q_len, H, topk, 0)
    out, lse = _outputs(q, out, lse, want_lse)
    if name == "mla_staged_sparse_decode":
        need = mla_staged_workspace_size(B * q_len, H, topk, splits)
        if workspace is None:
            workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
        ws_bytes = workspace.numel()
    else:
        workspace, ws_bytes = _workspace(workspace, B * q_len, H, splits, q.device)
    lib = load_library()
    _check(getattr(lib, name)(
        _ptr(q), _q_dtype(q), _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(),
        _ptr(block_table), block_table.shape[1], _ptr(topk_idx), topk, B, q_len, H,
        float(softmax_scale), splits, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return out, lse


def mla_dense_decode(q, kv_cache, page_stride_bytes, block_table, seq_lens, softmax_scale,
                     split_tokens: int = 4096, out=None, lse=None, workspace=None, want_lse=True,
                     stream=None):
    """Dense decode over positions 0..seq_len-q_len+t; returns (out, lse).

    ``split_tokens``: positions per row split (a multiple of 64); 0 takes the library's split
    size that keeps the launch in one wave of workgroups (``mla_dense_decode_split_tokens``).
    """
    return _dense("mla_dense_decode", q, kv_cache, page_stride_bytes, block_table, seq_lens,
                  softmax_scale, split_tokens, out, lse, workspace, want_lse, stream)


def mla_fp8_dense_decode(q, kv_cache, page_stride_bytes, block_table, seq_lens, softmax_scale,
                         split_tokens: int = 4096, out=None, lse=None, workspace=None,
                         want_lse=True, stream=None):
    """Dense decode over a cache of 576-byte FP8 rows; as :func:`mla_dense_decode`."""
    return _dense("mla_fp8_dense_decode", q, kv_cache, page_stride_bytes, block_table, seq_lens,
                  softmax_scale, split_tokens, out, lse, workspace, want_lse, stream)


def _dense(name, q, kv_cache, page_stride_bytes, block_table, seq_lens, softmax_scale,
           split_tokens, out, lse, workspace, want_lse, stream):
    torch = _torch()
    _require(q, "q")
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 4 or q.shape[3] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, q_len, H, 576]")
    B, q_len, H, _ = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [B]")
    if split_tokens == 0:          # the library's one-wave split size for this shape
        split_tokens = mla_dense_decode_split_tokens(B * q_len, H, block_table.shape[1])
    splits = mla_dense_decode_num_splits(block_table.shape[1], split_tokens)
    out, lse = _outputs(q, out, lse, want_lse)
    workspace, ws_bytes = _workspace(workspace, B * q_len, H, splits, q.device)
    lib = load_library()
    _check(getattr(lib, name)(
        _ptr(q), _q_dtype(q), _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, q_len, H,
        float(softmax_scale), int(split_tokens), splits, _ptr(out), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return out, lse


def mla_nvfp4_dequantize_rows(kv_cache, page_stride_bytes, slots, stream=None):
    """Decode the rows at ``slots`` (int64) into fp32 [n, 576] with the on-chip decoder."""
    torch = _torch()
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(slots, "slots", torch.int64)
    slots = slots.contiguous()
    out = torch.empty(slots.numel(), QK_DIM, device=kv_cache.device, dtype=torch.float32)
    lib = load_library()
    _check(lib.mla_nvfp4_dequantize_rows(_ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(),
                                         _ptr(slots), slots.numel(), _ptr(out), _stream(stream)))
    return out


def mla_nvfp4_stage_fp8(kv_cache, page_stride_bytes, block_table, topk_idx, staged_rows=None,
                        staged_idx=None, staged_block_table=None, stream=None):
    """Convert the selected NVFP4 rows to 576-byte FP8 rows (the staging pass of the staged path).

    Returns (staged_rows uint8 [T*P*576], staged_idx int32 [T, topk], staged_block_table int32
    [T, P/64]) with T = B*q_len and P = topk rounded up to a multiple of 64.
    """
    torch = _torch()
    _require(kv_cache, "kv_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 3 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous int32 [B, q_len, topk]")
    B, q_len, topk = topk_idx.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    T, P = B * q_len, (topk + 63) // 64 * 64
    dev = kv_cache.device
    if staged_rows is None:
        staged_rows = torch.empty(T * P * FP8_ROW_BYTES, device=dev, dtype=torch.uint8)
    if staged_idx is None:
        staged_idx = torch.empty(T, topk, device=dev, dtype=torch.int32)
    if staged_block_table is None:
        staged_block_table = torch.empty(T, P // 64, device=dev, dtype=torch.int32)
    if staged_rows.numel() < T * P * FP8_ROW_BYTES or staged_idx.numel() != T * topk \
            or staged_block_table.numel() != T * (P // 64):
        raise ValueError("staged buffers have the wrong size")
    lib = load_library()
    _check(lib.mla_nvfp4_stage_fp8(
        _ptr(kv_cache), int(page_stride_bytes), kv_cache.numel(), _ptr(block_table),
        block_table.shape[1], _ptr(topk_idx), topk, B, q_len, _ptr(staged_rows), _ptr(staged_idx),
        _ptr(staged_block_table), _stream(stream)))
    return staged_rows, staged_idx, staged_block_table


def mla_copy_kv_blocks(src_pool, dst_pool, layout: int, n_layers: int, page_bytes: int,
                       src_blocks, dst_blocks, stream=None):
    """Copy all layer pages of src_blocks[i] of src_pool to dst_blocks[i] of dst_pool (uint8
    device pools of the given layout, int32 device block lists)."""
    torch = _torch()
    _require(src_pool, "src_pool", torch.uint8)
    _require(dst_pool, "dst_pool", torch.uint8)
    _require(src_blocks, "src_blocks", torch.int32)
    _require(dst_blocks, "dst_blocks", torch.int32)
    if src_blocks.numel() != dst_blocks.numel() or not src_blocks.is_contiguous() \
            or not dst_blocks.is_contiguous():
        raise ValueError("block lists must be contiguous and of equal length")
    _check(load_library().mla_copy_kv_blocks(
        _ptr(src_pool), src_pool.numel(), _ptr(dst_pool), dst_pool.numel(), int(layout),
        int(n_layers), int(page_bytes), _ptr(src_blocks), _ptr(dst_blocks), src_blocks.numel(),
        _stream(stream)))


def mla_kv_transfer_regions(layout: int, n_layers: int, page_bytes: int, pool_blocks: int,
                            blocks) -> int:
    """Contiguous byte ranges covering all pages of ``blocks`` (host sequence of block ids)."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32))
    n = int(load_library().mla_kv_transfer_regions(
        int(layout), int(n_layers), int(page_bytes), int(pool_blocks),
        arr.ctypes.data_as(ctypes.c_void_p), arr.size))
    if n < 0:
        raise MlaError(MLA_ERR_INVALID_ARG, "invalid layout arguments or block id outside the pool")
    return n


def mla_topk_workspace_size(num_tokens: int, n_max: int, k: int) -> int:
    return int(load_library().mla_topk_workspace_size(num_tokens, n_max, k))


def mla_topk_indices(scores, seq_lens, k: int, out=None, workspace=None, stream=None):
    """Top-k positions per query token from fp32 scores [B, q_len, n_max]; returns int32
    [B, q_len, k] (ascending positions, -1 padded)."""
    torch = _torch()
    _require(scores, "scores", torch.float32)
    _require(seq_lens, "seq_lens", torch.int32)
    if scores.dim() != 3 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous fp32 [B, q_len, n_max]")
    B, q_len, n_max = scores.shape
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [B]")
    if out is None:
        out = torch.empty(B, q_len, k, dtype=torch.int32, device=scores.device)
    need = mla_topk_workspace_size(B * q_len, n_max, k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=scores.device)
    _check(load_library().mla_topk_indices(
        _ptr(scores), n_max, _ptr(seq_lens), B, q_len, int(k), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


INDEXER_HEADS = 64
INDEXER_DIM = 128
INDEXER_PAGE_BYTES = 8448


def mla_indexer_scores(q_fp8, head_weights, k_cache, page_stride: int, block_table, seq_lens,
                       n_max: int = None, out=None, stream=None):
    """FP8 indexer scores [B, q_len, n_max] (fp32): q_fp8 uint8 [B, q_len, 64, 128] (E4M3 bytes),
    head_weights fp32 [B, q_len, 64], k_cache uint8 indexer pages (64 keys of 128 bytes, then 64
    fp32 scales per page). Positions a token may not select are left as they are in ``out``."""
    torch = _torch()
    _require(q_fp8, "q_fp8", torch.uint8)
    _require(head_weights, "head_weights", torch.float32)
    _require(k_cache, "k_cache", torch.uint8)
    _require(block_table, "block_table", torch.int32)
    _require(seq_lens, "seq_lens", torch.int32)
    if q_fp8.dim() != 4 or q_fp8.shape[2:] != (INDEXER_HEADS, INDEXER_DIM) or not q_fp8.is_contiguous():
        raise ValueError("q_fp8 must be contiguous uint8 [B, q_len, 64, 128]")
    B, q_len = q_fp8.shape[:2]
    if head_weights.shape != (B, q_len, INDEXER_HEADS) or not head_weights.is_contiguous():
        raise ValueError("head_weights must be contiguous fp32 [B, q_len, 64]")
    if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_pages]")
    if seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [B]")
    if n_max is None:
        n_max = block_table.shape[1] * 64
    if out is None:
        out = torch.zeros(B, q_len, n_max, dtype=torch.float32, device=q_fp8.device)
    elif out.shape != (B, q_len, n_max) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, q_len, n_max]")
    _check(load_library().mla_indexer_scores(
        _ptr(q_fp8), _ptr(head_weights), _ptr(k_cache), int(page_stride), k_cache.numel(),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, q_len, int(n_max), _ptr(out),
        _stream(stream)))
    return out


def mla_set_timing_events(start, stop) -> None:
    """Record raw HIP events (handles as ints / c_void_p, or None) around the fused decode kernel."""
    _check(load_library().mla_set_timing_events(start, stop))


def mla_set_debug_checks(enabled: bool) -> None:
    """Turn the library's opt-in content checks of index arrays on or off (off by default; the
    environment variable MLA_DEBUG_CHECKS=1 turns them on at the first call)."""
    _check(load_library().mla_set_debug_checks(1 if enabled else 0))


def mla_debug_checks_enabled() -> bool:
    return bool(load_library().mla_debug_checks_enabled())


def _host_i32(a):
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def mla_check_sparse_indices(topk_idx, block_table, page_stride_bytes, cache_bytes,
                             row_bytes=ROW_BYTES) -> None:
    """Host check of a sparse call's index list [B, q_len, topk] against its block table
    [B, max_pages] (host arrays); raises MlaError naming the first bad entry."""
    idx, bt = _host_i32(topk_idx), _host_i32(block_table)
    B, q_len, topk = idx.shape
    _check(load_library().mla_check_sparse_indices(
        idx.ctypes.data_as(ctypes.c_void_p), B, q_len, topk, bt.ctypes.data_as(ctypes.c_void_p),
        bt.shape[1], int(page_stride_bytes), int(cache_bytes), int(row_bytes)))


def mla_check_dense_tables(seq_lens, q_len, block_table, page_stride_bytes, cache_bytes,
                           row_bytes=ROW_BYTES) -> None:
    """Host check of a dense call's seq_lens [B] and block table [B, max_pages]."""
    sl, bt = _host_i32(seq_lens), _host_i32(block_table)
    _check(load_library().mla_check_dense_tables(
        sl.ctypes.data_as(ctypes.c_void_p), sl.size, int(q_len), bt.ctypes.data_as(ctypes.c_void_p),
        bt.shape[1], int(page_stride_bytes), int(cache_bytes), int(row_bytes)))


def mla_check_slots(slots, page_stride_bytes, cache_bytes, row_bytes=ROW_BYTES) -> None:
    """Host check of an append's slot_mapping (int64 host array)."""
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    _check(load_library().mla_check_slots(sl.ctypes.data_as(ctypes.c_void_p), sl.size,
                                          int(page_stride_bytes), int(cache_bytes), int(row_bytes)))
