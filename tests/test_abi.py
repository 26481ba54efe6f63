"""The C-ABI library loads, exports every symbol its header declares, and rejects bad arguments
on the host before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from nvfp4_compressed_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)          # never dereferenced: validation fails first


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(mla_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mla_nvfp4_quantize_append", "mla_sparse_decode", "mla_dense_decode"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def _sparse(lib, **kw):
    a = dict(q=FAKE, q_dtype=0, cache=FAKE, stride=22528, cache_bytes=22528 * 4, bt=FAKE,
             max_pages=4, idx=FAKE, topk=256, B=1, q_len=1, H=16, scale=0.04, splits=1,
             out=FAKE, lse=None, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.mla_sparse_decode(a["q"], a["q_dtype"], a["cache"], a["stride"], a["cache_bytes"],
                                 a["bt"], a["max_pages"], a["idx"], a["topk"], a["B"], a["q_len"],
                                 a["H"], a["scale"], a["splits"], a["out"], a["lse"], a["ws"],
                                 a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(cache=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(idx=None), INVALID),
    (dict(out=None), INVALID),
    (dict(q_dtype=7), UNSUPPORTED),
    (dict(H=24), UNSUPPORTED),
    (dict(H=0), UNSUPPORTED),
    (dict(topk=0), UNSUPPORTED),
    (dict(topk=2049), UNSUPPORTED),
    (dict(stride=22528 - 16), INVALID),
    (dict(stride=22528 + 8), INVALID),
    (dict(cache=ctypes.c_void_p(0x10008)), INVALID),
    (dict(cache_bytes=100), INVALID),
    (dict(B=0), INVALID),
    (dict(q_len=0), INVALID),
    (dict(max_pages=0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(splits=0), INVALID),
    (dict(splits=4), WORKSPACE),
    (dict(splits=4, ws=ctypes.c_void_p(0x10040), ws_bytes=1 << 30), WORKSPACE),
    (dict(splits=4, ws=FAKE, ws_bytes=100), WORKSPACE),
])
def test_sparse_decode_rejects(lib, kw, code):
    assert _sparse(lib, **kw) == code
    assert lib.mla_last_error().decode() != ""


def test_dense_decode_rejects(lib):
    def call(**kw):
        a = dict(seq=FAKE, split=4096, splits=1, max_pages=4, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.mla_dense_decode(FAKE, 0, FAKE, 22528, 22528 * 4, FAKE, a["max_pages"], a["seq"],
                                    1, 1, 64, 0.04, a["split"], a["splits"], FAKE, None, a["ws"],
                                    a["ws_bytes"], None)
    assert call(seq=None) == INVALID
    assert call(split=100) == UNSUPPORTED
    assert call(split=16384) == UNSUPPORTED
    # must equal ceil(max_pages*64/split_tokens)
    assert call(splits=2, ws=FAKE, ws_bytes=1 << 30) == INVALID
    assert call(max_pages=200, split=4096, splits=4) == WORKSPACE


def test_quantize_append_rejects(lib):
    f = lib.mla_nvfp4_quantize_append
    assert f(FAKE, 512, FAKE, 64, FAKE, 0, FAKE, 22528, 22528, None) == OK        # n_rows = 0: no-op
    assert f(FAKE, 512, FAKE, 64, FAKE, -1, FAKE, 22528, 22528, None) == INVALID
    assert f(None, 512, FAKE, 64, FAKE, 5, FAKE, 22528, 22528, None) == INVALID
    assert f(FAKE, 500, FAKE, 64, FAKE, 5, FAKE, 22528, 22528, None) == INVALID
    assert f(FAKE, 516, FAKE, 64, FAKE, 5, FAKE, 22528, 22528, None) == INVALID
    assert f(FAKE, 512, FAKE, 32, FAKE, 5, FAKE, 22528, 22528, None) == INVALID
    assert f(FAKE, 512, FAKE, 64, FAKE, 5, None, 22528, 22528, None) == INVALID
    assert f(FAKE, 512, FAKE, 64, FAKE, 5, FAKE, 1000, 22528, None) == INVALID
    assert f(ctypes.c_void_p(0x10002), 512, FAKE, 64, FAKE, 5, FAKE, 22528, 22528, None) == INVALID


def test_dequantize_rows_rejects(lib):
    f = lib.mla_nvfp4_dequantize_rows
    assert f(FAKE, 22528, 22528, FAKE, 0, FAKE, None) == OK
    assert f(None, 22528, 22528, FAKE, 3, FAKE, None) == INVALID
    assert f(FAKE, 22528, 22528, None, 3, FAKE, None) == INVALID
    assert f(FAKE, 22528, 22528, FAKE, -2, FAKE, None) == INVALID


def test_launch_shaping(lib):
    # one wave of 256 compute units at 64 heads per workgroup
    assert lib.mla_sparse_decode_num_splits(32, 64, 2048, 0) == 8
    assert lib.mla_sparse_decode_num_splits(240, 64, 2048, 0) == 1
    assert lib.mla_sparse_decode_num_splits(1, 16, 256, 0) == 4        # >= 64 rows per split
    assert lib.mla_sparse_decode_num_splits(1, 64, 2048, 100) == 32
    assert lib.mla_dense_decode_num_splits(2336, 4096) == 37
    assert lib.mla_decode_workspace_size(32, 64, 1) == 0
    assert lib.mla_decode_workspace_size(32, 64, 8) == 32 * 8 * 64 * (512 * 2 + 4)
    assert lib.mla_status_string(3) == b"MLA_ERR_WORKSPACE"


def test_fp8_entry_points_reject(lib):
    f = lib.mla_fp8_append
    assert f(FAKE, 512, FAKE, 64, FAKE, 0, FAKE, 36864, 36864, None) == OK
    assert f(FAKE, 512, FAKE, 64, FAKE, 5, FAKE, 22528, 36864, None) == INVALID   # page < 64*576
    assert f(FAKE, 512, FAKE, 64, FAKE, 5, FAKE, 36864, 500, None) == INVALID     # < one row
    d = lib.mla_fp8_sparse_decode
    args = [FAKE, 0, FAKE, 36864, 36864 * 4, FAKE, 4, FAKE, 256, 1, 1, 16, 0.04, 1, FAKE, None,
            None, 0, None]
    bad = list(args)
    bad[3] = 22528                                   # an NVFP4 page stride is too small here
    assert d(*bad) == INVALID
    bad = list(args)
    bad[8] = 4096
    assert d(*bad) == UNSUPPORTED
    s = lib.mla_staged_sparse_decode
    nv = [FAKE, 0, FAKE, 22528, 22528 * 4, FAKE, 4, FAKE, 256, 1, 1, 16, 0.04, 1, FAKE, None,
          None, 0, None]
    assert s(*nv) == WORKSPACE                       # the staged path always needs a workspace
    nv[16], nv[17] = FAKE, 100
    assert s(*nv) == WORKSPACE
    g = lib.mla_nvfp4_stage_fp8
    assert g(FAKE, 22528, 22528 * 4, FAKE, 4, FAKE, 256, 1, 1, None, FAKE, FAKE, None) == INVALID
    assert g(FAKE, 22528, 22528 * 4, FAKE, 4, FAKE, 0, 1, 1, FAKE, FAKE, FAKE, None) == UNSUPPORTED


def test_staged_workspace_size(lib):
    T, H, k = 15, 16, 2048
    rows = T * k * 576
    idx = T * k * 4
    bt = (T * (k // 64) * 4 + 255) // 256 * 256
    assert lib.mla_staged_workspace_size(T, H, k, 1) == rows + idx + bt
    assert lib.mla_staged_workspace_size(T, H, k, 4) == rows + idx + bt + T * 4 * H * (512 * 2 + 4)
    # topk padded to whole 64-row pages
    assert lib.mla_staged_workspace_size(1, 16, 100, 1) == 128 * 576 + 512 + 256


def test_kv_layout_entry_points(lib):
    import numpy as np
    from oracle import layout as lo
    f = lib.mla_copy_kv_blocks
    P = 22528
    assert f(FAKE, 3 * P, FAKE, 3 * P, 0, 3, P, FAKE, FAKE, 0, None) == OK          # nothing to copy
    assert f(FAKE, 3 * P, FAKE, 3 * P, 2, 3, P, FAKE, FAKE, 1, None) == INVALID     # layout
    assert f(FAKE, 3 * P + 16, FAKE, 3 * P, 0, 3, P, FAKE, FAKE, 1, None) == INVALID  # not whole blocks
    assert f(FAKE, 3 * P, FAKE, 3 * P, 0, 3, P + 8, FAKE, FAKE, 1, None) == INVALID  # page multiple of 16
    assert f(None, 3 * P, FAKE, 3 * P, 0, 3, P, FAKE, FAKE, 1, None) == INVALID
    # descriptor counts against the oracle's merged ranges
    rng = np.random.default_rng(4)
    for layout in (0, 1):
        for blocks in ([5, 6, 7, 20], list(rng.choice(500, 60, replace=False)), list(range(100, 164))):
            arr = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32))
            n = lib.mla_kv_transfer_regions(layout, 7, P, 500, arr.ctypes.data_as(ctypes.c_void_p), arr.size)
            assert n == len(lo.transfer_regions(layout, blocks, 7, P, 500))
    bad = np.array([3, 500], dtype=np.int32)
    assert lib.mla_kv_transfer_regions(0, 7, P, 500, bad.ctypes.data_as(ctypes.c_void_p), 2) == -1


def test_topk_entry_point_rejects(lib):
    f = lib.mla_topk_indices
    ws = lib.mla_topk_workspace_size(4, 1000, 64)
    # one slice of 2048 positions per token: 8 segments of 256 (key, position) entries + counts
    assert ws == 4 * 8 * 256 * 8 + 4 * 8 * 4
    # 15 slices of 10,240 positions per token, 8 segments each, 32768 // 120 = 273 entries each
    assert lib.mla_topk_workspace_size(15, 149504, 2048) == 15 * 15 * 8 * (273 * 8 + 4)
    args = dict(s=FAKE, n=1000, sl=FAKE, B=2, q=2, k=64, o=FAKE, ws=FAKE, wb=1 << 20)
    def call(**kw):
        a = dict(args); a.update(kw)
        return f(a["s"], a["n"], a["sl"], a["B"], a["q"], a["k"], a["o"], a["ws"], a["wb"], None)
    assert call(s=None) == INVALID
    assert call(k=0) == UNSUPPORTED
    assert call(k=2049) == UNSUPPORTED
    assert call(n=(1 << 20) + 1) == UNSUPPORTED
    assert call(B=0) == INVALID
    assert call(wb=100) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == WORKSPACE


def test_overlap_list_generator():
    """The overlap-model input generator: distinct ascending positions, the stated share of one
    base set per request (host-side, no GPU)."""
    import numpy as np
    from nvfp4_compressed_mla_amd import workloads as wl
    idx = wl.gen_topk_overlap(3, 5, 64, [500, 200, 129], 0.75, 11, "cpu").numpy()
    for b in range(3):
        rows = [set(idx[b, t].tolist()) for t in range(5)]
        for t in range(5):
            assert len(rows[t]) == 64 and (np.diff(idx[b, t]) > 0).all()
            assert idx[b, t].min() >= 0 and idx[b, t].max() < [500, 200, 129][b]
        union = set().union(*rows)
        assert len(union) <= 64 + 5 * 16          # base set + 16 fresh positions per token
        inter = set.intersection(*rows)
        assert len(inter) <= 48
    with pytest.raises(ValueError):
        wl.gen_topk_overlap(1, 1, 64, [100], 0.5, 1, "cpu")


def test_dense_one_wave_split_helper(lib):
    """The dense split-size helper: one wave of 256 workgroups where the 8192-row cap allows."""
    f, ns = lib.mla_dense_decode_split_tokens, lib.mla_dense_decode_num_splits
    assert f(8, 64, 2339) == 4736 and ns(2339, 4736) == 32           # 8 x 32 = 256 workgroups
    for T, H, P in [(1, 16, 100), (3, 64, 2336), (8, 64, 2336), (16, 80, 3200), (64, 64, 500)]:
        st = f(T, H, P)
        assert st % 64 == 0 and 64 <= st <= 8192
        groups = -(-(H // 16) // 4)
        if st < 8192 and st > 64:
            assert T * groups * ns(P, st) <= 256
    assert f(0, 64, 10) == 4096 and f(4, 8, 10) == 4096



def test_indexer_entry_point_rejects(lib):
    f = lib.mla_indexer_scores
    args = dict(q=FAKE, w=FAKE, c=FAKE, stride=8448, cb=8448 * 4, bt=FAKE, mp=4, sl=FAKE, B=1, ql=2,
                n=256, s=FAKE)
    def call(**kw):
        a = dict(args); a.update(kw)
        return f(a["q"], a["w"], a["c"], a["stride"], a["cb"], a["bt"], a["mp"], a["sl"], a["B"],
                 a["ql"], a["n"], a["s"], None)
    for k in ("q", "w", "c", "bt", "sl", "s"):
        assert call(**{k: None}) == INVALID, k
    assert call(stride=8448 - 16) == INVALID          # smaller than a page
    assert call(stride=8448 + 8) == INVALID           # not a multiple of 16
    assert call(c=ctypes.c_void_p(0x10008)) == INVALID
    assert call(q=ctypes.c_void_p(0x10004)) == INVALID
    assert call(w=ctypes.c_void_p(0x10004)) == INVALID
    assert call(cb=100) == INVALID
    assert call(B=0) == INVALID and call(B=65536) == INVALID and call(ql=0) == INVALID
    assert call(mp=0) == INVALID
    assert call(n=0) == INVALID and call(n=(1 << 20) + 1) == INVALID


def test_shared_decode_entry_points(lib):
    f = lib.mla_sparse_decode_shared
    # 16 requests x 15 tokens -> 64 groups of 4; 4 splits at top-k 2048 (8,192-entry unions in
    # lists of at most 2,048 rows), 16 parts of 8,192 entries per group
    assert lib.mla_shared_decode_num_splits(16, 15, 16, 2048) == 4
    assert lib.mla_shared_decode_num_splits(1, 4, 16, 64) == 16
    n = 64 * 16 * 8192
    r256 = lambda b: (b + 255) // 256 * 256
    expect = r256(n * 4) + r256(n) + r256(64 * 16 * 4) + r256(240 * 4 * 16 * (512 * 2 + 4))
    assert lib.mla_shared_decode_workspace_size(16, 15, 16, 2048) == expect
    assert lib.mla_shared_decode_workspace_size(0, 15, 16, 2048) == 0
    args = dict(q=FAKE, qd=0, c=FAKE, stride=22528, cb=22528 * 4, bt=FAKE, mp=4, idx=FAKE, k=256,
                B=1, ql=4, H=16, sc=0.04, out=FAKE, lse=None, ws=FAKE, wb=1 << 30)
    def call(**kw):
        a = dict(args); a.update(kw)
        return f(a["q"], a["qd"], a["c"], a["stride"], a["cb"], a["bt"], a["mp"], a["idx"], a["k"],
                 a["B"], a["ql"], a["H"], a["sc"], a["out"], a["lse"], a["ws"], a["wb"], None)
    assert call(idx=None) == INVALID
    assert call(q=None) == INVALID
    assert call(k=0) == UNSUPPORTED and call(k=2049) == UNSUPPORTED
    assert call(H=24) == UNSUPPORTED
    assert call(mp=16385) == UNSUPPORTED              # more than 2^20 positions
    assert call(ws=None) == WORKSPACE
    assert call(wb=1024) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == WORKSPACE


def test_fused_append_decode_entry_point_rejects(lib):
    f = lib.mla_sparse_decode_append
    args = dict(q=FAKE, qd=0, c=FAKE, stride=22528, cb=22528 * 4, bt=FAKE, mp=4, idx=FAKE, k=256,
                B=1, ql=2, H=16, sc=0.04, S=2, lat=FAKE, ls=512, rope=FAKE, rs=64, slots=FAKE,
                out=FAKE, lse=None, ws=FAKE, wb=1 << 30)

    def call(**kw):
        a = dict(args); a.update(kw)
        return f(a["q"], a["qd"], a["c"], a["stride"], a["cb"], a["bt"], a["mp"], a["idx"], a["k"],
                 a["B"], a["ql"], a["H"], a["sc"], a["S"], a["lat"], a["ls"], a["rope"], a["rs"],
                 a["slots"], a["out"], a["lse"], a["ws"], a["wb"], None)
    assert call(lat=None) == INVALID and call(rope=None) == INVALID and call(slots=None) == INVALID
    assert call(ls=500) == INVALID and call(rs=32) == INVALID
    assert call(lat=ctypes.c_void_p(0x10008)) == INVALID           # latent not 16-byte aligned
    assert call(slots=ctypes.c_void_p(0x10004)) == INVALID         # slots not 8-byte aligned
    assert call(ql=17) == UNSUPPORTED                              # q_len above 16
    assert call(ws=None) == WORKSPACE                              # two splits keep partials
    assert call(wb=1024) == WORKSPACE
    assert call(idx=None) == INVALID and call(k=2049) == UNSUPPORTED
