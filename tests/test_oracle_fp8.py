"""Pins of the oracle's 576-byte FP8 baseline row and of the staged NVFP4 -> FP8 conversion.

Pins (none of them re-derives the oracle's own formula):
* rows and conversions worked by hand from the OCP definitions (tests/golden/fp8_handworked.json),
* torch.float8_e4m3fn as an independent implementation of E4M3 rounding (it returns NaN above
  the E4M3 range instead of saturating, so the comparison is restricted to |x| <= 448 and
  saturation is checked on its own),
* an exhaustive sweep of every (E2M1 code, finite scale byte) product, each product exact in
  fp64 and rounded by torch,
* the fp64 attention over an FP8 cache against the same attention over keys decoded by torch,
* the E4M3 half-ulp bound between staged FP8 values and the exact NVFP4 values.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import fp8 as f8
from oracle import nvfp4 as nv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_handworked.json")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def hexbytes(s):
    return [int(t, 16) for t in s.split()]


def test_fp8_row_size():
    assert f8.FP8_ROW_BYTES == 576 == nv.FP8_ROW_BYTES
    assert 64 * f8.FP8_ROW_BYTES == 36864


def test_fp8_row_matches_handworked_golden():
    g = json.load(open(GOLDEN))["fp8_row"]
    lat = np.zeros((1, 512))
    rope = np.zeros((1, 64))
    lat[0, g["latent"]["index"]] = g["latent"]["values"]
    rope[0, g["rope"]["index"]] = g["rope"]["values"]
    row = f8.quantize_rows_fp8(lat, rope)[0]
    want = np.zeros(576, dtype=np.uint8)
    want[g["latent"]["index"]] = hexbytes(g["latent"]["hex"])
    want[[512 + j for j in g["rope"]["index"]]] = hexbytes(g["rope"]["hex"])
    assert np.array_equal(row, want), np.nonzero(row != want)


def test_fp8_row_matches_torch_cast_in_range():
    rng = np.random.default_rng(5)
    lat = rng.standard_normal((64, 512)) * np.exp2(rng.integers(-12, 8, (64, 1)))
    rope = rng.standard_normal((64, 64)) * 30.0
    lat = np.clip(lat, -448, 448)
    rope = np.clip(rope, -448, 448)
    rows = f8.quantize_rows_fp8(lat, rope)
    assert np.array_equal(rows[:, :512], torch_e4m3(lat))
    assert np.array_equal(rows[:, 512:], torch_e4m3(rope))
    back_l, back_r = f8.dequantize_rows_fp8(rows)
    assert np.array_equal(back_l, torch_e4m3_value(rows[:, :512]))
    assert np.array_equal(back_r, torch_e4m3_value(rows[:, 512:]))


def test_fp8_row_saturates():
    lat = np.zeros((1, 512))
    lat[0, :4] = [449.0, 464.0, -1e6, 1e30]
    row = f8.quantize_rows_fp8(lat, np.zeros((1, 64)))[0]
    assert list(row[:4]) == [0x7E, 0x7E, 0xFE, 0x7E]


def _row_from_codes(codes16, scale_byte):
    """One 352-byte row whose group 0 holds the 16 given E2M1 codes and scale byte."""
    row = np.zeros(352, dtype=np.uint8)
    for k in range(8):
        row[k] = (codes16[2 * k] & 0xF) | ((codes16[2 * k + 1] & 0xF) << 4)
    row[256] = scale_byte
    return row


def test_staged_conversion_handworked():
    cases = json.load(open(GOLDEN))["staged"]["cases"]
    for c in cases:
        row = _row_from_codes([int(c["code"], 16)] + [0] * 15, int(c["scale"], 16))
        row[288:352] = np.arange(64, dtype=np.uint8) * 3     # rope bytes are copied as they are
        out = f8.nvfp4_rows_to_fp8(row[None])[0]
        assert out[0] == int(c["expect"], 16), (c, hex(out[0]))
        assert np.array_equal(out[512:], row[288:352])


def test_staged_conversion_every_code_and_scale():
    codes = np.arange(16)
    scales = [s for s in range(256) if s not in (0x7F, 0xFF) and not (s & 0x80)]
    rows = np.stack([_row_from_codes(codes, s) for s in scales])
    out = f8.nvfp4_rows_to_fp8(rows)[:, :16]
    for i, s in enumerate(scales):
        sv = torch_e4m3_value([s])[0]
        prod = np.array([(-1.0 if c & 8 else 1.0) * E2M1[c & 7] * sv for c in codes])  # exact
        want = torch_e4m3(np.clip(prod, -448.0, 448.0))
        assert np.array_equal(out[i], want), (hex(s), out[i], want)


def test_staged_values_within_half_ulp():
    rng = np.random.default_rng(9)
    lat = rng.standard_normal((32, 512)) * 0.3
    rope = rng.standard_normal((32, 64))
    rows = nv.quantize_rows(lat, rope)
    exact_l, exact_r = nv.dequantize_rows(rows)
    st_l, st_r = f8.dequantize_rows_fp8(f8.nvfp4_rows_to_fp8(rows))
    assert np.array_equal(st_r, exact_r)
    big = np.abs(exact_l) >= 2.0 ** -6
    rel = np.abs(st_l - exact_l)[big] / np.abs(exact_l)[big]
    assert rel.max() <= 2.0 ** -4
    assert np.all(np.abs(st_l - exact_l)[~big] <= 2.0 ** -10)


def test_sparse_decode_over_fp8_cache_against_torch_decoded_keys():
    rng = np.random.default_rng(11)
    page = 64 * 576
    ctx = [150, 70]
    n_pages = 5
    bt = np.array([[3, 0, 4], [1, 2, -1]], dtype=np.int64)
    cache = np.full(n_pages * page, 0xA5, dtype=np.uint8)
    all_rows = []
    for b, c in enumerate(ctx):
        rows = f8.quantize_rows_fp8(rng.standard_normal((c, 512)), rng.standard_normal((c, 64)) * 2)
        oc.write_rows(cache, page, [oc.logical_slot(bt[b], j) for j in range(c)], rows)
        all_rows.append(rows)
    q = rng.standard_normal((2, 1, 16, 576))
    idx = np.full((2, 1, 40), -1, dtype=np.int64)
    idx[0, 0, :40] = rng.choice(150, 40, replace=False)
    idx[1, 0, :25] = rng.choice(70, 25, replace=False)
    scale = 576 ** -0.5
    out, lse = oa.sparse_decode(q, cache, page, bt, idx, scale, row_bytes=576)
    for b in range(2):
        sel = idx[b, 0][idx[b, 0] >= 0]
        kv = torch_e4m3_value(all_rows[b][sel])
        want_o, want_l = oa.attend(q[b, 0], kv, kv[:, :512], scale)
        assert np.allclose(out[b, 0], want_o, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[b, 0], want_l, rtol=1e-12, atol=1e-12)
