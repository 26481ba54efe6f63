"""Pins of the oracle's NVFP4 / E4M3 row codec against facts fixed outside the oracle.

Pins used (none of them re-derives the oracle's own formula):
* the page's printed row sizes (576 -> 352 bytes),
* a row worked by hand from the OCP definitions (tests/golden/nvfp4_row_handworked.json),
* torch.float8_e4m3fn as an independent library implementation of E4M3,
* exact rational rounding (fractions.Fraction) for every bf16 group maximum,
* the closed-form E2M1 threshold table (exact products) for every bf16 value and every scale,
* exact round trips of grid values and the max-error bound of nearest rounding.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4 as nv
from oracle import cache as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_row_handworked.json")


def all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    vals = nv.bf16_bits_to_float(bits)
    return vals[np.isfinite(vals)]


# --- sizes printed on the page ([PI] "Making room for low-latency decode") ---------------------

def test_row_sizes_match_page():
    assert nv.FP8_ROW_BYTES == 576
    assert nv.ROW_BYTES == 352
    assert nv.ROW_BYTES == 512 // 2 + 512 // 16 + 64
    assert 64 * nv.ROW_BYTES == 22528   # one 64-token page


# --- E4M3 ---------------------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = nv.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                      # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))   # -0 keeps its sign


def test_e4m3_spot_values():
    d = nv.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x7E, 0x2C], dtype=np.uint8))
    assert list(d) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, 0.375]


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(nv.e4m3_encode(nv.e4m3_decode(codes)), codes)


def test_e4m3_midpoints_go_to_even_and_saturate():
    pos = np.array([c for c in range(0x7F)], dtype=np.uint8)
    v = nv.e4m3_decode(pos)
    mids = (v[:-1] + v[1:]) / 2
    got = nv.e4m3_encode(mids)
    expect = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, expect)
    # just off the midpoint goes to the nearer neighbour
    eps = (v[1:] - v[:-1]) / 1024
    assert np.array_equal(nv.e4m3_encode(mids - eps), pos[:-1])
    assert np.array_equal(nv.e4m3_encode(mids + eps), pos[1:])
    sat = nv.e4m3_encode(np.array([448.0, 460.0, 464.0, 1e6, -1e30]))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.uniform(-4, 2.5, 200000),
        rng.uniform(-463.9, 463.9, 20000),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464.0]          # torch turns overflow into NaN; the codec saturates
    ours = nv.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def _e4m3_exact(q: Fraction) -> int:
    """E4M3 round-to-nearest-even of an exact positive rational (Fraction), saturating."""
    if q >= 448:
        return 0x7E
    if q < Fraction(1, 64):
        m = round(q * 512)                    # Python rounds Fractions half to even
        return int(m)
    e = 0
    while q >= 2 ** (e + 1):
        e += 1
    while q < 2 ** e:
        e -= 1
    mant = round((q / Fraction(2) ** e - 1) * 8)
    if mant == 8:
        e, mant = e + 1, 0
    return ((e + 7) << 3) | int(mant)


def test_group_scale_exact_for_every_bf16_amax():
    vals = all_finite_bf16()
    amax = np.unique(vals[vals > 0])
    assert amax.size == 32639
    ours = nv.e4m3_encode(amax / 6.0)
    exact = np.array([_e4m3_exact(Fraction(float(a)) / 6) for a in amax], dtype=np.uint8)
    assert np.array_equal(ours, exact)
    # the tie the reading calls out: 6.375 / 6 = 1.0625 is a midpoint and goes to 1.0
    assert nv.e4m3_encode(np.array([6.375 / 6]))[0] == 0x38


# --- E2M1 ---------------------------------------------------------------------------------------

def test_e2m1_decode_table():
    vals = nv.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(vals[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(vals[8])


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16)
    assert np.array_equal(nv.e2m1_encode(nv.e2m1_decode(codes)), codes)


def _e2m1_threshold_code(a, s):
    """Closed-form E2M1 magnitude code of |x| = a against scale s, from the grid midpoints
    .25 .75 1.25 1.75 2.5 3.5 5 and the even-code tie rule (all products exact in fp64)."""
    return np.select(
        [a <= 0.25 * s, a < 0.75 * s, a <= 1.25 * s, a < 1.75 * s,
         a <= 2.5 * s, a < 3.5 * s, a <= 5.0 * s],
        [0, 1, 2, 3, 4, 5, 6], default=7)


def test_e2m1_nearest_matches_thresholds_exhaustive():
    x = all_finite_bf16()
    a = np.abs(x)
    sign = np.signbit(x).astype(np.int64) << 3
    scales = nv.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))   # every positive finite scale
    for s in scales:
        ours = nv.e2m1_encode(x / s).astype(np.int64)
        ref = _e2m1_threshold_code(a, s) | sign
        assert np.array_equal(ours, ref), f"scale {s}"


# --- rows ---------------------------------------------------------------------------------------

def _golden_row():
    g = json.load(open(GOLDEN))
    latent = np.zeros(512)
    codes = bytearray(256)
    scales = bytearray(32)
    for gi, grp in g["groups"].items():
        gi = int(gi)
        latent[16 * gi:16 * gi + 16] = np.array(grp["values"], dtype=np.float64)
        b = bytes.fromhex(grp["codes_hex"].replace(" ", ""))
        codes[8 * gi:8 * gi + 8] = b
        scales[gi] = int(grp["scale_hex"], 16)
    rope = np.zeros(64)
    rv = g["rope"]["values"]
    rope[:len(rv)] = rv
    rope_b = bytearray(64)
    rb = bytes.fromhex(g["rope"]["hex"].replace(" ", ""))
    rope_b[:len(rb)] = rb
    # negative zero entries must keep their sign when read from JSON
    for gi, grp in g["groups"].items():
        for i, v in enumerate(grp["values"]):
            if v == 0 and str(v).startswith("-"):
                latent[16 * int(gi) + i] = -0.0
    for i, v in enumerate(rv):
        if v == 0 and str(v).startswith("-"):
            rope[i] = -0.0
    expect = np.frombuffer(bytes(codes) + bytes(scales) + bytes(rope_b), dtype=np.uint8)
    return latent, rope, expect


def golden_row():
    """(latent[512], rope[64], expected 352 bytes) of the hand-worked fixture."""
    return _golden_row()


def test_quantize_matches_handworked_golden_row():
    latent, rope, expect = _golden_row()
    assert np.signbit(latent[4]) and np.signbit(rope[7])
    got = nv.quantize_rows(latent[None], rope[None])[0]
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, f"bytes differ at {bad[:8]}: got {got[bad[:8]]}, want {expect[bad[:8]]}"


def test_grid_rows_roundtrip_exactly():
    """Rows whose every group holds a +-6 code dequantize to values that re-encode identically."""
    rng = np.random.default_rng(11)
    n = 400
    codes = rng.integers(0, 16, size=(n, 512))
    codes[:, ::16] = rng.choice([7, 15], size=(n, 32))        # amax = 6 s in every group
    scales = rng.integers(1, 0x7F, size=(n, 32)).astype(np.uint8)
    # keep 6*s within E4M3 range after /6 (any finite s works since amax/6 == s exactly)
    rope = rng.integers(0, 256, size=(n, 64)).astype(np.uint8)
    rope[(rope & 0x7F) == 0x7F] = 0x00                          # no NaN codes
    row = np.zeros((n, 352), dtype=np.uint8)
    row[:, :256] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    row[:, 256:288] = scales
    row[:, 288:] = rope
    lat, rp = nv.dequantize_rows(row)
    again = nv.quantize_rows(lat, rp)
    assert np.array_equal(again, row)


def test_dequantize_error_bound_random_rows():
    """Nearest rounding: |x - deq| <= half the local grid gap times s, or the saturation excess."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 512)).astype(np.float32).astype(np.float64)
    r = rng.standard_normal((300, 64)).astype(np.float32).astype(np.float64)
    row = nv.quantize_rows(x, r)
    lat, rp = nv.dequantize_rows(row)
    s = np.repeat(nv.e4m3_decode(row[:, 256:288]), 16, axis=1)
    a = np.abs(x)
    half_gap = np.select([a <= 2 * s, a <= 4 * s], [0.25 * s, 0.5 * s], default=1.0 * s)
    excess = np.maximum(a - 6 * s, 0)
    assert np.all(np.abs(x - lat) <= half_gap + excess + 1e-300)
    # rope: E4M3 relative error <= 2^-4 in the normal range
    big = np.abs(r) >= 2.0 ** -6
    assert np.all(np.abs(r - rp)[big] <= np.abs(r)[big] * 2.0 ** -4)


def test_zero_and_tiny_groups():
    x = np.zeros((1, 512))
    x[0, 16:32] = [1e-4, -1e-4] * 8                  # amax/6 < 2^-10 -> scale 0
    x[0, 1] = -0.0
    row = nv.quantize_rows(x, np.zeros((1, 64)))[0]
    assert row[256] == 0 and row[257] == 0
    assert row[0] == 0x80                             # element 1 is -0 -> code 0x8 high nibble
    assert list(row[8:16]) == [0x80] * 8              # signs kept, magnitudes 0


def test_write_and_read_rows_through_pages():
    stride = 64 * 352 + 128            # a padded page stride
    cache = np.zeros(5 * stride, dtype=np.uint8)
    rows = np.arange(3 * 352, dtype=np.int64).reshape(3, 352).astype(np.uint8)
    bt = np.array([4, 1, 3])
    slots = [oc.logical_slot(bt, j) for j in (0, 70, 130)]
    oc.write_rows(cache, stride, slots + [-1], np.concatenate([rows, rows[:1]]))
    assert slots == [4 * 64, 64 + 6, 3 * 64 + 2]
    back = oc.read_rows(cache, stride, bt, [0, 70, 130])
    assert np.array_equal(back, rows)
    assert cache[4 * stride: 4 * stride + 352].tolist() == rows[0].tolist()
