"""NVFP4 latent + FP8 rope row codec, written from the format definitions (fp64 / integer).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

Row format, [PI] section "Making room for low-latency decode": a cache row holds the 512-value
latent as 4-bit values with one FP8 scale per 16 values (512/2 + 512/16 = 288 bytes) and the
64-value rope part as FP8 (64 bytes): 352 bytes, against 512 + 64 = 576 bytes for an all-FP8 row.

Readings taken where the page is silent, each with its reason:

* FP8 is OCP E4M3 (E4M3FN): bias 7, max 448, code 0x7F/0xFF is NaN, no infinities.
* The 4-bit element is OCP MX FP4 E2M1.
* Group scale: ``s = E4M3(amax / 6)``, round-to-nearest-even, saturating at 448, no second-level
  per-tensor scale (the 352-byte budget has no room for one).
* Element code: round ``x / s`` to the nearest E2M1 value, ties to the even code, saturating at 6.
  When ``s`` decodes to 0 every magnitude is 0 and the sign bit is kept.
* Rope: plain E4M3 of the value, scale 1.
* Byte order inside the row: bytes [0, 256) hold the element codes with element 2k in the low
  nibble of byte k; bytes [256, 288) hold the 32 group scales in group order; bytes [288, 352)
  hold the 64 rope bytes.
* Negative zero keeps its sign bit (E2M1 code 0x8, E4M3 byte 0x80).
"""

from __future__ import annotations

import numpy as np

LATENT_DIM = 512
ROPE_DIM = 64
GROUP = 16
N_GROUPS = LATENT_DIM // GROUP          # 32
CODE_BYTES = LATENT_DIM // 2            # 256: two 4-bit codes per byte
SCALE_BYTES = N_GROUPS                  # 32: one FP8 scale per 16 values
ROPE_BYTES = ROPE_DIM                   # 64: one FP8 byte per rope value
ROW_BYTES = CODE_BYTES + SCALE_BYTES + ROPE_BYTES   # 352
FP8_ROW_BYTES = LATENT_DIM + ROPE_DIM                # 576, the all-FP8 row it replaces

E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ----------------------------------------------------------------------------------------------
# E4M3 (OCP OFP8): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
# ----------------------------------------------------------------------------------------------

def e4m3_decode(code) -> np.ndarray:
    """Value of each E4M3 byte, by the OFP8 definition. NaN for the two NaN codes."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    subnormal = m / 8.0 * 2.0 ** -6
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Round each real value to the nearest E4M3 value, ties to even, saturating to +-448.

    The rounding is done on the exact fp64 value of ``x``: the exponent comes from ``frexp`` and
    the mantissa fraction is scaled by a power of two, so the only rounding is the final
    round-half-even of the 3-bit mantissa (``np.rint``). Non-finite input raises.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input is outside the codec's domain")
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range a < 2^-6: the grid step is 2^-9, code = round(a / 2^-9) in 0..8
    # (8 lands on the smallest normal 2^-6, whose code is also 8).
    sub = a < 2.0 ** -6
    code = np.where(sub, np.rint(np.ldexp(np.where(sub, a, 0.0), 9)).astype(np.int64), code)

    # Normal range: a = 2^e * (1 + f), f in [0, 1); mantissa = round(8 f).
    frac, ex = np.frexp(np.where(sub, 1.0, a))       # a = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1
    mant = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    ncode = ((e + 7) << 3) | mant
    code = np.where(sub, code, ncode)

    # Saturation: anything at or above the largest finite value maps to it (0x7E = 448).
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# E2M1 (OCP MX FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
# ----------------------------------------------------------------------------------------------

def e2m1_decode(code) -> np.ndarray:
    """Value of each 4-bit E2M1 code (low 4 bits of the input), by the MX definition."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int64)))
    return sign * mag


_E2M1_GRID = e2m1_decode(np.arange(8))   # magnitudes of codes 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code for each real value, ties to the even code, saturating at 6.

    Nearest-grid search written out: for |v| below 6 take the grid neighbours g[i] <= |v| < g[i+1]
    and keep the closer one; on an exact tie keep the one whose code is even.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 3
    a = np.abs(v)
    lo = np.searchsorted(_E2M1_GRID, a, side="right") - 1     # g[lo] <= a
    lo = np.clip(lo, 0, 7)
    hi = np.clip(lo + 1, 0, 7)
    d_lo = a - _E2M1_GRID[lo]
    d_hi = _E2M1_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= E2M1_MAX, 7, mag)
    return (mag | sign).astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# Row codec.
# ----------------------------------------------------------------------------------------------

def quantize_rows(latent, rope) -> np.ndarray:
    """Encode rows of (latent[512], rope[64]) real values into 352-byte NVFP4 rows.

    Per 16-value group g: ``amax = max |x|``, ``s = E4M3(amax / 6)``; each element code is
    ``E2M1(x / dec(s))``; when ``dec(s) == 0`` all magnitudes are 0 with signs kept.
    Rope bytes are ``E4M3(r)``.
    """
    x = np.asarray(latent, dtype=np.float64)
    r = np.asarray(rope, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != LATENT_DIM or r.shape != (x.shape[0], ROPE_DIM):
        raise ValueError("quantize_rows: expects latent [N,512] and rope [N,64]")
    if not (np.all(np.isfinite(x)) and np.all(np.isfinite(r))):
        raise ValueError("quantize_rows: non-finite input is outside the codec's domain")
    n = x.shape[0]
    xg = x.reshape(n, N_GROUPS, GROUP)
    amax = np.max(np.abs(xg), axis=2)
    scale_code = e4m3_encode(amax / 6.0)                    # [n, 32]
    s = e4m3_decode(scale_code)                             # >= 0, finite
    zero_scale = (s == 0.0)[:, :, None]
    ratio = xg / np.where(zero_scale, 1.0, s[:, :, None])
    codes = e2m1_encode(ratio).astype(np.int64)
    codes = np.where(zero_scale, codes & 0x8, codes)        # magnitude 0, sign kept
    codes = codes.reshape(n, LATENT_DIM)

    row = np.zeros((n, ROW_BYTES), dtype=np.uint8)
    row[:, :CODE_BYTES] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    row[:, CODE_BYTES:CODE_BYTES + SCALE_BYTES] = scale_code
    row[:, CODE_BYTES + SCALE_BYTES:] = e4m3_encode(r)
    return row


def unpack_row_fields(rows):
    """Split 352-byte rows into (element codes [N,512], scale bytes [N,32], rope bytes [N,64])."""
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.ndim != 2 or rows.shape[1] != ROW_BYTES:
        raise ValueError("unpack_row_fields: expects uint8 [N,352]")
    packed = rows[:, :CODE_BYTES].astype(np.int64)
    codes = np.empty((rows.shape[0], LATENT_DIM), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    return codes, rows[:, CODE_BYTES:CODE_BYTES + SCALE_BYTES], rows[:, CODE_BYTES + SCALE_BYTES:]


def dequantize_rows(rows):
    """Decode 352-byte rows into (latent [N,512], rope [N,64]) fp64 values.

    ``latent[i] = E2M1(code_i) * E4M3(scale_{i // 16})`` and ``rope[j] = E4M3(rope_j)``; both are
    exact in fp64.
    """
    codes, scales, rope = unpack_row_fields(rows)
    s = e4m3_decode(scales)                                  # [N, 32]
    lat = e2m1_decode(codes) * np.repeat(s, GROUP, axis=1)
    return lat, e4m3_decode(rope)


def bf16_bits_to_float(bits) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns (uint16): the bf16 word is the top half of fp32."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)
