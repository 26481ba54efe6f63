"""FP8 576-byte baseline row and the staged NVFP4 -> FP8 row conversion (fp64 / integer).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``); never imported by the product path.

[PI] section "Making room for low-latency decode": before the NVFP4 change a cache row held the
512-value latent and the 64-value rope part as FP8, 576 bytes. Section "Native NVFP4 sparse MLA
decode kernel" compares the fused NVFP4 kernel with (a) the existing FP8 attention kernel on such
rows and (b) a staged path that first unpacks the selected NVFP4 rows into a temporary FP8 buffer
and then runs that FP8 kernel.

Readings taken where the page is silent:

* The 576-byte row is bytes [0, 512) = E4M3 of latent element i at byte i, bytes [512, 576) =
  E4M3 of rope element j at byte 512 + j, scale 1 for both (there is no room for scales).
* E4M3 rounding is the same as for the NVFP4 scales: nearest, ties to even, saturating at 448.
* The staged conversion takes the exact NVFP4 value of each element (E2M1 code times E4M3 group
  scale) and rounds it to E4M3; rope bytes are already E4M3 and are copied.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import LATENT_DIM, ROPE_DIM, dequantize_rows, e4m3_decode, e4m3_encode

FP8_ROW_BYTES = LATENT_DIM + ROPE_DIM     # 576


def quantize_rows_fp8(latent, rope) -> np.ndarray:
    """Encode rows of (latent[512], rope[64]) real values into 576-byte FP8 rows."""
    x = np.asarray(latent, dtype=np.float64)
    r = np.asarray(rope, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != LATENT_DIM or r.shape != (x.shape[0], ROPE_DIM):
        raise ValueError("quantize_rows_fp8: expects latent [N,512] and rope [N,64]")
    row = np.zeros((x.shape[0], FP8_ROW_BYTES), dtype=np.uint8)
    row[:, :LATENT_DIM] = e4m3_encode(x)
    row[:, LATENT_DIM:] = e4m3_encode(r)
    return row


def dequantize_rows_fp8(rows):
    """Decode 576-byte FP8 rows into (latent [N,512], rope [N,64]) fp64 values (exact)."""
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.ndim != 2 or rows.shape[1] != FP8_ROW_BYTES:
        raise ValueError("dequantize_rows_fp8: expects uint8 [N,576]")
    return e4m3_decode(rows[:, :LATENT_DIM]), e4m3_decode(rows[:, LATENT_DIM:])


def nvfp4_rows_to_fp8(rows352) -> np.ndarray:
    """The staged conversion: exact NVFP4 values rounded to E4M3, as 576-byte rows."""
    lat, rope = dequantize_rows(rows352)
    return quantize_rows_fp8(lat, rope)
