"""Host checks of the arithmetic shortcuts the quantize-append kernel takes (no GPU needed).

The kernel takes the group scale byte from ``amax * fl32(1/6)`` (no division), and rounds each
element by handing the quotient ``x / s`` to the hardware E2M1 conversion (nearest, ties to even,
saturating at 6). The quotient is ``q1 = fma(fma(-q0, s, x), r, q0)`` with ``q0 = x * r`` and
``r = fl32(1 / s)``, after a clamp of x to +-8s, with the sign of x. Both shortcuts are checked here
against exact references over every input they can see: every positive finite bf16 group maximum,
and every finite bf16 element against every E4M3 scale. The kernel's own output is checked
bit-exactly against the oracle codec in the GPU tests.
"""

from fractions import Fraction

import numpy as np

from oracle import nvfp4 as nv


def _all_finite_bf16():
    vals = nv.bf16_bits_to_float(np.arange(65536, dtype=np.uint32))
    return vals[np.isfinite(vals)]


def _e4m3_of_exact(q: Fraction) -> int:
    """Nearest E4M3 code of a positive rational, ties to even, saturating at 448 (exact)."""
    if q >= 448:
        return 0x7E
    if q < Fraction(1, 64):                          # subnormal grid, step 2^-9
        n = q * 512
        f = int(n)
        r = n - f
        return f + (1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1) else 0)
    e = 0
    while q >= 2 ** (e + 1):
        e += 1
    while q < Fraction(2) ** e:
        e -= 1
    m = (q / Fraction(2) ** e - 1) * 8
    f = int(m)
    r = m - f
    f += 1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1) else 0
    if f == 8:
        e, f = e + 1, 0
    return ((e + 7) << 3) | f


def test_scale_from_multiply_by_fp32_sixth_is_exact_for_every_bf16_amax():
    amax = np.unique(np.abs(_all_finite_bf16()))
    amax = amax[amax > 0]
    assert amax.size == 32639
    # the kernel's route: one fp32 multiply (round to nearest even), then E4M3 of that fp32 value
    prod = (amax.astype(np.float32) * np.float32(1.0 / 6.0)).astype(np.float64)
    ours = nv.e4m3_encode(prod)
    exact = np.array([_e4m3_of_exact(Fraction(float(a)) / 6) for a in amax], dtype=np.uint8)
    bad = np.nonzero(ours != exact)[0]
    assert bad.size == 0, f"amax {amax[bad[:4]]}: {ours[bad[:4]]} vs {exact[bad[:4]]}"


def _quotient_codes(x, s):
    """The kernel's quotient route in fp32, emulated exactly: the residual x - q0*s is exact in
    fp64 and rounded once (one fma); the correction e*r + q0 is formed in fp64 and rounded to fp32,
    which can differ from the fma by one ulp only next to an fp32 midpoint, never at a grid
    midpoint (there q1 is exact). Rounding to the grid: nearest, ties to even, saturating."""
    x32 = x.astype(np.float32)
    s32 = np.float32(s)
    r = np.float32(1.0) / s32 if s > 0 else np.float32(0.0)
    bound = np.float32(8.0) * max(s32, np.float32(2.0 ** -20))
    xc = np.clip(x32, -bound, bound)
    q0 = (xc * r).astype(np.float32)
    e = (xc.astype(np.float64) - q0.astype(np.float64) * np.float64(s32)).astype(np.float32)
    q1 = (e.astype(np.float64) * np.float64(r) + q0.astype(np.float64)).astype(np.float32)
    q1 = np.copysign(q1, xc)
    a = np.abs(q1.astype(np.float64))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(a[:, None] - grid[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    mag = np.where(cand[:, ::2].any(axis=1), 2 * np.argmax(cand[:, ::2], axis=1),
                   2 * np.argmax(cand[:, 1::2], axis=1) + 1)
    mag = np.where(a >= 6.0, 7, mag)
    return mag | (np.signbit(q1).astype(np.int64) << 3)


def test_quotient_route_matches_exact_codes_for_every_bf16_and_scale():
    x = _all_finite_bf16()
    a = np.abs(x)
    sign = np.signbit(x).astype(np.int64) << 3
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    scales = nv.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))      # zero and every positive
    for s in scales:
        got = _quotient_codes(x, s)
        if s == 0:
            want = sign                                                # magnitude 0, sign kept
        else:
            d = np.abs(a[:, None] - grid[None, :] * s)                 # exact in fp64
            cand = d == d.min(axis=1, keepdims=True)
            mag = np.where(cand[:, ::2].any(axis=1), 2 * np.argmax(cand[:, ::2], axis=1),
                           2 * np.argmax(cand[:, 1::2], axis=1) + 1)
            want = np.where(a >= 6 * s, 7, mag) | sign
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"scale {s}: x={x[bad[:4]]} got {got[bad[:4]]} want {want[bad[:4]]}"
    # the signed zeros keep their sign through the quotient
    assert _quotient_codes(np.array([-0.0, 0.0]), 1.0).tolist() == [8, 0]
