"""Host checks of the arithmetic shortcuts the quantize-append kernel takes (no GPU needed).

The kernel does not divide: it takes the group scale byte from ``amax * fl32(1/6)`` and finds each
element's 3-bit E2M1 magnitude with three comparisons against the grid midpoints times the scale.
Both are checked here against exact references over every input they can see: every positive
finite bf16 group maximum, and every finite bf16 element against every positive E4M3 scale.
The kernel's own output is checked bit-exactly against the oracle codec in the GPU tests.
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


def _search_magnitude(a, s):
    """The kernel's three-comparison search, restated with NumPy selects (fp32 products)."""
    s = np.float32(s)
    mids = [np.float32(k) * s if s > 0 else np.float32(65536.0)
            for k in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)]
    a = a.astype(np.float32)
    hi = a >= mids[3]
    u0 = np.where(hi, mids[4], mids[0])
    u1 = np.where(hi, mids[5], mids[1])
    u2 = np.where(hi, mids[6], mids[2])
    mid = a >= u1
    odd = np.where(mid, a > u2, a > u0)
    return hi.astype(np.int64) * 4 + mid.astype(np.int64) * 2 + odd.astype(np.int64)


def test_three_comparison_search_equals_nearest_grid_value_for_every_bf16_and_scale():
    a = np.abs(_all_finite_bf16())
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    scales = nv.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))      # zero and every positive
    for s in scales:
        got = _search_magnitude(a, s)
        if s == 0:
            assert np.all(got[a < 6 * 2.0 ** -10] == 0)                # the groups that get s = 0
            continue
        # nearest grid value of a / s by brute force over the 8 values, ties to the even code
        # (an exact comparison: every |a - g s| is exact in fp64)
        d = np.abs(a[:, None] - grid[None, :] * s)
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        even_pick = np.where(cand[:, ::2].any(axis=1),
                             2 * np.argmax(cand[:, ::2], axis=1),
                             2 * np.argmax(cand[:, 1::2], axis=1) + 1)
        want = np.where(a >= 6 * s, 7, even_pick)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"scale {s}: a={a[bad[:4]]} got {got[bad[:4]]} want {want[bad[:4]]}"
