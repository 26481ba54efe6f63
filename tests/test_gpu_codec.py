"""GPU quantize-append and on-chip decoder: bit-exact against the oracle codec."""

import os

import numpy as np
import pytest
import torch

from oracle import cache as oc
from oracle import nvfp4 as nv

pytestmark = pytest.mark.gpu

PAGE = 64 * 352


def _lib():
    import nvfp4_compressed_mla_amd as m
    return m


def _bf16_bits_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run_append(latent, rope, slots, page_stride, n_pages):
    m = _lib()
    cache = torch.full((n_pages * page_stride,), 0xAB, dtype=torch.uint8, device="cuda")
    m.mla_nvfp4_quantize_append(latent, rope, slots, cache, page_stride)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


def _expect(latent, rope, slots, page_stride, n_pages):
    cache = np.full(n_pages * page_stride, 0xAB, dtype=np.uint8)
    rows = nv.quantize_rows(_bf16_bits_to_f64(latent), _bf16_bits_to_f64(rope))
    oc.write_rows(cache, page_stride, slots.cpu().numpy(), rows)
    return cache


def _compare(got, want, what):
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[:6]}: got {got[bad[:6]]} want {want[bad[:6]]}"


def test_append_random_rows_bit_exact():
    print("case: random N(0,1) rows x 3 scales, padded page stride", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    n = 2000
    lat = (torch.randn(n, 512, generator=g, device="cuda") *
           torch.tensor([1.0, 1e-3, 300.0], device="cuda").repeat_interleave(n // 3 + 1)[:n, None]).bfloat16()
    rope = (torch.randn(n, 64, generator=g, device="cuda") * 50).bfloat16()
    stride = PAGE + 512
    n_pages = (n + 63) // 64 + 2
    slots = torch.randperm(n_pages * 64, generator=g, device="cuda")[:n].to(torch.int64)
    _compare(_run_append(lat, rope, slots, stride, n_pages), _expect(lat, rope, slots, stride, n_pages),
             "random rows")


def test_append_large_launch_bit_exact():
    """A launch past 65,536 rows (two row pairs per wavefront) with a ragged tail, random slots,
    a few -1 slots and magnitudes spread over the scale range."""
    print("case: 65,573-row append (large-launch path)", flush=True)
    g = torch.Generator(device="cuda").manual_seed(21)
    n = 65536 + 37
    mag = torch.exp2(torch.randint(-12, 10, (n, 1), generator=g, device="cuda").float())
    lat = (torch.randn(n, 512, generator=g, device="cuda") * mag).bfloat16()
    rope = (torch.randn(n, 64, generator=g, device="cuda") * mag).bfloat16()
    n_pages = (n + 63) // 64 + 3
    slots = torch.randperm(n_pages * 64, generator=g, device="cuda")[:n].to(torch.int64)
    slots[::997] = -1
    _compare(_run_append(lat, rope, slots, PAGE, n_pages), _expect(lat, rope, slots, PAGE, n_pages),
             "large launch")


def test_append_handworked_golden_row():
    print("case: hand-worked golden row", flush=True)
    from tests.test_oracle_codec import golden_row
    latent, rope, expect = golden_row()
    lat = torch.tensor(latent, dtype=torch.float64).to(torch.bfloat16)[None].cuda()
    rp = torch.tensor(rope, dtype=torch.float64).to(torch.bfloat16)[None].cuda()
    assert np.array_equal(_bf16_bits_to_f64(lat)[0], latent)     # values are bf16-exact
    assert torch.signbit(lat[0, 4]) and torch.signbit(rp[0, 7])
    got = _run_append(lat, rp, torch.tensor([3], dtype=torch.int64, device="cuda"), PAGE, 1)
    _compare(got[3 * 352:4 * 352], expect, "golden row")


def test_append_every_bf16_group_max():
    """Every positive finite bf16 value appears as a group maximum (scale route exhaustive),
    with ties, tiny groups, saturation and signed zeros in the other elements."""
    print("case: exhaustive bf16 group maxima", flush=True)
    bits = torch.arange(1, 0x7F80, dtype=torch.int32)                 # positive finite bf16
    amax = bits.to(torch.int16).view(torch.bfloat16).float()
    n_groups = amax.numel()
    n_rows = (n_groups + 31) // 32
    g = torch.Generator().manual_seed(9)
    frac = torch.rand(n_rows * 32, 16, generator=g) * 2 - 1
    pad = torch.zeros(n_rows * 32 - n_groups)
    m = torch.cat([amax, pad + 1.0])
    vals = (frac * m[:, None])
    vals[:, 0] = m                                                     # the maximum itself
    vals[:, 1] = -m * 0.5
    vals[:, 2] = -0.0
    # exact tie points against the scale that amax implies are produced naturally across values
    lat = vals.reshape(n_rows, 512).bfloat16().cuda()
    rope = (torch.randn(n_rows, 64, generator=g) * 10).bfloat16().cuda()
    slots = torch.arange(n_rows, dtype=torch.int64, device="cuda")
    n_pages = (n_rows + 63) // 64
    _compare(_run_append(lat, rope, slots, PAGE, n_pages), _expect(lat, rope, slots, PAGE, n_pages),
             "exhaustive group maxima")


def test_append_every_finite_bf16_rope_value():
    """Every finite bf16 value (both signs, zeros, subnormals, values past the E4M3 range) as a
    rope element: the rope route of the encoder is checked exhaustively."""
    print("case: exhaustive bf16 rope values", flush=True)
    bits = torch.arange(0, 65536, dtype=torch.int32)
    vals = bits.to(torch.int16).view(torch.bfloat16).float()
    vals = vals[torch.isfinite(vals)]
    n_rows = (vals.numel() + 63) // 64
    rope = torch.cat([vals, torch.zeros(n_rows * 64 - vals.numel())]).reshape(n_rows, 64)
    g = torch.Generator().manual_seed(13)
    lat = torch.randn(n_rows, 512, generator=g).bfloat16().cuda()
    rope = rope.bfloat16().cuda()
    slots = torch.arange(n_rows, dtype=torch.int64, device="cuda")
    n_pages = (n_rows + 63) // 64
    _compare(_run_append(lat, rope, slots, PAGE, n_pages), _expect(lat, rope, slots, PAGE, n_pages),
             "exhaustive rope values")


def test_append_ties_on_grid_midpoints():
    """Elements exactly on E2M1 midpoints for many scales, and rope on E4M3 midpoints."""
    print("case: midpoint ties", flush=True)
    scales = nv.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for s in scales:
        grp = np.concatenate([[6.0 * s], mids * s, -mids * s, [0.0]])
        rows.append(grp)
    groups = np.array(rows)                       # [126, 16]
    bf = torch.tensor(groups).to(torch.bfloat16).double().numpy()
    keep = np.all(bf == groups, axis=1)           # only groups exactly representable in bf16
    groups = groups[keep]
    n_rows = (len(groups) + 31) // 32
    full = np.zeros((n_rows * 32, 16))
    full[:len(groups)] = groups
    lat = torch.tensor(full.reshape(n_rows, 512)).to(torch.bfloat16).cuda()
    e4 = nv.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    rope_mid = ((e4[:-1] + e4[1:]) / 2)
    rope_vals = np.resize(rope_mid, n_rows * 64).reshape(n_rows, 64)
    rope = torch.tensor(rope_vals).to(torch.bfloat16).cuda()
    slots = torch.arange(n_rows, dtype=torch.int64, device="cuda")
    n_pages = (n_rows + 63) // 64
    _compare(_run_append(lat, rope, slots, PAGE, n_pages), _expect(lat, rope, slots, PAGE, n_pages),
             "midpoint ties")


def test_append_skips_minus_one_and_out_of_range_slots():
    print("case: slot -1 and out-of-range slots", flush=True)
    n = 130
    g = torch.Generator(device="cuda").manual_seed(2)
    lat = torch.randn(n, 512, generator=g, device="cuda").bfloat16()
    rope = torch.randn(n, 64, generator=g, device="cuda").bfloat16()
    n_pages = 3
    slots = torch.arange(n, dtype=torch.int64, device="cuda")
    slots[5] = -1
    slots[7] = n_pages * 64 + 10          # beyond the cache
    slots[9] = -123456789
    got = _run_append(lat, rope, slots, PAGE, n_pages)
    s_host = slots.cpu().numpy().copy()
    s_host[s_host >= n_pages * 64] = -1
    s_host[s_host < 0] = -1
    want = _expect(lat, rope, torch.tensor(s_host), PAGE, n_pages)
    _compare(got, want, "skip slots")


def test_append_block_major_stride():
    """A page stride covering several layers (block-major layout): rows land at the right bytes
    and the other layers' bytes are untouched."""
    print("case: block-major page stride", flush=True)
    layers = 3
    stride = layers * PAGE
    n = 200
    g = torch.Generator(device="cuda").manual_seed(4)
    lat = torch.randn(n, 512, generator=g, device="cuda").bfloat16()
    rope = torch.randn(n, 64, generator=g, device="cuda").bfloat16()
    n_pages = 5
    slots = torch.randperm(n_pages * 64, generator=g, device="cuda")[:n].to(torch.int64)
    _compare(_run_append(lat, rope, slots, stride, n_pages), _expect(lat, rope, slots, stride, n_pages),
             "block-major stride")


def test_dequantize_hook_matches_oracle_decode():
    print("case: on-chip decoder vs oracle dequantize", flush=True)
    m = _lib()
    g = np.random.default_rng(12)
    n = 1500
    codes = g.integers(0, 256, size=(n, 256), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(n, 32), dtype=np.uint8) | (g.integers(0, 2, size=(n, 32)) << 7).astype(np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x38
    rope = g.integers(0, 256, size=(n, 64), dtype=np.uint8)
    rope[(rope & 0x7F) == 0x7F] = 0x00
    rows = np.concatenate([codes, scales, rope], axis=1)
    n_pages = (n + 63) // 64
    cache = np.zeros(n_pages * PAGE, dtype=np.uint8)
    slots = g.permutation(n_pages * 64)[:n]
    oc.write_rows(cache, PAGE, slots, rows)
    dev = torch.from_numpy(cache).cuda()
    s = torch.from_numpy(np.concatenate([slots, [-1, n_pages * 64 + 3]])).to(torch.int64).cuda()
    out = m.mla_nvfp4_dequantize_rows(dev, PAGE, s).cpu().numpy().astype(np.float64)
    lat, rp = nv.dequantize_rows(rows)
    want = np.concatenate([lat, rp], axis=1)
    assert np.array_equal(out[:n], want), f"decoder mismatch at rows {np.nonzero(np.any(out[:n] != want, axis=1))[0][:5]}"
    assert np.array_equal(np.signbit(out[:n]), np.signbit(want))
    assert np.all(out[n:] == 0)
