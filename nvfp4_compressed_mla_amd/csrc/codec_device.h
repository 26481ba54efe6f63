// Device-side NVFP4 / E4M3 encoders for gfx950 (CDNA4), used by the quantize-append and FP8
// kernels (formats and row layout as in nvfp4_device.h).
//
// Encoding is bit-exact with the format's round-to-nearest-even definition:
//   * E4M3: e4m3_encode rounds the fp32 mantissa to 3 bits with round-half-even on the raw bits
//     (integer arithmetic); e4m3_encode2_hw takes the gfx950 FP8 conversion after a clamp to
//     +-448, which gives the same bytes for every bf16 input;
//   * E2M1: the quotient x / s goes to the gfx950 FP4 conversion (nearest, ties to even,
//     saturating); the quotient is corrected with an exact fma residual so that it is exact
//     whenever x lies on a midpoint of the grid times the scale (see e2m1_encode8_hw).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"

namespace mla {

// ---- encode --------------------------------------------------------------------------------

// Nearest E4M3 byte of a finite fp32 value, ties to even, magnitudes >= 448 saturate to 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const float af = __uint_as_float(a);
  uint32_t code;
  if (af >= 448.0f) {
    code = 0x7Eu;
  } else if (af < 0.015625f) {            // below 2^-6: subnormal grid, step 2^-9
    code = (uint32_t)__builtin_rintf(af * 512.0f);   // exact scaling, round half even; 8 -> 2^-6
  } else {                                 // normal: keep 3 mantissa bits, round half even
    const uint32_t e = (a >> 23) - 120u;   // E4M3 biased exponent (fp32 bias 127, E4M3 bias 7)
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (keep & 1u));
    code = ((e << 3) | keep) + up;         // a carry out of the mantissa bumps the exponent
  }
  return code | sign;
}

// The same encoding by the gfx950 FP8 conversion, which rounds to nearest even (OCP E4M3);
// clamping to +-448 first makes every finite value saturate to 0x7E / 0xFE like e4m3_encode.
// Two values per call: x0 -> byte 0, x1 -> byte 1. Checked against the oracle codec on the GPU
// for every finite bf16 value and every group scale the encoder can produce.
__device__ __forceinline__ uint32_t e4m3_encode2_hw(float x0, float x1) {
  const float c0 = __builtin_amdgcn_fmed3f(x0, -448.0f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(x1, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
}

// Value of E4M3 byte 0 of w by the gfx950 conversion (exact).
__device__ __forceinline__ float e4m3_to_float_hw(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
}

// Value of an E4M3 byte (finite codes).
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = (e == 0u) ? (float)m * (1.0f / 512.0f)
                              : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// Eight E2M1 codes (element order, low nibble first) of x[0..7] against a decoded group scale s
// via the gfx950 FP4 conversion, which rounds to nearest even and saturates at 6 (checked
// against the E2M1 definition, signed zeros included). Its input is the quotient x / s, made exact
// wherever the rounding decision needs it:
//   q0 = x * r with r = fl(1/s); e = fma(-q0, s, x) is the exact residual (s has 4 significant
//   bits); q1 = fma(e, r, q0) is x / s to within a tiny fraction of an ulp.
// When x lies exactly on a midpoint t*s of the grid (t = .25 .75 1.25 1.75 2.5 3.5 5), q1 == t
// exactly and the conversion's ties-to-even gives the even code; any other bf16 x is at least
// 2^-10 away from every midpoint in units of s, far beyond the error of q1. x is first clamped to
// +-8s (anything past 6s encodes to 6 anyway) so that the products stay finite. A zero scale
// (s = 0, r = 0) gives signed zeros, i.e. magnitude 0 with the element's sign; the quotient
// takes the sign of x explicitly (for x = -0 the residual is +0 and the last fma returns +0).
__device__ __forceinline__ uint32_t e2m1_encode8_hw(const float* x, float s, float r, float bound) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xc = __builtin_amdgcn_fmed3f(x[i], -bound, bound);
    const float q0 = xc * r;
    const float e = __builtin_fmaf(-q0, s, xc);
    // the element's sign, also for x = -0, where the two fmas would return +0
    q[i] = __builtin_copysignf(__builtin_fmaf(e, r, q0), xc);
  }
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// One NVFP4 row per half wavefront: lanes 0-31 encode one row, lanes 32-63 another. Lane g of a
// half holds latent group g of its row (16 bf16 values as packed pairs: xa = values 0..7,
// xb = values 8..15) and rope elements g (ra) and 32 + g (rb) as bf16 bits. The result is the
// lane's 8 code bytes (row bytes 8g..8g+7) and, for g < 24, the row dword at byte 256 + 4g:
// scale bytes 4g..4g+3 (g < 8), rope bytes 4(g-8).. (g < 16), rope bytes 32 + 4(g-16).. (else).
// The scale byte is E4M3(amax * fl32(1/6)): for every finite bf16 amax this rounds to the same
// byte as the exact quotient amax / 6 (checked exhaustively on the host). Every lane of the wave
// must take part (the scale and rope bytes are gathered with lane shuffles).
struct Nvfp4LaneOut {
  uint32_t c0, c1, tail;
};

__device__ __forceinline__ Nvfp4LaneOut nvfp4_encode_lane(uint4v xa, uint4v xb, uint32_t ra, uint32_t rb) {
  const int lane = threadIdx.x & 63;
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_float(xa[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_float(xa[i] >> 16);
    v[8 + 2 * i] = bf16_bits_to_float(xb[i] & 0xFFFFu);
    v[8 + 2 * i + 1] = bf16_bits_to_float(xb[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  const uint32_t sbyte = e4m3_encode2_hw(amax * (1.0f / 6.0f), 0.0f) & 0xFFu;
  const float sc = e4m3_to_float_hw(sbyte);
  const float rinv = sc > 0.0f ? 1.0f / sc : 0.0f;          // IEEE division, once per group
  const float bound = 8.0f * fmaxf(sc, 0x1p-20f);
  Nvfp4LaneOut o;
  o.c0 = e2m1_encode8_hw(v, sc, rinv, bound);              // elements 0..7
  o.c1 = e2m1_encode8_hw(v + 8, sc, rinv, bound);          // elements 8..15
  const uint32_t rpair = e4m3_encode2_hw(bf16_bits_to_float(ra), bf16_bits_to_float(rb));
  const uint32_t rba = rpair & 0xFFu, rbb = rpair >> 8;
  // scale dword k (groups 4k..4k+3) is built on lane 4k of the half, rope dword k (elements
  // 4k..4k+3) on lane 4k (k < 8) or 4(k - 8) (k >= 8)
  const uint32_t sword = sbyte | (__shfl_down(sbyte, 1) << 8) | (__shfl_down(sbyte, 2) << 16) |
                         (__shfl_down(sbyte, 3) << 24);
  const uint32_t rwa = rba | (__shfl_down(rba, 1) << 8) | (__shfl_down(rba, 2) << 16) |
                       (__shfl_down(rba, 3) << 24);
  const uint32_t rwb = rbb | (__shfl_down(rbb, 1) << 8) | (__shfl_down(rbb, 2) << 16) |
                       (__shfl_down(rbb, 3) << 24);
  const int src = (lane & 32) | (4 * (lane & 7));
  const uint32_t w_s = __shfl(sword, src), w_a = __shfl(rwa, src), w_b = __shfl(rwb, src);
  const int g = lane & 31;
  o.tail = g < 8 ? w_s : (g < 16 ? w_a : w_b);
  return o;
}

}  // namespace mla
