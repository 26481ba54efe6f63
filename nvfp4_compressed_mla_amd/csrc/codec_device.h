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

}  // namespace mla
