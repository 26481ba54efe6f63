// Device-side NVFP4 / E4M3 codec pieces for gfx950 (CDNA4).
//
// Formats: OCP OFP8 E4M3 (bias 7, max 448, no infinities) for the group scales and the rope
// part; OCP MX FP4 E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6) for the latent elements. Row format
// from "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Making room
// for low-latency decode": 4-bit latent values with one FP8 scale per 16 values plus a 64-value
// FP8 rope part, 352 bytes per row.
//
// Encoding is bit-exact with the format's round-to-nearest-even definition:
//   * E4M3: e4m3_encode rounds the fp32 mantissa to 3 bits with round-half-even on the raw bits
//     (integer arithmetic); e4m3_encode2_hw takes the gfx950 FP8 conversion after a clamp to
//     +-448, which gives the same bytes for every bf16 input;
//   * E2M1: the quotient x / s goes to the gfx950 FP4 conversion (nearest, ties to even,
//     saturating); the quotient is corrected with an exact fma residual so that it is exact
//     whenever x lies on a midpoint of the grid times the scale (see e2m1_encode8_hw).
// Decoding to FP16 MFMA operands uses the gfx950 packed conversions with unit scale, then one
// packed FP16 multiply by the group scale; every product e2m1 * e4m3 is exact in FP16
// (at most 6 significant bits, magnitudes in [2^-10, 2688]).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kQkDim = 576;
constexpr int kRowBytes = 352;
constexpr int kCodeBytes = 256;   // 512 4-bit codes
constexpr int kScaleOff = 256;    // 32 E4M3 group scales
constexpr int kRopeOff = 288;     // 64 E4M3 rope values
constexpr int kPageRows = 64;
// FP8 baseline row (576 bytes): latent element i at byte i, rope element j at byte 512 + j, both
// E4M3 with unit scale.
constexpr int kFp8RowBytes = 576;

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
__device__ __forceinline__ uint32_t e2m1_encode8_hw(const float (&x)[8], float s, float r, float bound) {
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

// ---- decode to FP16 operands ------------------------------------------------------------------

// Two E2M1 codes in byte `sel` of w -> FP16 pair (low nibble first), unit scale.
template <int SEL>
__device__ __forceinline__ half2v fp4x2_to_half2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two E4M3 bytes in 16-bit word `HI` of w -> FP16 pair (low byte first), unit scale.
template <bool HI>
__device__ __forceinline__ half2v fp8x2_to_half2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight E2M1 codes of one dword (8 consecutive elements of one group) times an FP16 scale pair
// -> eight FP16 values in element order.
__device__ __forceinline__ half8v decode_fp4x8(uint32_t w, half2v s2) {
  const half2v p0 = fp4x2_to_half2<0>(w) * s2;
  const half2v p1 = fp4x2_to_half2<1>(w) * s2;
  const half2v p2 = fp4x2_to_half2<2>(w) * s2;
  const half2v p3 = fp4x2_to_half2<3>(w) * s2;
  return half8v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight E4M3 bytes (two dwords) -> eight FP16 values in byte order.
__device__ __forceinline__ half8v decode_fp8x8(uint32_t lo, uint32_t hi) {
  const half2v p0 = fp8x2_to_half2<false>(lo);
  const half2v p1 = fp8x2_to_half2<true>(lo);
  const half2v p2 = fp8x2_to_half2<false>(hi);
  const half2v p3 = fp8x2_to_half2<true>(hi);
  return half8v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// E4M3 scale byte -> FP16 pair (s, s).
__device__ __forceinline__ half2v scale_pair(uint32_t b) {
  const half2v s = fp8x2_to_half2<false>(b & 0xFFu);
  return half2v{s[0], s[0]};
}

}  // namespace mla
