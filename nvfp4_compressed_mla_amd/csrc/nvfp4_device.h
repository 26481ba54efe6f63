// Device-side NVFP4 / E4M3 pieces shared by the kernels for gfx950 (CDNA4): element types, the
// row format, and the decoder to FP16 MFMA operands. The encoders live in codec_device.h.
//
// Formats: OCP OFP8 E4M3 (bias 7, max 448, no infinities) for the group scales and the rope
// part; OCP MX FP4 E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6) for the latent elements. Row format
// from "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Making room
// for low-latency decode": 4-bit latent values with one FP8 scale per 16 values plus a 64-value
// FP8 rope part, 352 bytes per row.
//
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
