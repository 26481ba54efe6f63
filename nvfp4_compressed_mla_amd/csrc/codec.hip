// Quantize-on-append and the row-dequantize test hook.
//
// Quantize-append (page "Prime Inference: Fast, Reliable Serving for Frontier Open Models",
// section "Making room for low-latency decode": the MLA latent is compressed to NVFP4 -- 4-bit
// values with one FP8 scale per 16 values -- and the 64-value rope part stays FP8) is a pure
// streaming pass: 1152 bytes of bf16 in, one 352-byte row out, so it is bound by HBM bandwidth.
// One wavefront owns one row: lane l reads latent elements 8l..8l+7 with one 16-byte load (its
// group of 16 is shared with lane l^1), and rope element l. Group maxima are combined across the
// lane pair, the scale byte and the eight 4-bit codes are computed with exact integer/compare
// arithmetic, and the row leaves as dword stores: 64 code dwords, 8 scale dwords (gathered with
// lane shuffles) and 16 rope dwords.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "nvfp4_device.h"

namespace mla {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

__global__ __launch_bounds__(256) void quantize_append_kernel(
    const uint16_t* __restrict__ latent, int64_t latent_stride,
    const uint16_t* __restrict__ rope, int64_t rope_stride,
    const int64_t* __restrict__ slots, int64_t n_rows,
    uint8_t* __restrict__ cache, int64_t page_stride, int64_t cache_bytes) {
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t wave_stride = (int64_t)gridDim.x * 4;
  for (int64_t row = wave0; row < n_rows; row += wave_stride) {
    const int64_t slot = slots[row];
    if (slot < 0) continue;                                   // wave-uniform
    const int64_t off = (slot / kPageRows) * page_stride + (slot % kPageRows) * kRowBytes;
    if (off < 0 || off + kRowBytes > cache_bytes) continue;   // outside the cache: not written

    const uint4v x8 = *(const uint4v*)(latent + row * latent_stride + lane * 8);
    const uint32_t rbits = rope[row * rope_stride + lane];

    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_float(x8[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_float(x8[i] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));                  // the other half of the group

    const uint32_t sbyte = e4m3_encode(amax / 6.0f);          // IEEE division, then RNE to E4M3
    const float s = e4m3_to_float(sbyte);
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) codes |= e2m1_encode(v[i], s) << (4 * i);

    const uint32_t rbyte = e4m3_encode(bf16_bits_to_float(rbits));

    // Gather 4 scale bytes (lanes 8m, 8m+2, 8m+4, 8m+6) and 4 rope bytes (lanes 4m..4m+3).
    const uint32_t s1 = __shfl_down(sbyte, 2), s2 = __shfl_down(sbyte, 4), s3 = __shfl_down(sbyte, 6);
    const uint32_t r1 = __shfl_down(rbyte, 1), r2 = __shfl_down(rbyte, 2), r3 = __shfl_down(rbyte, 3);

    uint8_t* dst = cache + off;
    ((uint32_t*)dst)[lane] = codes;
    if ((lane & 7) == 0)
      ((uint32_t*)(dst + kScaleOff))[lane >> 3] = sbyte | (s1 << 8) | (s2 << 16) | (s3 << 24);
    if ((lane & 3) == 0)
      ((uint32_t*)(dst + kRopeOff))[lane >> 2] = rbyte | (r1 << 8) | (r2 << 16) | (r3 << 24);
  }
}

// One wavefront per requested row: lane l decodes latent elements 8l..8l+7 through the same FP16
// operand decoder the attention kernels use; lanes 0..7 decode the rope bytes 8l..8l+7.
__global__ __launch_bounds__(256) void dequantize_rows_kernel(
    const uint8_t* __restrict__ cache, int64_t page_stride, int64_t cache_bytes,
    const int64_t* __restrict__ slots, int64_t n, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int64_t slot = slots[row];
  const int64_t off = slot < 0 ? -1 : (slot / kPageRows) * page_stride + (slot % kPageRows) * kRowBytes;
  float* o = out + row * kQkDim;
  if (off < 0 || off + kRowBytes > cache_bytes) {
#pragma unroll
    for (int i = 0; i < 9; ++i) o[lane * 9 + i] = 0.0f;
    return;
  }
  const uint8_t* r = cache + off;
  const uint32_t w = ((const uint32_t*)r)[lane];
  const uint32_t sb = r[kScaleOff + (lane >> 1)];
  const half8v h = decode_fp4x8(w, scale_pair(sb));
#pragma unroll
  for (int i = 0; i < 8; ++i) o[lane * 8 + i] = (float)h[i];
  if (lane < 8) {
    const uint2v rb = *(const uint2v*)(r + kRopeOff + lane * 8);
    const half8v hr = decode_fp8x8(rb[0], rb[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[kLatent + lane * 8 + i] = (float)hr[i];
  }
}

hipError_t launch_quantize_append(const void* latent, int64_t latent_stride, const void* rope,
                                  int64_t rope_stride, const int64_t* slots, int64_t n_rows,
                                  void* cache, int64_t page_stride, int64_t cache_bytes,
                                  hipStream_t stream) {
  const int64_t waves = n_rows;
  int64_t blocks = (waves + 3) / 4;
  const int64_t max_blocks = 256 * 32;   // grid-stride beyond 32 blocks per compute unit
  if (blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL(quantize_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)latent, latent_stride, (const uint16_t*)rope, rope_stride,
                     slots, n_rows, (uint8_t*)cache, page_stride, cache_bytes);
  return hipGetLastError();
}

hipError_t launch_dequantize_rows(const void* cache, int64_t page_stride, int64_t cache_bytes,
                                  const int64_t* slots, int64_t n, float* out, hipStream_t stream) {
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(dequantize_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint8_t*)cache, page_stride, cache_bytes, slots, n, out);
  return hipGetLastError();
}

}  // namespace mla
