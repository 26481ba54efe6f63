// Quantize-on-append and the row-dequantize test hook.
//
// Quantize-append (page "Prime Inference: Fast, Reliable Serving for Frontier Open Models",
// section "Making room for low-latency decode": the MLA latent is compressed to NVFP4 -- 4-bit
// values with one FP8 scale per 16 values -- and the 64-value rope part stays FP8) is a pure
// streaming pass: 1152 bytes of bf16 in, one 352-byte row out, so it is bound by HBM bandwidth.
// Each lane encodes one 16-value group and two rope values: the scale byte is the gfx950 E4M3
// conversion of amax * fl32(1/6), the sixteen 4-bit codes are the gfx950 E2M1 conversion of an
// fma-corrected quotient x / scale (exact on every E2M1 grid midpoint, so the conversion's ties
// to even give the format's rounding); a row leaves as two stores: 256 code bytes (8 per lane),
// then 8 scale dwords and 16 rope dwords gathered with lane shuffles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "codec_device.h"
#include "nvfp4_device.h"

namespace mla {

// Layout: lane l of a wavefront owns group g = l & 31 (16 latent values) of row 2i + (l >> 5),
// so the per-group work (amax, scale byte, grid midpoints) is done once per group and each half
// of the wave encodes one row. A wave takes PAIRS row pairs per iteration and issues all their
// loads (slots, latent, rope) before encoding the first, which keeps several rows in flight
// (PAIRS = 2 for large appends; small appends take one pair per wave, for the shortest latency).
// The encode is shared with the fused append + decode kernel (nvfp4_encode_lane), so both write
// the same bytes.
constexpr int64_t kAppendLargeRows = 65536;   // from here on two row pairs per wave

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int PAIRS>
__global__ __launch_bounds__(256) void quantize_append_kernel(
    const uint16_t* __restrict__ latent, int64_t latent_stride,
    const uint16_t* __restrict__ rope, int64_t rope_stride,
    const int64_t* __restrict__ slots, int64_t n_rows,
    uint8_t* __restrict__ cache, int64_t page_stride, int64_t cache_bytes) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, g = lane & 31;
  constexpr int kRowsPerIter = 2 * PAIRS;
  const int64_t n_iters = (n_rows + kRowsPerIter - 1) / kRowsPerIter;
  const int64_t wave_stride = (int64_t)gridDim.x * 4;
  // Workgroup b runs on XCD b % 8 (the grid is a multiple of 8). Consecutive rows are given to
  // workgroups of one XCD, so the rows of a page, whose 352-byte rows share 128-byte lines, are
  // written through one L2.
  const int64_t wg = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  for (int64_t it = wg * 4 + (threadIdx.x >> 6); it < n_iters; it += wave_stride) {
    const int64_t row0 = it * kRowsPerIter;
    // Branch-free loads: rows past the end re-read the last row and are not written.
    const int64_t slot_l = slots[min(row0 + min(lane, kRowsPerIter - 1), n_rows - 1)];
    uint4v xa[PAIRS], xb[PAIRS];
    uint32_t ra[PAIRS], rb[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      const int64_t row = min(row0 + 2 * p + half, n_rows - 1);
      const uint16_t* lrow = latent + row * latent_stride + 16 * g;
      xa[p] = *(const uint4v*)lrow;
      xb[p] = *(const uint4v*)(lrow + 8);
      ra[p] = rope[row * rope_stride + g];               // rope element g
      rb[p] = rope[row * rope_stride + 32 + g];          // rope element 32 + g
    }
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      const int64_t row = row0 + 2 * p + half;
      const int64_t slot = half ? readlane64(slot_l, 2 * p + 1) : readlane64(slot_l, 2 * p);
      const int64_t off = (slot / kPageRows) * page_stride + (slot % kPageRows) * kRowBytes;
      // rows past the end, slots of -1 and slots outside the cache are not written
      const bool write = row < n_rows && slot >= 0 && off >= 0 && off + kRowBytes <= cache_bytes;

      const Nvfp4LaneOut e = nvfp4_encode_lane(xa[p], xb[p], ra[p], rb[p]);
      if (write) {
        uint8_t* dst = cache + off;
        *(uint2v*)(dst + 8 * g) = uint2v{e.c0, e.c1};              // bytes 0..255: codes
        if (g < 24) ((uint32_t*)(dst + kScaleOff))[g] = e.tail;     // bytes 256..351
      }
    }
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
  const bool large = n_rows >= kAppendLargeRows;
  const int64_t rows_per_wave = large ? 4 : 2;
  const int64_t waves = (n_rows + rows_per_wave - 1) / rows_per_wave;
  int64_t blocks = (waves + 3) / 4;
  const int64_t max_blocks = 256 * 256;  // grid-stride beyond 256 blocks per compute unit
  if (blocks > max_blocks) blocks = max_blocks;
  blocks = (blocks + 7) & ~(int64_t)7;   // a multiple of 8: the same count on every XCD
  if (large)
    hipLaunchKernelGGL(quantize_append_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t*)latent, latent_stride, (const uint16_t*)rope, rope_stride,
                       slots, n_rows, (uint8_t*)cache, page_stride, cache_bytes);
  else
    hipLaunchKernelGGL(quantize_append_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream,
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
