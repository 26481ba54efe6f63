// FP8 baseline rows and the staged NVFP4 -> FP8 conversion.
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models": before the NVFP4
// change (section "Making room for low-latency decode") a cache row held the 512 latent and the
// 64 rope values as FP8, 576 bytes. Section "Native NVFP4 sparse MLA decode kernel" measures the
// fused NVFP4 kernel against the FP8 attention kernel on such rows, and against a staged path
// that first unpacks the selected NVFP4 rows into a temporary FP8 buffer and then runs the FP8
// kernel. This file holds the append of FP8 rows and that staging pass; the FP8 attention is the
// fused decode kernel instantiated for 576-byte rows.
//
// Both passes are streaming (HBM-bound) and bit-exact by construction:
//  * append: every bf16 value -> nearest E4M3, ties to even, saturating at 448 (the gfx950 FP8
//    conversion after a clamp to +-448, bit-exact with the integer rounding of the fp32 bits for
//    every bf16 input);
//  * staging: an NVFP4 value is an E2M1 magnitude (8 choices) times its group's E4M3 scale, so
//    its E4M3 rounding depends only on (scale byte, magnitude). Each workgroup first tabulates
//    those 128 x 8 bytes in LDS (the products are exact in fp32), after which a row costs one
//    table read per group and a byte permute per 4 values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "codec_device.h"
#include "nvfp4_device.h"

namespace mla {

__global__ __launch_bounds__(256) void fp8_append_kernel(
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
    const int64_t off = (slot / kPageRows) * page_stride + (slot % kPageRows) * kFp8RowBytes;
    if (off < 0 || off + kFp8RowBytes > cache_bytes) continue;

    // lane l: latent elements 8l..8l+7 -> bytes 8l..8l+7; rope element l -> byte 512+l
    const uint4v x8 = *(const uint4v*)(latent + row * latent_stride + lane * 8);
    const uint32_t rbits = rope[row * rope_stride + lane];
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i >> 1] |= e4m3_encode2_hw(__uint_as_float(x8[i] << 16), __uint_as_float(x8[i] & 0xFFFF0000u))
                   << (16 * (i & 1));
    const uint32_t rbyte = e4m3_encode2_hw(__uint_as_float(rbits << 16), 0.0f) & 0xFFu;
    const uint32_t r1 = __shfl_down(rbyte, 1), r2 = __shfl_down(rbyte, 2), r3 = __shfl_down(rbyte, 3);

    uint8_t* dst = cache + off;
    *(uint2v*)(dst + 8 * lane) = uint2v{w[0], w[1]};
    if ((lane & 3) == 0)
      *(uint32_t*)(dst + kLatent + lane) = rbyte | (r1 << 8) | (r2 << 16) | (r3 << 24);
  }
}

// Four E2M1 codes (the low 16 bits of h, element order) -> four E4M3 bytes through the table of
// one scale (bytes of t: magnitude index 0..7); `flip` holds the scale's sign in every byte.
__device__ __forceinline__ uint32_t nib4_to_fp8(uint32_t h, uint2v t, uint32_t flip) {
  uint32_t x = (h | (h << 8)) & 0x00FF00FFu;                // nibbles 0,1 | 2,3 -> bytes 0 | 2
  x = (x | (x << 4)) & 0x0F0F0F0Fu;                         // one nibble per byte
  const uint32_t mag = x & 0x07070707u;
  const uint32_t sgn = ((x & 0x08080808u) << 4) ^ flip;
  return __builtin_amdgcn_perm(t[1], t[0], mag) | sgn;      // byte k = table[mag_k]
}

__device__ __forceinline__ uint4v group_to_fp8(uint2v codes, uint2v t, uint32_t flip) {
  return uint4v{nib4_to_fp8(codes[0] & 0xFFFFu, t, flip), nib4_to_fp8(codes[0] >> 16, t, flip),
                nib4_to_fp8(codes[1] & 0xFFFFu, t, flip), nib4_to_fp8(codes[1] >> 16, t, flip)};
}

// Staging: list entry e of query token tok (row r = tok*topk + e) is resolved like the decode
// kernel does (-1, out-of-table positions, negative pages and rows outside the cache are empty);
// a non-empty entry's row is written as a 576-byte FP8 row at staged slot tok*topk_pad + e, and
// the staged index list gets e (or -1). staged_bt maps page p of "request" tok to page
// tok*(topk_pad/64) + p, so the FP8 kernel reads the staged rows through ordinary paging.
// 16 lanes per row: lane i converts latent groups i and i+16 and copies 4 rope bytes.
// kStageRows: list entries in flight per 16-lane group (more for large launches, where the
// workgroups outnumber what the chip holds at once; one for small ones, to spread the latency
// chains over more workgroups)
template <int kStageRows>
__global__ __launch_bounds__(256) void stage_fp8_kernel(
    const uint8_t* __restrict__ cache, int64_t page_stride, int64_t cache_bytes,
    const int32_t* __restrict__ block_table, int32_t max_pages,
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t q_len, int32_t topk_pad,
    int64_t total_rows, uint8_t* __restrict__ staged, int32_t* __restrict__ staged_idx,
    int32_t* __restrict__ staged_bt) {
  __shared__ uint2v tab[128];
  const int li = threadIdx.x & 15;
  const int pages2 = topk_pad >> 6;
  const int64_t r_step = (int64_t)gridDim.x * 16;
  const int group = threadIdx.x >> 4;
  // the trip count depends on the workgroup only (every thread reaches the barrier below)
  for (int64_t base = (int64_t)blockIdx.x * 16; base < total_rows; base += r_step * kStageRows) {
    const int64_t rb = base + group;
    // kStageRows entries rb, rb + r_step, ...: all index loads, then all block-table loads,
    // then all row loads, so their latencies overlap
    int j[kStageRows], pg[kStageRows];
    int64_t off[kStageRows];
#pragma unroll
    for (int k = 0; k < kStageRows; ++k) {
      const int64_t r = rb + k * r_step;
      j[k] = r < total_rows ? topk_idx[r] : -1;
    }
#pragma unroll
    for (int k = 0; k < kStageRows; ++k) {
      const int64_t r = rb + k * r_step;
      const bool in = j[k] >= 0 && (int64_t)j[k] < (int64_t)max_pages * kPageRows;
      const int b = (int)((in ? r : 0) / topk / q_len);
      pg[k] = in ? block_table[(int64_t)b * max_pages + (j[k] >> 6)] : -1;
    }
#pragma unroll
    for (int k = 0; k < kStageRows; ++k) {
      const int64_t o = (int64_t)pg[k] * page_stride + (int64_t)(j[k] & 63) * kRowBytes;
      off[k] = (pg[k] >= 0 && o + kRowBytes <= cache_bytes) ? o : -1;
    }
    uint2v c0[kStageRows], c1[kStageRows];
    uint32_t s0[kStageRows], s1[kStageRows], rp[kStageRows];
#pragma unroll
    for (int k = 0; k < kStageRows; ++k) {
      if (off[k] >= 0) {
        const uint8_t* src = cache + off[k];
        c0[k] = *(const uint2v*)(src + 8 * li);
        c1[k] = *(const uint2v*)(src + 128 + 8 * li);
        s0[k] = src[kScaleOff + li];
        s1[k] = src[kScaleOff + 16 + li];
        rp[k] = *(const uint32_t*)(src + kRopeOff + 4 * li);
      }
    }
    if (base == (int64_t)blockIdx.x * 16) {
      // tab[s] byte m = E4M3(E2M1 magnitude m * value of scale byte s), s = 0..127; built once,
      // while the first entries' loads are in flight
      const int s = threadIdx.x >> 1, part = threadIdx.x & 1;
      const float sv = e4m3_to_float((uint32_t)s);
      const float mags[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) word |= e4m3_encode(mags[4 * part + k] * sv) << (8 * k);
      ((uint32_t*)tab)[2 * s + part] = word;
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kStageRows; ++k) {
      const int64_t r = rb + k * r_step;
      if (r >= total_rows) break;
      const int64_t tok = r / topk;
      const int e = (int)(r - tok * topk);
      if (li == 0) {
        staged_idx[r] = off[k] >= 0 ? e : -1;
        if ((e & 63) == 0) staged_bt[tok * pages2 + (e >> 6)] = (int32_t)(tok * pages2 + (e >> 6));
      }
      if (off[k] >= 0) {
        const uint32_t f0 = (s0[k] & 0x80u) ? 0x80808080u : 0u, f1 = (s1[k] & 0x80u) ? 0x80808080u : 0u;
        uint8_t* dst = staged + (tok * topk_pad + e) * kFp8RowBytes;
        *(uint4v*)(dst + 16 * li) = group_to_fp8(c0[k], tab[s0[k] & 127u], f0);
        *(uint4v*)(dst + 256 + 16 * li) = group_to_fp8(c1[k], tab[s1[k] & 127u], f1);
        *(uint32_t*)(dst + kLatent + 4 * li) = rp[k];
      }
    }
  }
}

hipError_t launch_fp8_append(const void* latent, int64_t latent_stride, const void* rope,
                             int64_t rope_stride, const int64_t* slots, int64_t n_rows, void* cache,
                             int64_t page_stride, int64_t cache_bytes, hipStream_t stream) {
  int64_t blocks = (n_rows + 3) / 4;
  const int64_t max_blocks = 256 * 32;
  if (blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL(fp8_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)latent, latent_stride, (const uint16_t*)rope, rope_stride,
                     slots, n_rows, (uint8_t*)cache, page_stride, cache_bytes);
  return hipGetLastError();
}

hipError_t launch_stage_fp8(const void* cache, int64_t page_stride, int64_t cache_bytes,
                            const int32_t* block_table, int32_t max_pages, const int32_t* topk_idx,
                            int32_t topk, int32_t T, int32_t q_len, void* staged,
                            int32_t* staged_idx, int32_t* staged_bt, hipStream_t stream) {
  const int32_t topk_pad = (topk + 63) & ~63;
  const int64_t total = (int64_t)T * topk;
  const bool big = total >= 65536;
  const int rows = big ? 4 : 1;
  int64_t blocks = (total + 16 * rows - 1) / (16 * rows);
  const int64_t max_blocks = 256 * 8;
  if (blocks > max_blocks) blocks = max_blocks;
  if (big)
    hipLaunchKernelGGL(stage_fp8_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)cache, page_stride, cache_bytes, block_table, max_pages,
                       topk_idx, topk, q_len, topk_pad, total, (uint8_t*)staged, staged_idx,
                       staged_bt);
  else
    hipLaunchKernelGGL(stage_fp8_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t*)cache, page_stride, cache_bytes, block_table, max_pages,
                       topk_idx, topk, q_len, topk_pad, total, (uint8_t*)staged, staged_idx,
                       staged_bt);
  return hipGetLastError();
}

}  // namespace mla
