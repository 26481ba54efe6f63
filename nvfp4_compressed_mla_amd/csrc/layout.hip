// Block transfer between multi-layer KV page pools.
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Changing the
// layout to reduce fragmentation": in the layer-major layout (LBHNC) the cache of each layer is
// stored on its own, so one logical 64-token block is spread over one region per layer; in the
// block-major layout (BLHNC) the pages of all layers of a block sit side by side, and a block
// moves as one contiguous region. A pool holds pool_blocks blocks x n_layers pages of page_bytes:
//   block-major: page (b, l) at (b * n_layers + l) * page_bytes
//   layer-major: page (b, l) at (l * pool_blocks + b) * page_bytes
// Layer l of a block-major pool is an ordinary paged cache at base l * page_bytes with page stride
// n_layers * page_bytes, which is what the decode kernels take.
//
// The copy is one launch for any number of blocks and either layout (each workgroup moves whole
// pages with 16-byte loads and stores, four in flight per lane), so the per-descriptor cost that
// fragmentation adds to a transfer engine does not arise on the device; what the layout still
// decides is the number of contiguous regions another engine would have to move.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "nvfp4_device.h"

namespace mla {

__device__ __forceinline__ int64_t pool_page(int32_t layout, int64_t block, int64_t layer,
                                             int64_t n_layers, int64_t pool_blocks) {
  return layout == 0 ? block * n_layers + layer : layer * pool_blocks + block;
}

__global__ __launch_bounds__(256) void copy_pages_kernel(
    const uint8_t* __restrict__ src, int64_t src_pool_blocks, uint8_t* __restrict__ dst,
    int64_t dst_pool_blocks, int32_t layout, int32_t n_layers, int64_t page_bytes,
    const int32_t* __restrict__ src_blocks, const int32_t* __restrict__ dst_blocks,
    int64_t n_pages) {
  const int64_t pieces = page_bytes / 16;
  for (int64_t pg = blockIdx.x; pg < n_pages; pg += gridDim.x) {      // workgroup-uniform
    const int64_t i = pg / n_layers;
    const int64_t l = pg - i * n_layers;
    const int64_t sb = src_blocks[i], db = dst_blocks[i];
    if (sb < 0 || sb >= src_pool_blocks || db < 0 || db >= dst_pool_blocks) continue;
    const uint4v* s4 = (const uint4v*)(src + pool_page(layout, sb, l, n_layers, src_pool_blocks) * page_bytes);
    uint4v* d4 = (uint4v*)(dst + pool_page(layout, db, l, n_layers, dst_pool_blocks) * page_bytes);
    int64_t k = threadIdx.x;
    for (; k + 3 * 256 < pieces; k += 4 * 256) {
      const uint4v a = s4[k], b = s4[k + 256], c = s4[k + 512], d = s4[k + 768];
      d4[k] = a;
      d4[k + 256] = b;
      d4[k + 512] = c;
      d4[k + 768] = d;
    }
    for (; k < pieces; k += 256) d4[k] = s4[k];
  }
}

hipError_t launch_copy_pages(const void* src, int64_t src_pool_blocks, void* dst,
                             int64_t dst_pool_blocks, int32_t layout, int32_t n_layers,
                             int64_t page_bytes, const int32_t* src_blocks,
                             const int32_t* dst_blocks, int32_t n_blocks, hipStream_t stream) {
  const int64_t n_pages = (int64_t)n_blocks * n_layers;
  int64_t grid = n_pages < 256 * 16 ? n_pages : 256 * 16;
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint8_t*)src, src_pool_blocks, (uint8_t*)dst, dst_pool_blocks, layout,
                     n_layers, page_bytes, src_blocks, dst_blocks, n_pages);
  return hipGetLastError();
}

}  // namespace mla
